// Host-only stand-ins for the kernel launchers, so that the C ABI's host
// code (argument validation, workspace layout, parameter packing) can be
// built with the address and undefined-behaviour sanitizers and run on a
// machine without a GPU.  Each stand-in counts its calls and enqueues nothing.
#include "dn_internal.h"

int g_launches = 0;

namespace dn {

size_t fwd_smem_bytes(int, int) { return 0; }
size_t fwd_ref_smem_bytes(int, int) { return 0; }
hipError_t launch_fwd(const FwdParams &, int, int, bool, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_c32(const FwdParams &, int, bool, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_ref(const FwdParams &, int, int, bool, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_step(const StepParams &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_longhorn(const LonghornParams &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prologue(const PrologueParams &, int, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_conv(const ConvParams &, int, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_chunk_table(const int32_t *, int, int32_t *, int32_t *, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdParams &, int, int, hipStream_t, hipEvent_t, hipEvent_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_scan(const BwdParams &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_bwd_chunk(const BwdParams &, int, hipStream_t) { ++g_launches; return hipSuccess; }

}  // namespace dn
