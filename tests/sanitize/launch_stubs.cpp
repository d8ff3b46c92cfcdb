// Host-only stand-ins for the kernel launchers, so that the C ABI's host
// code (argument validation, workspace layout, parameter packing) can be
// built with the address and undefined-behaviour sanitizers and run on a
// machine without a GPU.  Each stand-in counts its calls and enqueues nothing;
// while g_fail is set it reports a launch failure instead (the error path of
// the ABI, which must map it to DN_EHIP).
#include "dn_internal.h"

int g_launches = 0;
int g_fail = 0;

static hipError_t launched() {
  ++g_launches;
  return g_fail ? hipErrorLaunchFailure : hipSuccess;
}

namespace dn {

size_t fwd_smem_bytes(int, int) { return 0; }
size_t fwd_ref_smem_bytes(int, int) { return 0; }
hipError_t launch_fwd(const FwdParams &, int, int, bool, bool, hipStream_t) { return launched(); }
hipError_t launch_fwd_c32(const FwdParams &, int, bool, bool, hipStream_t) { return launched(); }
hipError_t launch_fwd_ref(const FwdParams &, int, int, bool, bool, hipStream_t) { return launched(); }
hipError_t launch_step(const StepParams &, int, int, hipStream_t) { return launched(); }
hipError_t launch_longhorn(const LonghornParams &, int, int, hipStream_t) { return launched(); }
hipError_t launch_prologue(const PrologueParams &, int, int, bool, hipStream_t) { return launched(); }
hipError_t launch_conv(const ConvParams &, int, bool, hipStream_t) { return launched(); }
hipError_t launch_chunk_table(const int32_t *, int, int32_t *, int32_t *, int, int, hipStream_t) {
  return launched();
}
hipError_t launch_seq_order(const int32_t *, int, int32_t *, hipStream_t) { return launched(); }
hipError_t launch_bwd(const BwdParams &, int, int, hipStream_t, hipEvent_t, hipEvent_t) { return launched(); }
hipError_t launch_bwd_scan(const BwdParams &, int, hipStream_t) { return launched(); }
hipError_t launch_bwd_chunk(const BwdParams &, int, hipStream_t) { return launched(); }

}  // namespace dn
