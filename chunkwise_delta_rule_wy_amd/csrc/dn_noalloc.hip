// dn_chunk_bwd_noalloc: the recomputing backward pass with its workspace in a
// static device buffer, for callers that cannot allocate device memory.
//
// `scratch` is a file-scope device array.  On the host its name stands for a
// host-side shadow, not a device address, so host code never passes it to a
// kernel or a copy: the device address of each GPU's copy is looked up once
// per device with hipGetSymbolAddress, on the first call on that device (with
// that device current), and kept in `g_scratch`.
#include <mutex>

#include "dn.h"
#include "dn_entry.h"
#include "dn_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[DN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::once_flag g_once[MAX_DEVICES];
hipError_t g_status[MAX_DEVICES];
void *g_scratch[MAX_DEVICES];

// Device address of the current device's scratch buffer.
dn_status scratch_address(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return DN_EHIP;
  std::call_once(g_once[dev], [dev] {
    void *p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = p;
  });
  if (g_status[dev] != hipSuccess || g_scratch[dev] == nullptr) return DN_EHIP;
  *ptr = g_scratch[dev];
  return DN_OK;
}

}  // namespace

extern "C" dn_status dn_chunk_bwd_noalloc(const dn_shape *s, const void *q, const void *k, const void *v,
                                          const float *beta, const float *g, const float *h0,
                                          const int32_t *cu_seqlens, const void *dO, const float *dhT, float *dq,
                                          float *dk, float *dv, float *dbeta, float *dg, float *dh0,
                                          hipStream_t stream) {
  // the arguments first, then the size, then the device: nothing is looked
  // up or enqueued for a call that fails
  dn_status st = dn::bwd_check(s, q, k, v, beta, g, cu_seqlens, dO, dq, dk, dv, dbeta, dg);
  if (st != DN_OK) return st;
  if (dn_chunk_bwd_workspace(s) > DN_NOALLOC_SCRATCH_BYTES) return DN_ESCRATCH;
  void *ws = nullptr;
  st = scratch_address(&ws);
  if (st != DN_OK) return st;
  return dn::bwd_recompute(s, q, k, v, beta, g, h0, cu_seqlens, dO, dhT, dq, dk, dv, dbeta, dg, dh0, ws,
                           DN_NOALLOC_SCRATCH_BYTES, stream);
}
