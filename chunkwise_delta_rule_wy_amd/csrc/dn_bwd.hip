// Backward pass kernels (placeholder until the reverse sweep lands).
#include "dn_internal.h"

namespace dn {

// Device-side chunk table for packed sequences: chunk_base[n] is the global
// index of sequence n's first 64-token chunk, chunk_seq[c] the sequence of
// global chunk c (-1 past the end).  One workgroup; no host copy of cu_seqlens.
__global__ void chunk_table_kernel(const int32_t *cu, int N, int32_t *chunk_base, int32_t *chunk_seq,
                                   int max_chunks) {
  __shared__ int32_t base[1025];
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int n = 0; n < N; ++n) {
      const int len = cu[n + 1] - cu[n];
      if (n < 1024) base[n] = acc;
      chunk_base[n] = acc;
      acc += (len + 63) / 64;
    }
    chunk_base[N] = acc;
    if (N < 1025) base[N] = acc;
  }
  __syncthreads();
  const int total = chunk_base[N];
  for (int c = threadIdx.x; c < max_chunks; c += blockDim.x) {
    int seq = -1;
    if (c < total) {
      int lo = 0, hi = N - 1;  // last n with chunk_base[n] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        const int bm = mid < 1025 ? base[mid] : chunk_base[mid];
        if (bm <= c) lo = mid; else hi = mid - 1;
      }
      seq = lo;
    }
    chunk_seq[c] = seq;
  }
}

hipError_t launch_chunk_table(const int32_t *cu, int N, int32_t *chunk_base, int32_t *chunk_seq,
                              int max_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, cu, N, chunk_base, chunk_seq,
                     max_chunks);
  return hipGetLastError();
}

size_t bwd_smem_bytes(int, int) { return 0; }

hipError_t launch_bwd(const BwdParams &, int, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace dn
