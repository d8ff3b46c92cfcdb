// Backward pass of the chunkwise (gated) delta rule for gfx950.
//
// The forward pass keeps chunk states on chip, so the backward pass first
// recomputes them (the forward kernel in its state-storing variant writes
// h_c, the state entering chunk c), following the recompute-in-the-backward
// design of "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length" (page 1, answer Q2).  Then:
//
// 1. scan_bf16_kernel (dn_scan.hip): one workgroup per (sequence, head, 64-wide
//    d_v tile) walks the chunks in reverse with dh (the gradient w.r.t. the
//    state at the end of the current chunk) in registers, and stores it for
//    every chunk:
//        dV' = P^T dO + diag(w) K dh        (w_r = exp(b_63 - b_r))
//        dX  = T^T dV'
//        dh <- gamma_63 dh + Q^T diag(gamma) dO - K^T diag(gamma) dX
//    dh0 is dh after the first chunk.
//
// 2. bwd_chunk_kernel (dn_bwd_chunk.hip): one workgroup per (chunk, head) with
//    every d_v column computes dq, dk, dv, dbeta and dg from the chunk's
//    inputs, the stored state h_c and the stored dh.
//
// For packed input this file also builds the two tables in the workspace that
// the passes read: the chunk table (the global chunks of every sequence) and
// the order of the sequences, longest first, in which the sequential passes
// hand them to workgroups.
//
// States and state gradients are stored in bf16, transposed (S = h^T,
// [chunk][H][d_v][d_k]): each lane writes the bf16 fragment it feeds its own
// MFMAs with, and the chunk kernel loads them directly into LDS.
//
// Backward is implemented for bf16 inputs (fp32 accumulation and fp32
// gradients).
#include "dn_internal.h"

namespace dn {

// --------------------------------------------------------------- chunk table
// chunk_base[n] is the global index of sequence n's first chunk of C tokens,
// chunk_seq[c] the sequence of global chunk c (-1 past the last chunk).
// Thread t sums the chunk counts of sequences [t R, (t + 1) R), R = ceil(N /
// 256); an exclusive scan of the 256 partial sums in LDS gives each thread
// its first chunk; then every thread fills its sequences' bases and, by
// binary search, a stripe of chunk_seq.
constexpr int TABLE_THREADS = 256;

__global__ __launch_bounds__(TABLE_THREADS) void chunk_table_kernel(const int32_t *cu, int N, int32_t *chunk_base,
                                                                    int32_t *chunk_seq, int max_chunks, int C) {
  __shared__ int part[TABLE_THREADS];
  const int t = threadIdx.x;
  const int per = (N + TABLE_THREADS - 1) / TABLE_THREADS;
  const int n0 = min(N, t * per), n1 = min(N, n0 + per);
  int sum = 0;
  for (int n = n0; n < n1; ++n) sum += (cu[n + 1] - cu[n] + C - 1) / C;
  part[t] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan over the partial sums
  for (int d = 1; d < TABLE_THREADS; d <<= 1) {
    const int add = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int acc = part[t] - sum;  // exclusive prefix
  for (int n = n0; n < n1; ++n) {
    chunk_base[n] = acc;
    acc += (cu[n + 1] - cu[n] + C - 1) / C;
  }
  if (t == TABLE_THREADS - 1) chunk_base[N] = part[TABLE_THREADS - 1];
  __syncthreads();  // chunk_base (global) complete and visible to the workgroup
  const int total = part[TABLE_THREADS - 1];
  for (int c = t; c < max_chunks; c += TABLE_THREADS) {
    int seq = -1;
    if (c < total) {
      int lo = 0, hi = N - 1;  // last n with chunk_base[n] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (chunk_base[mid] <= c) lo = mid;
        else hi = mid - 1;
      }
      seq = lo;
    }
    chunk_seq[c] = seq;
  }
}

hipError_t launch_chunk_table(const int32_t *cu, int N, int32_t *chunk_base, int32_t *chunk_seq,
                              int max_chunks, int chunk, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(TABLE_THREADS), 0, stream, cu, N, chunk_base, chunk_seq,
                     max_chunks, chunk);
  return hipGetLastError();
}

// ------------------------------------------------------------ sequence order
// order[r] is the sequence with the r-th most tokens, ties broken by the lower
// index: the rank of sequence n is the number of sequences that come before it
// in that total order, so the ranks are a permutation of 0 .. N - 1.  Thread n
// ranks sequence n against every length, read through LDS in tiles that all
// threads of the workgroup scan in step (broadcast reads).
constexpr int ORDER_THREADS = 256;
constexpr int ORDER_TILE = 2048;

__global__ __launch_bounds__(ORDER_THREADS) void seq_order_kernel(const int32_t *cu, int N, int32_t *order) {
  __shared__ int lens[ORDER_TILE];
  const int n = blockIdx.x * ORDER_THREADS + threadIdx.x;
  const int len_n = n < N ? cu[n + 1] - cu[n] : 0;
  int rank = 0;
  for (int m0 = 0; m0 < N; m0 += ORDER_TILE) {
    const int cnt = min(ORDER_TILE, N - m0);
    __syncthreads();  // the previous tile is no longer read
    for (int i = threadIdx.x; i < cnt; i += ORDER_THREADS) lens[i] = cu[m0 + i + 1] - cu[m0 + i];
    __syncthreads();
    for (int i = 0; i < cnt; ++i) {
      const int lm = lens[i];
      rank += (lm > len_n) || (lm == len_n && m0 + i < n);
    }
  }
  if (n < N) order[rank] = n;
}

hipError_t launch_seq_order(const int32_t *cu, int N, int32_t *order, hipStream_t stream) {
  if (N <= 0 || N > MAX_ORDERED_SEQS) return hipErrorInvalidValue;
  hipLaunchKernelGGL(seq_order_kernel, dim3((N + ORDER_THREADS - 1) / ORDER_THREADS), dim3(ORDER_THREADS), 0, stream,
                     cu, N, order);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams &p, int dtype, int DK, hipStream_t stream, hipEvent_t ev_scan,
                      hipEvent_t ev_chunk) {
  if (dtype != 1) return hipErrorInvalidValue;  // bf16 only
  hipError_t e = launch_bwd_scan(p, DK, stream);
  if (e != hipSuccess) return e;
  if (ev_scan && (e = hipEventRecord(ev_scan, stream)) != hipSuccess) return e;
  e = launch_bwd_chunk(p, DK, stream);
  if (e != hipSuccess) return e;
  if (ev_chunk) e = hipEventRecord(ev_chunk, stream);
  return e;
}

}  // namespace dn
