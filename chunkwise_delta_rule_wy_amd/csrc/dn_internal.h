// Internal launch interface between the C ABI (dn_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dn_device.h"

namespace dn {

struct FwdParams {
  const void *q, *k, *v;
  const float *beta, *g, *h0;
  const int32_t *cu;          // device offsets, or null for fixed length
  void *o;                    // may be null when o is not written
  float *hT;                  // may be null
  bf16 *states;               // chunk-start states S = h^T, bf16 [chunk][H][DV][DK] (backward only)
  const int32_t *chunk_base;  // varlen: first global chunk of each sequence (backward only)
  const int32_t *seq_order;   // varlen: the sequences longest first, or null (their own order)
  int B, T, H, DV, N, NC;     // NC: chunks per sequence for fixed length
  int ntiles;                 // DV / 64
  int xcd_map;                // 1 when (N * H) % 8 == 0
};

struct BwdParams {
  const void *q, *k, *v, *dO;
  const float *beta, *g, *dhT;
  const int32_t *cu;
  const int32_t *chunk_base;  // varlen: first global chunk of each sequence
  const int32_t *chunk_seq;   // varlen: sequence of each global chunk
  const int32_t *seq_order;   // varlen: the sequences longest first, or null (their own order)
  const bf16 *states;         // chunk-start states S = h^T, bf16 [chunk][H][DV][DK]
  bf16 *dstates;              // gradient w.r.t. each chunk's end state, same layout
  float *dq, *dk, *dv, *dbeta, *dg, *dh0;
  int B, T, H, DV, N, NC;
  int ntiles, xcd_map;
  int total_chunks;           // upper bound of chunks (grid of the chunk-parallel pass)
  int chunk;                  // chunk length: 64, or 32 for the plain gradients
  // input prologue folded into the chunk-gradient kernel (q_in set): dq, dk,
  // dbeta, dg receive the gradients of q_in, k_in, b_in, x_in instead
  const void *q_in, *k_in;
  const float *x_in;
  float gate_scale;
  // Longhorn step size folded in (beta_raw set): beta holds eps = beta_raw /
  // (1 + beta_raw |k|^2), dbeta receives the gradient of beta_raw and dk the
  // step size's key term
  const float *beta_raw;
};

struct StepParams {
  const void *q, *k, *v;
  const float *beta, *g;
  float *state;
  void *o;
  int B, H, DV;
};

// Longhorn step size (eps set) or its backward (dk set): rows = B T H key rows
struct LonghornParams {
  const void *k;
  const float *beta;
  float *eps;                 // forward output
  const float *deps;          // backward input
  float *dbeta, *dk;          // backward outputs (dk accumulated)
  int64_t rows;
};

// Input prologue (forward: q, k, beta, g from q_in, k_in, b_in, x_in) and its
// backward (dq_in, dk_in, db_in, dx_in from dq, dk, dbeta, dg); rows = B T H
struct PrologueParams {
  const void *q_in, *k_in;
  const float *b_in, *x_in;   // x_in null: no gate
  float gate_scale;
  void *q, *k;
  float *beta, *g;
  const float *dq, *dk, *dbeta, *dg;
  float *dq_in, *dk_in, *db_in, *dx_in;
  int64_t rows;
};

// Depthwise causal short convolution over TT = B T tokens of C = H D channels
// (x, y [TT][C] in the dtype; w, dw [C][W] fp32; dy, dx [TT][C] fp32)
struct ConvParams {
  const void *x;
  const float *w;
  const int32_t *cu;          // packed sequences, or null: sequences of T tokens
  void *y;
  const float *dy;
  float *dx, *dw;
  int64_t TT;
  int T, N;                   // tokens per sequence (cu null); sequences (cu set)
  int C, W;
  int norm_lanes;             // 0, or D / 8: L2-normalise every (token, head) row of D channels
};

struct SeqInfo {
  int b, t0, len;
};

__device__ __forceinline__ SeqInfo seq_info(const int32_t *cu, int n, int T) {
  SeqInfo s;
  if (cu) {
    s.b = 0;
    s.t0 = cu[n];
    s.len = cu[n + 1] - s.t0;
  } else {
    s.b = n;
    s.t0 = 0;
    s.len = T;
  }
  return s;
}

// (pair, tile) of a workgroup.  Workgroups are dealt to the 8 XCDs round
// robin; the d_v tiles of one (sequence, head) share K and Q, so they are
// placed on one XCD (one L2).
__device__ __forceinline__ void wg_coords(int x, int ntiles, int xcd_map, int &pair, int &tile) {
  if (xcd_map) {
    const int xcd = x & 7, slot = x >> 3;
    pair = (slot / ntiles) * 8 + xcd;
    tile = slot % ntiles;
  } else {
    pair = x / ntiles;
    tile = x % ntiles;
  }
}

// Sequence of the pair rank r (pair index / H).  Packed input with an order
// table walks the sequences longest first: the workgroups of the longest
// sequence, whose chunk chain is the pass's critical path, then start in the
// first wave of workgroups instead of waiting for a CU.
__device__ __forceinline__ int pair_seq(const int32_t *order, int r) { return order ? order[r] : r; }

size_t fwd_smem_bytes(int dtype, int DK);
size_t fwd_ref_smem_bytes(int dtype, int DK);
hipError_t launch_fwd(const FwdParams &p, int dtype, int DK, bool store_states, bool write_o,
                      hipStream_t stream);
// the forward pass with 32-token chunks (bf16)
hipError_t launch_fwd_c32(const FwdParams &p, int DK, bool store_states, bool write_o, hipStream_t stream);
hipError_t launch_fwd_ref(const FwdParams &p, int dtype, int DK, bool store_states,
                          bool write_o, hipStream_t stream);
hipError_t launch_step(const StepParams &p, int dtype, int DK, hipStream_t stream);
hipError_t launch_longhorn(const LonghornParams &p, int dtype, int DK, hipStream_t stream);
hipError_t launch_prologue(const PrologueParams &p, int dtype, int DK, bool backward, hipStream_t stream);
// forward (y) or backward (dx, dw; dw is cleared first); W in 1..4
hipError_t launch_conv(const ConvParams &p, int dtype, bool backward, hipStream_t stream);
hipError_t launch_chunk_table(const int32_t *cu, int N, int32_t *chunk_base, int32_t *chunk_seq,
                              int max_chunks, int chunk, hipStream_t stream);
// order[r] = the sequence with the r-th most tokens (ties: the lower index
// first), for N <= MAX_ORDERED_SEQS sequences
constexpr int MAX_ORDERED_SEQS = 65536;
hipError_t launch_seq_order(const int32_t *cu, int N, int32_t *order, hipStream_t stream);
// ev_scan / ev_chunk (may be null) are recorded on `stream` after the scan and
// after the chunk-gradient kernel
hipError_t launch_bwd(const BwdParams &p, int dtype, int DK, hipStream_t stream, hipEvent_t ev_scan = nullptr,
                      hipEvent_t ev_chunk = nullptr);
hipError_t launch_bwd_scan(const BwdParams &p, int DK, hipStream_t stream);
hipError_t launch_bwd_chunk(const BwdParams &p, int DK, hipStream_t stream);

}  // namespace dn
