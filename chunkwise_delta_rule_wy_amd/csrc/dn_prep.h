// Per-chunk preparation shared by the forward and backward kernels:
//
//   A  = strictLower(diag(beta) (K K^T) * Gamma)      (fp32)
//   P  = (Q K^T) * Gamma, j <= r                       (E)
//   R  = (I + A)^-1,  T = R diag(beta)                 (E)
//
// with Gamma_rj = exp(b_r - b_j).  The products run on MFMA (phase A, five
// 16x16 tiles per wave); the inverse is blocked: the four 16x16 diagonal
// blocks by fp32 forward substitution (every wave, lane (bi, c) computing
// column c of block bi), the off-diagonal blocks by
// R_ij = -R_ii sum_{m=j}^{i-1} A_im R_mj with 16x16x16 MFMAs.  Wave w writes
// block row w of T / R.  This is the UT form of the chunk's WY factors (Gated
// DeltaNet review thread, review 2, which names the UT transform as the
// tensor-core-friendly replacement of the row-by-row WY recurrence of
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", page 1, answer Q1).
//
// Which matrices are produced, row-major or transposed, is a compile-time
// bit set, so every epilogue is straight-line code.  Row-major outputs keep a
// zero upper triangle, transposed ones a zero lower triangle: the caller
// zeroes the selected tiles once (prep_zero) and the prep never writes there.
#pragma once

#include "dn_chunk.h"

namespace dn {

enum : unsigned {
  OUT_P = 1u,    // P row-major
  OUT_PT = 2u,   // P transposed
  OUT_T = 4u,    // T row-major
  OUT_TT = 8u,   // T transposed
  OUT_R = 16u,   // R row-major
  OUT_RT = 32u,  // R transposed
  OUT_AG = 64u,  // strictLower((K K^T) * Gamma) row-major (no beta)
};

constexpr int PREP_LDA = CH + 4;  // fp32 A, padded rows
constexpr int PREP_LDT = 16 + 4;  // fp32 transposed diagonal blocks of A
template <typename E> constexpr int prep_ldr() { return sizeof(E) == 2 ? 20 : 16; }

template <typename E>
struct PrepScratch {  // LDS the prep needs besides its outputs
  float A[CH * PREP_LDA];
  float ATd[4][16 * PREP_LDT];
  E Rr[4][4][16 * prep_ldr<E>()];  // per wave: diagonal R blocks, row-major
  E Rc[4][4][16 * prep_ldr<E>()];  // per wave: diagonal R blocks, column-major
};

template <typename E>
struct PrepOut {
  E *P, *PT, *T, *TT, *R, *RT, *AG;  // 64 x 64 swizzled tiles (selected ones)
};

// zero the selected output tiles (once per kernel)
template <typename E, unsigned OUT>
__device__ __forceinline__ void prep_zero(const PrepOut<E> &o) {
  for (int i = threadIdx.x; i < CH * CH; i += NTHR) {
    const E z = to_e<E>(0.f);
    if (OUT & OUT_P) o.P[i] = z;
    if (OUT & OUT_PT) o.PT[i] = z;
    if (OUT & OUT_T) o.T[i] = z;
    if (OUT & OUT_TT) o.TT[i] = z;
    if (OUT & OUT_R) o.R[i] = z;
    if (OUT & OUT_RT) o.RT[i] = z;
    if (OUT & OUT_AG) o.AG[i] = z;
  }
}

// Transpose a swizzled 64 x D tile into a swizzled D x 64 tile; each thread
// moves 4-row x 16-byte blocks.
template <typename E, int D>
__device__ __forceinline__ void transpose_tile(E *dst, const E *src) {
  using TS = Tile<E, D>;
  using TD = Tile<E, CH>;
  constexpr int EPU = TS::EPU;
  constexpr int NBLK = (CH / 4) * TS::U;
  for (int blk = threadIdx.x; blk < NBLK; blk += NTHR) {
    const int rq = blk / TS::U, u = blk % TS::U;
    E v[4][EPU];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u128 *>(v[i]) = *reinterpret_cast<const u128 *>(src + TS::unit_off(4 * rq + i, u));
#pragma unroll
    for (int e = 0; e < EPU; ++e) {
      typename four<E>::type col;
#pragma unroll
      for (int i = 0; i < 4; ++i) col[i] = v[i][e];
      *reinterpret_cast<typename four<E>::type *>(dst + TD::off(u * EPU + e, 4 * rq)) = col;
    }
  }
}

// store 4 consecutive values of row `row` starting at column c0 (c0 % 4 == 0)
template <typename E>
__device__ __forceinline__ void put4(E *tile, int row, int c0, const f32x4 &v) {
  typename four<E>::type x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = to_e<E>(v[i]);
  *reinterpret_cast<typename four<E>::type *>(tile + Tile<E, CH>::off(row, c0)) = x;
}

// Phase A for one wave role: lower tiles of K K^T (ISK) or Q K^T, two tile
// rows per wave (ODD: rows 1 and 2, else rows 0 and 3; five tiles either way).
template <typename E, int DK, unsigned OUT, bool GATED, bool ISK, bool ODD>
__device__ __forceinline__ void prep_a_role(PrepScratch<E> &s, const PrepOut<E> &o, const E *Kc,
                                            const E *src, const Gates &G) {
  using TT = Tile<E, CH>;
  constexpr int KB = DK / 32;
  const int l = lane_id(), n = l & 15, g = l >> 4;
#pragma unroll
  for (int t = 0; t < 5; ++t) {
    const int ti = ODD ? (t < 2 ? 1 : 2) : (t < 1 ? 0 : 3);
    const int tj = ODD ? (t < 2 ? t : t - 2) : (t < 1 ? 0 : t - 1);
    F32<E> a[KB], bq[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      a[kb] = frag<E, DK>(src, 16 * ti + n, kb);
      bq[kb] = frag<E, DK>(Kc, 16 * tj + n, kb);
    }
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, a[kb], bq[kb]);
    const int j = 16 * tj + n;
    const float bj = G.b[j];
    const f32x4 br = *reinterpret_cast<const f32x4 *>(&G.b[16 * ti + 4 * g]);
    const f32x4 be = *reinterpret_cast<const f32x4 *>(&G.beta[16 * ti + 4 * g]);
    f32x4 v;
    f32x4 ag;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ti + 4 * g + e;
      const float gr = GATED ? __expf(j <= r ? br[e] - bj : 0.f) : 1.f;
      if (ISK) {
        ag[e] = (j < r) ? gr * acc[e] : 0.f;
        v[e] = be[e] * ag[e];
        s.A[r * PREP_LDA + j] = v[e];
        if (OUT & OUT_AG) o.AG[TT::off(r, j)] = to_e<E>(ag[e]);
      } else {
        v[e] = (j <= r) ? gr * acc[e] : 0.f;
        if (OUT & OUT_P) o.P[TT::off(r, j)] = to_e<E>(v[e]);
      }
    }
    if (ISK && ti == tj) *reinterpret_cast<f32x4 *>(&s.ATd[ti][n * PREP_LDT + 4 * g]) = v;
    if (!ISK && (OUT & OUT_PT)) put4<E>(o.PT, j, 16 * ti + 4 * g, v);
  }
}

template <typename E, int DK, unsigned OUT, bool GATED>
__device__ __forceinline__ void prep_a(PrepScratch<E> &s, const PrepOut<E> &o, const E *Kc, const E *Qc,
                                       const Gates &G) {
  constexpr bool NEED_Q = (OUT & (OUT_P | OUT_PT)) != 0;
  const int w = wave_id();
  if (w == 0) prep_a_role<E, DK, OUT, GATED, true, false>(s, o, Kc, Kc, G);
  else if (w == 1) prep_a_role<E, DK, OUT, GATED, true, true>(s, o, Kc, Kc, G);
  else if (NEED_Q && w == 2) prep_a_role<E, DK, OUT, GATED, false, false>(s, o, Kc, Qc, G);
  else if (NEED_Q && w == 3) prep_a_role<E, DK, OUT, GATED, false, true>(s, o, Kc, Qc, G);
}

// Write R block (i, j) (accumulator layout: lane (n, g) holds rows 4g + e of
// column n) into the selected outputs.
template <typename E, unsigned OUT>
__device__ __forceinline__ void prep_put(const PrepOut<E> &o, const Gates &G, int i, int j, const f32x4 &R) {
  using TT = Tile<E, CH>;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const float bj = G.beta[16 * j + n];
  const f32x4 Tv = R * bj;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (OUT & OUT_T) o.T[TT::off(16 * i + 4 * g + e, 16 * j + n)] = to_e<E>(Tv[e]);
    if (OUT & OUT_R) o.R[TT::off(16 * i + 4 * g + e, 16 * j + n)] = to_e<E>(R[e]);
  }
  if (OUT & OUT_TT) put4<E>(o.TT, 16 * j + n, 16 * i + 4 * g, Tv);
  if (OUT & OUT_RT) put4<E>(o.RT, 16 * j + n, 16 * i + 4 * g, R);
}

// Diagonal blocks of R (every wave, into its scratch); wave w also writes
// block (w, w) of the outputs.
template <typename E, unsigned OUT>
__device__ __forceinline__ void prep_inv_diag(PrepScratch<E> &s, const PrepOut<E> &o, const Gates &G) {
  using TT = Tile<E, CH>;
  constexpr int LDR = prep_ldr<E>();
  const int w = wave_id(), l = lane_id(), bi = l >> 4, c = l & 15;
  float x[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = (r == c) ? 1.f : 0.f;
  const float *at = s.ATd[bi];
#pragma unroll
  for (int j = 0; j < 15; ++j) {
    // column j of A_bi: x[r] -= A[r][j] x[j] for r > j
    f32x4 colv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) colv[q] = *reinterpret_cast<const f32x4 *>(at + j * PREP_LDT + 4 * q);
#pragma unroll
    for (int r = j + 1; r < 16; ++r) x[r] -= colv[r >> 2][r & 3] * x[j];
  }
  E *rr = s.Rr[w][bi];
  E *rc = s.Rc[w][bi];
#pragma unroll
  for (int r = 0; r < 16; ++r) rr[r * LDR + c] = to_e<E>(x[r]);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    typename four<E>::type v4;
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = to_e<E>(x[4 * q + i]);
    *reinterpret_cast<typename four<E>::type *>(rc + c * LDR + 4 * q) = v4;
  }
  if (bi == w) {
    const float bc = G.beta[16 * w + c];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (OUT & OUT_T) o.T[TT::off(16 * w + r, 16 * w + c)] = to_e<E>(x[r] * bc);
      if (OUT & OUT_R) o.R[TT::off(16 * w + r, 16 * w + c)] = to_e<E>(x[r]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 xv = {x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]};
      if (OUT & OUT_TT) put4<E>(o.TT, 16 * w + c, 16 * w + 4 * q, xv * bc);
      if (OUT & OUT_RT) put4<E>(o.RT, 16 * w + c, 16 * w + 4 * q, xv);
    }
  }
}

// Off-diagonal blocks of R needed by wave W's block row (straight-line code).
template <typename E, unsigned OUT, int W>
__device__ __forceinline__ void prep_inv_offdiag_w(PrepScratch<E> &s, const PrepOut<E> &o, const Gates &G) {
  constexpr int LDR = prep_ldr<E>();
  constexpr int BS = 16 * LDR;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const E *rr = &s.Rr[W][0][0];
  const E *rc = &s.Rc[W][0][0];
  auto ablk = [&](int i, int k) {  // A_ik rows, fp32 -> E
    f32x4 v = *reinterpret_cast<const f32x4 *>(&s.A[(16 * i + n) * PREP_LDA + 16 * k + 4 * g]);
    F16<E> f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = to_e<E>(v[e]);
    return f;
  };
  auto adiag = [&](int i) { return *reinterpret_cast<const F16<E> *>(rr + i * BS + n * LDR + 4 * g); };
  auto bdiag = [&](int j) { return *reinterpret_cast<const F16<E> *>(rc + j * BS + n * LDR + 4 * g); };
  f32x4 y;
  y = mma16(zero4(), ablk(1, 0), bdiag(0));
  const f32x4 R10 = -mma16(zero4(), adiag(1), bfrag16<E>(y));
  if constexpr (W == 1) {
    prep_put<E, OUT>(o, G, 1, 0, R10);
  } else {
    y = mma16(zero4(), ablk(2, 1), bdiag(1));
    const f32x4 R21 = -mma16(zero4(), adiag(2), bfrag16<E>(y));
    y = mma16(zero4(), ablk(2, 0), bdiag(0));
    y = mma16(y, ablk(2, 1), bfrag16<E>(R10));
    const f32x4 R20 = -mma16(zero4(), adiag(2), bfrag16<E>(y));
    if constexpr (W == 2) {
      prep_put<E, OUT>(o, G, 2, 0, R20);
      prep_put<E, OUT>(o, G, 2, 1, R21);
    } else {
      y = mma16(zero4(), ablk(3, 2), bdiag(2));
      const f32x4 R32 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
      y = mma16(zero4(), ablk(3, 1), bdiag(1));
      y = mma16(y, ablk(3, 2), bfrag16<E>(R21));
      const f32x4 R31 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
      y = mma16(zero4(), ablk(3, 0), bdiag(0));
      y = mma16(y, ablk(3, 1), bfrag16<E>(R10));
      y = mma16(y, ablk(3, 2), bfrag16<E>(R20));
      const f32x4 R30 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
      prep_put<E, OUT>(o, G, 3, 0, R30);
      prep_put<E, OUT>(o, G, 3, 1, R31);
      prep_put<E, OUT>(o, G, 3, 2, R32);
    }
  }
}

template <typename E, unsigned OUT>
__device__ __forceinline__ void prep_inv_offdiag(PrepScratch<E> &s, const PrepOut<E> &o, const Gates &G) {
  const int w = wave_id();
  if (w == 1) prep_inv_offdiag_w<E, OUT, 1>(s, o, G);
  else if (w == 2) prep_inv_offdiag_w<E, OUT, 2>(s, o, G);
  else if (w == 3) prep_inv_offdiag_w<E, OUT, 3>(s, o, G);
}

}  // namespace dn
