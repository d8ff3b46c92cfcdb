// Backward pass of the chunkwise (gated) delta rule for gfx950.
//
// The forward pass keeps chunk states on chip, so the backward pass first
// recomputes them (the forward kernel in its state-storing variant writes
// h_c, the state entering chunk c), following the recompute-in-the-backward
// design of "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length" (page 1, answer Q2).  Then:
//
// 1. scan_kernel: one workgroup per (sequence, head, 64-wide d_v tile) walks
//    the chunks in reverse with dh (the gradient w.r.t. the state at the end
//    of the current chunk) in registers, and stores it for every chunk:
//        dV' = P^T dO + diag(w) K dh        (w_r = exp(b_64 - b_r))
//        dX  = T^T dV'
//        dh <- gamma_64 dh + Q^T diag(gamma) dO - K^T diag(gamma) dX
//    dh0 is dh after the first chunk.
//
// 2. chunk_kernel: one workgroup per (chunk, head) with every d_v column,
//    so the products that contract over d_v need no cross-workgroup sums:
//        X = V - diag(gamma) K h,  V' = T X,  dV', dX as above (dv = dX)
//        dP = (dO V'^T) masked,  dT = dV' X^T,  dR = dT diag(beta)
//        dA = -strictLower(R^T dR R^T)
//        dq = diag(gamma) dO h^T + (dP * Gamma) K
//        dk = (dP * Gamma)^T Q - diag(gamma) dX h^T + diag(w) V' dh^T
//             + F K + F^T K,          F = dA * Gamma * (beta 1^T)
//        dbeta_j = sum_r R_rj dT_rj + sum_l dA_jl (K K^T * Gamma)_jl
//        db = gamma * rowsum(dO * Q h) - rowsum(dX * (V - X))
//             - w * rowsum(V' dh^T * K) + rowsum(E) - colsum(E)
//             + e_64 [sum_r w_r (V' dh^T)_r . k_r + gamma_64 <dh, h>],
//        E = dP * P + dA * A,   dg = reverse cumsum of db in the chunk.
//    These are the derivatives of the chunk form written out (the chunk form
//    itself is an exact refactoring of the token recurrence, so the result is
//    the gradient of the recurrence).
//
// Backward is implemented for bf16 inputs (fp32 accumulation and fp32
// gradients).
#include "dn_internal.h"
#include "dn_prep.h"

namespace dn {

// --------------------------------------------------------------- chunk table
// chunk_base[n] is the global index of sequence n's first chunk,
// chunk_seq[c] the sequence of global chunk c (-1 past the last chunk).
__global__ void chunk_table_kernel(const int32_t *cu, int N, int32_t *chunk_base, int32_t *chunk_seq,
                                   int max_chunks) {
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int n = 0; n < N; ++n) {
      chunk_base[n] = acc;
      acc += (cu[n + 1] - cu[n] + 63) / 64;
    }
    chunk_base[N] = acc;
  }
  __syncthreads();
  const int total = chunk_base[N];
  for (int c = threadIdx.x; c < max_chunks; c += blockDim.x) {
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
                              int max_chunks, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, stream, cu, N, chunk_base, chunk_seq,
                     max_chunks);
  return hipGetLastError();
}

// (sequence, token offset, length) of a sequence
struct Seq {
  int b, t0, len;
};
__device__ __forceinline__ Seq seq_of(const BwdParams &p, int n) {
  Seq s;
  if (p.cu) {
    s.b = 0;
    s.t0 = p.cu[n];
    s.len = p.cu[n + 1] - s.t0;
  } else {
    s.b = n;
    s.t0 = 0;
    s.len = p.T;
  }
  return s;
}
__device__ __forceinline__ int global_chunk(const BwdParams &p, int n, int c) {
  return p.chunk_base ? p.chunk_base[n] + c : n * p.NC + c;
}

// ------------------------------------------------------------- reverse scan
template <int DK>
struct ScanSmem {
  bf16 K[2][CH * DK];
  bf16 Q[CH * DK];
  bf16 dO[2][CH * DVT];
  bf16 KT[DK * CH];
  bf16 QT[DK * CH];
  bf16 PT[CH * CH];
  bf16 TT[CH * CH];
  PrepScratch<bf16> ps;
  Gates G[2];
};

// B fragment of a row-major 64 x 64 tile with the contraction over its rows:
// lane (n, g) takes rows 32kb + 8g .. +7 of column col.
__device__ __forceinline__ F32<bf16> bfrag_rows(const bf16 *tile, int col, int kb) {
  using TT = Tile<bf16, CH>;
  const int g = lane_id() >> 4;
  F32<bf16> f;
#pragma unroll
  for (int j = 0; j < 8; ++j) f[j] = tile[TT::off(32 * kb + 8 * g + j, col)];
  return f;
}
// same, each row r scaled by s[r]
__device__ __forceinline__ F32<bf16> bfrag_rows_scaled(const bf16 *tile, int col, int kb, const float *s) {
  using TT = Tile<bf16, CH>;
  const int g = lane_id() >> 4;
  const f32x4 s0 = *reinterpret_cast<const f32x4 *>(s + 32 * kb + 8 * g);
  const f32x4 s1 = *reinterpret_cast<const f32x4 *>(s + 32 * kb + 8 * g + 4);
  F32<bf16> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = to_e<bf16>(s0[j] * to_f<bf16>(tile[TT::off(32 * kb + 8 * g + j, col)]));
    f[4 + j] = to_e<bf16>(s1[j] * to_f<bf16>(tile[TT::off(32 * kb + 8 * g + 4 + j, col)]));
  }
  return f;
}

template <int DK, bool GATED>
__global__ __launch_bounds__(NTHR, 1) void scan_kernel(BwdParams p) {
  using SM = ScanSmem<DK>;
  using E = bf16;
  constexpr int KB = DK / 32, MTK = DK / 16;
  constexpr unsigned OUT = OUT_PT | OUT_TT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);

  int pair, tile;
  {
    const int x = blockIdx.x;
    if (p.xcd_map) {
      const int xcd = x & 7, slot = x >> 3;
      pair = (slot / p.ntiles) * 8 + xcd;
      tile = slot % p.ntiles;
    } else {
      pair = x / p.ntiles;
      tile = x % p.ntiles;
    }
  }
  if (pair >= p.N * p.H) return;
  const int n_seq = pair / p.H, h = pair % p.H;
  const int dv0 = tile * DVT;
  const Seq sq = seq_of(p, n_seq);
  const int nch = (sq.len + CH - 1) / CH;
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gdo = static_cast<const E *>(p.dO);
  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const int cl = 16 * w + n;       // column inside the tile
  const int col = dv0 + cl;        // d_v column
  const size_t row_base = (size_t)sq.b * p.T + sq.t0;

  PrepOut<E> po = {};
  po.PT = sm.PT;
  po.TT = sm.TT;
  prep_zero<E, OUT>(po);

  // dh: lane (n, g) holds rows prow(mt, 4g + i) of column `col`
  f32x4 hacc[MTK];
  const size_t st_base = ((size_t)n_seq * p.H + h) * DK * p.DV;
#pragma unroll
  for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hacc[mt][i] = p.dhT ? p.dhT[st_base + (size_t)prow(mt, 4 * g + i) * p.DV + col] : 0.f;

  auto chunk_len = [&](int c) { return min(CH, sq.len - c * CH); };
  auto load_scalars = [&](int c) {
    const int L = chunk_len(c);
    float s = 0.f;
    if (l < L) {
      const size_t idx = (row_base + (size_t)c * CH + l) * p.H + h;
      if (GATED && w == 0) s = p.g[idx];
      if (w == 1) s = p.beta[idx];
    }
    return s;
  };
  auto issue_kdo = [&](int c, int buf) {
    const int L = chunk_len(c);
    const size_t r0 = row_base + (size_t)c * CH;
    dma_tile<E, DK>(sm.K[buf], gk, r0, p.H, h, DK, 0, L);
    dma_tile<E, DVT>(sm.dO[buf], gdo, r0, p.H, h, p.DV, dv0, L);
  };
  auto issue_q = [&](int c) {
    dma_tile<E, DK>(sm.Q, gq, row_base + (size_t)c * CH, p.H, h, DK, 0, chunk_len(c));
  };

  float sc = 0.f;
  if (nch > 0) {
    issue_kdo(nch - 1, 0);
    issue_q(nch - 1);
    sc = load_scalars(nch - 1);
  }
  for (int it = 0; it < nch; ++it) {
    const int c = nch - 1 - it;
    const int cur = it & 1;
    const int L = chunk_len(c);
    const E *Kc = sm.K[cur];
    const E *dOc = sm.dO[cur];
    Gates &G = sm.G[it & 1];
    wait_vmem();
    if (L < CH) {
      zero_rows<E, DK>(sm.K[cur], L);
      zero_rows<E, DK>(sm.Q, L);
      zero_rows<E, DVT>(sm.dO[cur], L);
    }
    write_gates(G, w == 0 ? sc : 0.f, w == 1 ? sc : 0.f);
    __syncthreads();
    if (c > 0) issue_kdo(c - 1, cur ^ 1);

    // dh of this chunk's end state, for the chunk-parallel pass
    {
      float *dst = p.dstates + ((size_t)global_chunk(p, n_seq, c) * p.H + h) * DK * p.DV;
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(size_t)prow(mt, 4 * g + i) * p.DV + col] = hacc[mt][i];
    }
    transpose_tile<E, DK>(sm.KT, Kc);
    transpose_tile<E, DK>(sm.QT, sm.Q);
    prep_a<E, DK, OUT, GATED>(sm.ps, po, Kc, sm.Q, G);
    __syncthreads();
    if (c > 0) {
      issue_q(c - 1);  // Q was consumed by phase A and the transpose
      sc = load_scalars(c - 1);
    }

    // K dh and P^T dO, overlapped with the UT inverse
    F32<E> hb[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) hb[kb] = bfrag<E>(hacc[2 * kb], hacc[2 * kb + 1]);
    f32x4 kd[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      kd[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kd[mt] = mma32(kd[mt], frag<E, DK>(Kc, prow(mt, n), kb), hb[kb]);
    }
    prep_inv_diag<E, OUT>(sm.ps, po, G);
    const F32<E> dob0 = bfrag_rows(dOc, cl, 0), dob1 = bfrag_rows(dOc, cl, 1);
    f32x4 pd[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      pd[mt] = mma32(mma32(zero4(), frag<E, CH>(sm.PT, prow(mt, n), 0), dob0),
                     frag<E, CH>(sm.PT, prow(mt, n), 1), dob1);
    wave_lds_fence();
    prep_inv_offdiag<E, OUT>(sm.ps, po, G);
    mfma_settle();
    __syncthreads();

    // dV' = P^T dO + diag(w) K dh ;  dX = T^T dV'
    f32x4 dvp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 wl = *reinterpret_cast<const f32x4 *>(&G.wl[prow(mt, 4 * g)]);
      dvp[mt] = pd[mt] + wl * kd[mt];
    }
    const F32<E> vb0 = bfrag<E>(dvp[0], dvp[1]), vb1 = bfrag<E>(dvp[2], dvp[3]);
    f32x4 gdx[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 dx = mma32(mma32(zero4(), frag<E, CH>(sm.TT, prow(mt, n), 0), vb0),
                             frag<E, CH>(sm.TT, prow(mt, n), 1), vb1);
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(&G.gam[prow(mt, 4 * g)]);
      gdx[mt] = -(gm * dx);
    }
    // dh <- gamma_64 dh + Q^T diag(gamma) dO - K^T diag(gamma) dX
    const F32<E> gob0 = bfrag_rows_scaled(dOc, cl, 0, G.gam), gob1 = bfrag_rows_scaled(dOc, cl, 1, G.gam);
    const F32<E> xb0 = bfrag<E>(gdx[0], gdx[1]), xb1 = bfrag<E>(gdx[2], gdx[3]);
    const float glast = G.gam[CH - 1];
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) {
      f32x4 acc = hacc[mt] * glast;
      acc = mma32(acc, frag<E, CH>(sm.QT, prow(mt, n), 0), gob0);
      acc = mma32(acc, frag<E, CH>(sm.QT, prow(mt, n), 1), gob1);
      acc = mma32(acc, frag<E, CH>(sm.KT, prow(mt, n), 0), xb0);
      acc = mma32(acc, frag<E, CH>(sm.KT, prow(mt, n), 1), xb1);
      hacc[mt] = acc;
    }
    mfma_settle();
  }
  if (p.dh0) {
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.dh0[st_base + (size_t)prow(mt, 4 * g + i) * p.DV + col] = hacc[mt][i];
  }
}

// ------------------------------------------------------- chunk-parallel pass
template <int DK>
struct ChunkSmem {
  bf16 K[CH * DK];
  bf16 Q[CH * DK];
  bf16 R[CH * CH];
  bf16 RT[CH * CH];
  bf16 P[CH * CH];
  bf16 PT[CH * CH];
  bf16 AG[CH * CH];
  Gates G;
  float red[4][CH];   // per-wave partial column sums
  float red2[4][CH];
  float db[CH], dbeta[CH];
  float hdh[NTHR / 64];
  float s3[NTHR / 64];
  union U {
    PrepScratch<bf16> ps;
    struct Loop {  // one d_v tile
      bf16 h[DK * CH];
      bf16 dh[DK * CH];
      bf16 dO[CH * CH];
      bf16 V[CH * CH];
      bf16 X[CH * CH];
      bf16 Vp[CH * CH];
      bf16 dVp[CH * CH];
      bf16 dX[CH * CH];
    } lp;
    struct Fin {  // final products
      bf16 KT[DK * CH];
      bf16 QT[DK * CH];
      bf16 dR[CH * CH];
      bf16 Zt[CH * CH];
      bf16 dPG[CH * CH];
      bf16 dPGT[CH * CH];
      bf16 F[CH * CH];
      bf16 FT[CH * CH];
    } fin;
  } u;
};

// load rows [0, L) of a 64-row slice of a [rows, H, D] bf16 tensor into a
// swizzled tile (rows >= L zero)
template <int COLS>
__device__ __forceinline__ void load_tile(bf16 *tile, const bf16 *g, size_t row0, int H, int h, int D, int col0,
                                          int L) {
  using TL = Tile<bf16, COLS>;
  for (int p = threadIdx.x; p < CH * TL::U; p += NTHR) {
    const int r = p / TL::U, u = p % TL::U;
    u128 v = zero128();
    if (r < L) v = ldg128(g + ((row0 + r) * H + h) * (size_t)D + col0 + u * 8);
    *reinterpret_cast<u128 *>(tile + TL::unit_off(r, u)) = v;
  }
}

// load a DK x 64 slice (columns dv0 .. dv0+63) of an fp32 [DK, DV] state into
// a bf16 tile; returns this thread's share of sum(a * b) over two such states
template <int DK>
__device__ __forceinline__ float load_state_pair(bf16 *ta, bf16 *tb, const float *a, const float *b, int DV,
                                                 int dv0) {
  using TL = Tile<bf16, CH>;
  float dot = 0.f;
  for (int p = threadIdx.x; p < DK * TL::U; p += NTHR) {
    const int r = p / TL::U, u = p % TL::U;
    const float *pa = a + (size_t)r * DV + dv0 + u * 8;
    const float *pb = b + (size_t)r * DV + dv0 + u * 8;
    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(pa), a1 = *reinterpret_cast<const f32x4 *>(pa + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(pb), b1 = *reinterpret_cast<const f32x4 *>(pb + 4);
    F32<bf16> va, vb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      va[i] = to_e<bf16>(a0[i]);
      va[4 + i] = to_e<bf16>(a1[i]);
      vb[i] = to_e<bf16>(b0[i]);
      vb[4 + i] = to_e<bf16>(b1[i]);
      dot += a0[i] * b0[i] + a1[i] * b1[i];
    }
    *reinterpret_cast<F32<bf16> *>(ta + TL::unit_off(r, u)) = va;
    *reinterpret_cast<F32<bf16> *>(tb + TL::unit_off(r, u)) = vb;
  }
  return dot;
}

// sum over the 16 lanes of a lane group (same g)
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// sum over the 4 lane groups (same n)
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <int DK, bool GATED>
__global__ __launch_bounds__(NTHR, 1) void chunk_kernel(BwdParams p) {
  using SM = ChunkSmem<DK>;
  using E = bf16;
  using TT = Tile<E, CH>;
  constexpr int KB = DK / 32, NTK = DK / 16;
  constexpr unsigned OUT = OUT_P | OUT_PT | OUT_R | OUT_RT | OUT_AG;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);

  const int cgl = blockIdx.x / p.H, h = blockIdx.x % p.H;
  int n_seq, c;
  if (p.chunk_seq) {
    if (cgl >= p.total_chunks) return;
    n_seq = p.chunk_seq[cgl];
    if (n_seq < 0) return;
    c = cgl - p.chunk_base[n_seq];
  } else {
    n_seq = cgl / p.NC;
    c = cgl % p.NC;
  }
  const Seq sq = seq_of(p, n_seq);
  const int L = min(CH, sq.len - c * CH);
  const size_t r0 = (size_t)sq.b * p.T + sq.t0 + (size_t)c * CH;  // global row of the chunk
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gv = static_cast<const E *>(p.v);
  const E *gdo = static_cast<const E *>(p.dO);
  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;

  PrepOut<E> po = {};
  po.P = sm.P;
  po.PT = sm.PT;
  po.R = sm.R;
  po.RT = sm.RT;
  po.AG = sm.AG;
  prep_zero<E, OUT>(po);
  load_tile<DK>(sm.K, gk, r0, p.H, h, DK, 0, L);
  load_tile<DK>(sm.Q, gq, r0, p.H, h, DK, 0, L);
  {
    float s = 0.f;
    if (l < L) {
      const size_t idx = (r0 + l) * p.H + h;
      if (GATED && w == 0) s = p.g[idx];
      if (w == 1) s = p.beta[idx];
    }
    write_gates(sm.G, w == 0 ? s : 0.f, w == 1 ? s : 0.f);
  }
  __syncthreads();
  const Gates &G = sm.G;
  prep_a<E, DK, OUT, GATED>(sm.u.ps, po, sm.K, sm.Q, G);
  __syncthreads();
  prep_inv_diag<E, OUT>(sm.u.ps, po, G);
  wave_lds_fence();
  prep_inv_offdiag<E, OUT>(sm.u.ps, po, G);
  mfma_settle();
  __syncthreads();

  const size_t cgidx = (size_t)global_chunk(p, n_seq, c);
  const float *hs = p.states + (cgidx * p.H + h) * DK * p.DV;
  const float *dhs = p.dstates + (cgidx * p.H + h) * DK * p.DV;

  // accumulators over d_v; wave w owns rows 16w .. 16w+15
  f32x4 dP[4], dT[4], DQ[NTK], DX[NTK], DH[NTK];
#pragma unroll
  for (int t = 0; t < 4; ++t) dP[t] = dT[t] = zero4();
#pragma unroll
  for (int t = 0; t < NTK; ++t) DQ[t] = DX[t] = DH[t] = zero4();
  float hdh = 0.f;
  auto &lp = sm.u.lp;
  const int cl = 16 * w + n;  // this lane's column inside a d_v tile

  for (int tile = 0; tile < p.ntiles; ++tile) {
    const int dv0 = tile * DVT;
    __syncthreads();  // previous tile's readers are done
    hdh += load_state_pair<DK>(lp.h, lp.dh, hs, dhs, p.DV, dv0);
    load_tile<CH>(lp.dO, gdo, r0, p.H, h, p.DV, dv0, L);
    load_tile<CH>(lp.V, gv, r0, p.H, h, p.DV, dv0, L);
    __syncthreads();

    // ---- chain for this wave's 16 columns (rows in prow order)
    F32<E> hb[KB], db_[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      F32<E> a, b;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[j] = lp.h[TT::off(32 * kb + 8 * g + j, cl)];
        b[j] = lp.dh[TT::off(32 * kb + 8 * g + j, cl)];
      }
      hb[kb] = a;
      db_[kb] = b;
    }
    f32x4 x[4], kd[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 yk = zero4(), k2 = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const F32<E> ka = frag<E, DK>(sm.K, prow(mt, n), kb);
        yk = mma32(yk, ka, hb[kb]);
        k2 = mma32(k2, ka, db_[kb]);
      }
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(&G.gam[prow(mt, 4 * g)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[mt][i] = to_f<E>(lp.V[TT::off(prow(mt, 4 * g + i), cl)]) - gm[i] * yk[i];
      kd[mt] = k2;
    }
    // V' = R diag(beta) X
    f32x4 bx[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) bx[mt] = x[mt] * *reinterpret_cast<const f32x4 *>(&G.beta[prow(mt, 4 * g)]);
    const F32<E> xb0 = bfrag<E>(bx[0], bx[1]), xb1 = bfrag<E>(bx[2], bx[3]);
    const F32<E> ob0 = bfrag_rows(lp.dO, cl, 0), ob1 = bfrag_rows(lp.dO, cl, 1);
    f32x4 vp[4], dvp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      vp[mt] = mma32(mma32(zero4(), frag<E, CH>(sm.R, prow(mt, n), 0), xb0), frag<E, CH>(sm.R, prow(mt, n), 1), xb1);
      const f32x4 pd = mma32(mma32(zero4(), frag<E, CH>(sm.PT, prow(mt, n), 0), ob0),
                             frag<E, CH>(sm.PT, prow(mt, n), 1), ob1);
      const f32x4 wl = *reinterpret_cast<const f32x4 *>(&G.wl[prow(mt, 4 * g)]);
      dvp[mt] = pd + wl * kd[mt];
    }
    // dX = diag(beta) R^T dV'
    const F32<E> vb0 = bfrag<E>(dvp[0], dvp[1]), vb1 = bfrag<E>(dvp[2], dvp[3]);
    f32x4 dx[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 rt = mma32(mma32(zero4(), frag<E, CH>(sm.RT, prow(mt, n), 0), vb0),
                             frag<E, CH>(sm.RT, prow(mt, n), 1), vb1);
      dx[mt] = rt * *reinterpret_cast<const f32x4 *>(&G.beta[prow(mt, 4 * g)]);
    }
    // outputs of the chain: dv, and X, V', dV', dX row-major for the d_v products
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = prow(mt, 4 * g + i);
        if (r < L) p.dv[((r0 + r) * p.H + h) * p.DV + dv0 + cl] = dx[mt][i];
        lp.X[TT::off(r, cl)] = to_e<E>(x[mt][i]);
        lp.Vp[TT::off(r, cl)] = to_e<E>(vp[mt][i]);
        lp.dVp[TT::off(r, cl)] = to_e<E>(dvp[mt][i]);
        lp.dX[TT::off(r, cl)] = to_e<E>(dx[mt][i]);
      }
    __syncthreads();

    // ---- products contracting over this tile's 64 d_v columns
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ra = 16 * w + n;
      const F32<E> a_do = frag<E, CH>(lp.dO, ra, kb);
      const F32<E> a_dvp = frag<E, CH>(lp.dVp, ra, kb);
      const F32<E> a_dx = frag<E, CH>(lp.dX, ra, kb);
      const F32<E> a_vp = frag<E, CH>(lp.Vp, ra, kb);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dP[t] = mma32(dP[t], a_do, frag<E, CH>(lp.Vp, 16 * t + n, kb));
        dT[t] = mma32(dT[t], a_dvp, frag<E, CH>(lp.X, 16 * t + n, kb));
      }
#pragma unroll
      for (int t = 0; t < NTK; ++t) {
        const F32<E> bh = frag<E, CH>(lp.h, 16 * t + n, kb);
        DQ[t] = mma32(DQ[t], a_do, bh);
        DX[t] = mma32(DX[t], a_dx, bh);
        DH[t] = mma32(DH[t], a_vp, frag<E, CH>(lp.dh, 16 * t + n, kb));
      }
    }
  }
  mfma_settle();
  {
    const float s = wave_sum(hdh);  // this wave's share of <dh, h>
    if (l == 0) sm.hdh[w] = s;
  }
  __syncthreads();

  auto &fn = sm.u.fin;
  const int rbase = 16 * w + 4 * g;  // rows rbase + i of this lane's tiles
  const f32x4 bet_r = *reinterpret_cast<const f32x4 *>(&G.beta[rbase]);
  const f32x4 gam_r = *reinterpret_cast<const f32x4 *>(&G.gam[rbase]);
  const f32x4 wl_r = *reinterpret_cast<const f32x4 *>(&G.wl[rbase]);
  const f32x4 b_r = *reinterpret_cast<const f32x4 *>(&G.b[rbase]);

  // dPG = dP * Gamma (j <= r); E1 = dP * P; dR = dT diag(beta); colsum(R * dT)
  f32x4 dPG[4], E1[4];
  float csT[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 16 * t + n;
    const float bj = G.b[j], betj = G.beta[j];
    float ct = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + i;
      const float gr = GATED ? __expf(j <= r ? b_r[i] - bj : 0.f) : 1.f;
      dPG[t][i] = (j <= r) ? dP[t][i] * gr : 0.f;
      E1[t][i] = dP[t][i] * to_f<E>(sm.P[TT::off(r, j)]);
      ct += to_f<E>(sm.R[TT::off(r, j)]) * dT[t][i];
      fn.dR[TT::off(r, j)] = to_e<E>(dT[t][i] * betj);
    }
    csT[t] = sum_groups(ct);
  }
  __syncthreads();  // dR complete
  // Z = dR R^T, stored transposed
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const f32x4 z = mma32(mma32(zero4(), frag<E, CH>(fn.dR, 16 * w + n, 0), frag<E, CH>(sm.R, 16 * t + n, 0)),
                          frag<E, CH>(fn.dR, 16 * w + n, 1), frag<E, CH>(sm.R, 16 * t + n, 1));
    put4<E>(fn.Zt, 16 * t + n, rbase, z);
  }
  __syncthreads();
  // dA = -strictLower(R^T Z);  F = dA * Gamma * beta_r;  E = E1 + dA * A
  f32x4 F[4];
  f32x4 Erow = zero4(), dbr = zero4();
  float csE[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const f32x4 m = mma32(mma32(zero4(), frag<E, CH>(sm.RT, 16 * w + n, 0), frag<E, CH>(fn.Zt, 16 * t + n, 0)),
                          frag<E, CH>(sm.RT, 16 * w + n, 1), frag<E, CH>(fn.Zt, 16 * t + n, 1));
    const int j = 16 * t + n;
    const float bj = G.b[j];
    float ce = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + i;
      const float da = (j < r) ? -m[i] : 0.f;
      const float ag = to_f<E>(sm.AG[TT::off(r, j)]);   // (K K^T * Gamma)_rj, j < r
      const float gr = GATED ? __expf(j < r ? b_r[i] - bj : 0.f) : 1.f;
      F[t][i] = da * gr * bet_r[i];
      dbr[i] += da * ag;
      const float e = E1[t][i] + da * ag * bet_r[i];
      Erow[i] += e;
      ce += e;
    }
    csE[t] = sum_groups(ce);
  }
  if (g == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sm.red[w][16 * t + n] = csT[t];
      sm.red2[w][16 * t + n] = csE[t];
    }
  }
  // row terms: gamma_r q_r . DQ_r - gamma_r k_r . DX_r - w_r k_r . DH_r ;
  // and sum_r w_r k_r . DH_r for the last row
  f32x4 rowt = zero4();
  float s3 = 0.f;
#pragma unroll
  for (int t = 0; t < NTK; ++t) {
    const int i2 = 16 * t + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + i;
      const float qv = to_f<E>(sm.Q[Tile<E, DK>::off(r, i2)]);
      const float kv = to_f<E>(sm.K[Tile<E, DK>::off(r, i2)]);
      const float kdh = kv * DH[t][i];
      rowt[i] += gam_r[i] * (qv * DQ[t][i] - kv * DX[t][i]) - wl_r[i] * kdh;
      s3 += wl_r[i] * kdh;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rowt[i] = sum16(rowt[i] + Erow[i]);
    dbr[i] = sum16(dbr[i]);
  }
  s3 = wave_sum(s3);
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.db[rbase + i] = rowt[i];
      sm.dbeta[rbase + i] = dbr[i];
    }
  }
  if (l == 0) sm.s3[w] = s3;
  // dPG, dPG^T, F, F^T; K^T, Q^T
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int j = 16 * t + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fn.dPG[TT::off(rbase + i, j)] = to_e<E>(dPG[t][i]);
      fn.F[TT::off(rbase + i, j)] = to_e<E>(F[t][i]);
    }
    put4<E>(fn.dPGT, j, rbase, dPG[t]);
    put4<E>(fn.FT, j, rbase, F[t]);
  }
  transpose_tile<E, DK>(fn.KT, sm.K);
  transpose_tile<E, DK>(fn.QT, sm.Q);
  __syncthreads();

  // dq = diag(gamma) dO h^T + dPG K ;  dk = dPG^T Q - diag(gamma) dX h^T + diag(w) V' dh^T + F K + F^T K
#pragma unroll
  for (int t = 0; t < NTK; ++t) {
    const F32<E> k0 = frag<E, CH>(fn.KT, 16 * t + n, 0), k1 = frag<E, CH>(fn.KT, 16 * t + n, 1);
    const F32<E> q0 = frag<E, CH>(fn.QT, 16 * t + n, 0), q1 = frag<E, CH>(fn.QT, 16 * t + n, 1);
    f32x4 dq = gam_r * DQ[t];
    dq = mma32(dq, frag<E, CH>(fn.dPG, 16 * w + n, 0), k0);
    dq = mma32(dq, frag<E, CH>(fn.dPG, 16 * w + n, 1), k1);
    f32x4 dk = wl_r * DH[t] - gam_r * DX[t];
    dk = mma32(dk, frag<E, CH>(fn.dPGT, 16 * w + n, 0), q0);
    dk = mma32(dk, frag<E, CH>(fn.dPGT, 16 * w + n, 1), q1);
    dk = mma32(dk, frag<E, CH>(fn.F, 16 * w + n, 0), k0);
    dk = mma32(dk, frag<E, CH>(fn.F, 16 * w + n, 1), k1);
    dk = mma32(dk, frag<E, CH>(fn.FT, 16 * w + n, 0), k0);
    dk = mma32(dk, frag<E, CH>(fn.FT, 16 * w + n, 1), k1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rbase + i;
      if (r < L) {
        const size_t o = ((r0 + r) * p.H + h) * DK + 16 * t + n;
        p.dq[o] = dq[i];
        p.dk[o] = dk[i];
      }
    }
  }
  // dbeta, db -> dg (reverse cumulative sum inside the chunk)
  if (w == 0) {
    const int r = l;
    float cT = 0.f, cE = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      cT += sm.red[ww][r];
      cE += sm.red2[ww][r];
    }
    float db = sm.db[r] - cE;
    if (r == CH - 1) {
      const float s3t = sm.s3[0] + sm.s3[1] + sm.s3[2] + sm.s3[3];
      const float hdt = sm.hdh[0] + sm.hdh[1] + sm.hdh[2] + sm.hdh[3];
      db += s3t + G.gam[CH - 1] * hdt;
    }
    const float incl = wave_incl_scan(db);
    const float total = __shfl(incl, 63, 64);
    const float dgv = total - incl + db;  // sum_{r' >= r} db_r'
    if (r < L) {
      const size_t idx = (r0 + r) * p.H + h;
      p.dbeta[idx] = cT + sm.dbeta[r];
      if (GATED) p.dg[idx] = dgv;
    }
  }
}

template <typename K>
static hipError_t launch_k(K kern, size_t smem, int grid, const BwdParams &p, hipStream_t stream) {
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), smem, stream, p);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t stream) {
  const bool gated = p.g != nullptr;
  hipError_t e = launch_k(gated ? scan_kernel<DK, true> : scan_kernel<DK, false>, sizeof(ScanSmem<DK>),
                          p.N * p.H * p.ntiles, p, stream);
  if (e != hipSuccess) return e;
  const int nchunks = p.chunk_seq ? p.total_chunks : p.N * p.NC;
  return launch_k(gated ? chunk_kernel<DK, true> : chunk_kernel<DK, false>, sizeof(ChunkSmem<DK>),
                  nchunks * p.H, p, stream);
}

size_t bwd_smem_bytes(int dtype, int DK) {
  if (dtype != 1) return 0;
  return DK == 64 ? sizeof(ChunkSmem<64>) : sizeof(ChunkSmem<128>);
}

hipError_t launch_bwd(const BwdParams &p, int dtype, int DK, hipStream_t stream) {
  if (dtype != 1) return hipErrorInvalidValue;  // bf16 only
  return DK == 64 ? launch_bwd_t<64>(p, stream) : launch_bwd_t<128>(p, stream);
}

}  // namespace dn
