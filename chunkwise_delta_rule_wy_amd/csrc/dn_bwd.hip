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
// 2. bwd_chunk_kernel (dn_bwd_chunk.hip): one workgroup per (chunk, head) with
//    every d_v column computes dq, dk, dv, dbeta and dg from the chunk's
//    inputs, the stored state h_c and the stored dh.
//
// States and state gradients are stored in bf16, transposed (S = h^T,
// [chunk][H][d_v][d_k]): each lane writes the bf16 fragment it feeds its own
// MFMAs with, and the chunk kernel loads them directly into LDS.
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

    // dh of this chunk's end state, for the chunk-parallel pass (dS = dh^T, bf16)
    {
      bf16 *dst = p.dstates + (((size_t)global_chunk(p, n_seq, c) * p.H + h) * p.DV + col) * DK + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        *reinterpret_cast<bf16x8 *>(dst + 32 * kb) = bfrag<bf16>(hacc[2 * kb], hacc[2 * kb + 1]);
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
  return launch_bwd_chunk(p, DK, stream);
}

hipError_t launch_bwd(const BwdParams &p, int dtype, int DK, hipStream_t stream) {
  if (dtype != 1) return hipErrorInvalidValue;  // bf16 only
  return DK == 64 ? launch_bwd_t<64>(p, stream) : launch_bwd_t<128>(p, stream);
}

}  // namespace dn
