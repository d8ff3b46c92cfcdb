// Fused chunkwise forward pass of the (gated) delta rule for gfx950: the
// generic-element kernel, used for fp32 inputs (d_k = 64).
//
// One workgroup (4 waves) owns one (sequence, head, 64-wide d_v tile) and walks
// that sequence's 64-token chunks in order, keeping its slice of the state
// h = S^T (d_k x 64, fp32) in registers the whole time.  Per chunk:
//
//   load     K, Q (64 x d_k) and the V tile (64 x 64) arrive by direct
//            global->LDS loads issued one chunk ahead into a second buffer;
//            b = cumsum(g), gamma = exp(b), and K^T is formed in LDS
//   phase A  A = strictLower(diag(beta) (K K^T) * Gamma),  P = (Q K^T) * Gamma
//            with Gamma_rj = exp(b_r - b_j) for j <= r (MFMA, 5 tiles a wave)
//   phase B  R = (I + A)^-1, T = R diag(beta): 16x16 diagonal blocks by fp32
//            forward substitution, off-diagonal blocks R_ij = -R_ii sum_m
//            A_im R_mj by small MFMAs; every wave computes what its block row
//            of T needs, overlapped with Y_K = K h and Y_Q = Q h
//   phase C  X = V - diag(gamma) Y_K,  V' = T X,
//            O = diag(gamma) Y_Q + P V',
//            h <- gamma_64 h + K^T diag(exp(b_64 - b)) V'
//
// This is the WY/UT form of a chunk ("Parallelizing Linear Transformers with
// the Delta Rule over Sequence Length": products of Householder-like
// transitions in WY form, page 3 abstract; the UT transform named in the Gated
// DeltaNet review thread, review 2), with the gate entering through
// cumulative decay ratios (page 1, answer W2).  Each wave owns 16 of the 64
// d_v columns for the whole state chain, so the chain needs no cross-wave
// exchange: only read-only operands (K, Q, K^T, T, P) are shared through LDS.
// Partial chunks are zero-padded rows (k = q = v = 0, beta = g = 0), which
// leave A, T, V', gamma_64 and the state unchanged.
#include "dn_internal.h"
#include "dn_prep.h"

namespace dn {

template <typename E, int DK>
struct FwdCfg {
  static constexpr int NBUF = sizeof(E) == 2 ? 2 : 1;  // fp32 tiles fit LDS only once
  static constexpr int KB = DK / 32;                   // 32-index blocks over d_k
  static constexpr int MTK = DK / 16;                  // state row tiles per wave
};

template <typename E, int DK>
struct FwdSmem {
  using C = FwdCfg<E, DK>;
  E K[C::NBUF][CH * DK];
  E Q[C::NBUF][CH * DK];
  E V[C::NBUF][CH * DVT];
  E KT[DK * CH];
  E T[CH * CH];
  E P[CH * CH];
  PrepScratch<E> ps;
  Gates G[2];
};

template <typename E, int DK, bool GATED, bool WRITE_O>
__global__ __launch_bounds__(NTHR, 1) void fwd_kernel(FwdParams p) {
  using C = FwdCfg<E, DK>;
  using SM = FwdSmem<E, DK>;
  using TV = Tile<E, DVT>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);

  int pair, tile;
  wg_coords(blockIdx.x, p.ntiles, p.xcd_map, pair, tile);
  if (pair >= p.N * p.H) return;
  const int n_seq = pair_seq(p.seq_order, pair / p.H), h = pair % p.H;
  const int dv0 = tile * DVT;
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  const int nch = (si.len + CH - 1) / CH;
  const E *gq = static_cast<const E *>(p.q);
  const E *gk = static_cast<const E *>(p.k);
  const E *gv = static_cast<const E *>(p.v);
  E *go = static_cast<E *>(p.o);

  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const int col = dv0 + 16 * w + n;  // this lane's d_v column
  const size_t row_base = (size_t)si.b * p.T + si.t0;  // global row of the sequence start

  constexpr unsigned OUT = WRITE_O ? (OUT_P | OUT_T) : OUT_T;
  PrepOut<E> po = {};
  po.P = sm.P;
  po.T = sm.T;
  prep_zero<E, OUT>(po);  // upper triangles of T and P stay zero

  // state slice: lane (n, g) holds rows prow(mt, 4g + i) of column `col`
  f32x4 hacc[C::MTK];
  const size_t st_base = ((size_t)n_seq * p.H + h) * DK * p.DV;
#pragma unroll
  for (int mt = 0; mt < C::MTK; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      hacc[mt][i] = p.h0 ? p.h0[st_base + (size_t)prow(mt, 4 * g + i) * p.DV + col] : 0.f;

  // scalar inputs of a chunk: wave 0 holds g, wave 1 holds beta of row `l`
  auto load_scalars = [&](int c) {
    const int L = min(CH, si.len - c * CH);
    float s = 0.f;
    if (l < L) {
      const size_t idx = (row_base + (size_t)c * CH + l) * p.H + h;
      if (GATED && w == 0) s = p.g[idx];
      if (w == 1) s = p.beta[idx];
    }
    return s;
  };
  auto issue_loads = [&](int c, int buf) {
    const int L = min(CH, si.len - c * CH);
    const size_t r0 = row_base + (size_t)c * CH;
    dma_tile<E, DK>(sm.K[buf], gk, r0, p.H, h, DK, 0, L);
    if (WRITE_O) dma_tile<E, DK>(sm.Q[buf], gq, r0, p.H, h, DK, 0, L);
    dma_tile<E, DVT>(sm.V[buf], gv, r0, p.H, h, p.DV, dv0, L);
  };

  float sc = 0.f;
  if (nch > 0) {
    issue_loads(0, 0);
    sc = load_scalars(0);
  }
  typename four<E>::type ov[4];  // output of the previous chunk, stored one iteration late
  int prevL = 0;
  size_t prev_r0 = 0;

  for (int c = 0; c < nch; ++c) {
    const int cur = C::NBUF == 2 ? (c & 1) : 0;
    const int L = min(CH, si.len - c * CH);
    const E *Kc = sm.K[cur];
    const E *Qc = sm.Q[cur];
    const E *Vc = sm.V[cur];
    Gates &G = sm.G[c & 1];
    wait_vmem();
    if (WRITE_O && c > 0) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = prow(mt, 4 * g + i);
          if (r < prevL) go[((prev_r0 + r) * p.H + h) * p.DV + col] = ov[mt][i];
        }
    }
    if (L < CH) {
      zero_rows<E, DK>(sm.K[cur], L);
      if (WRITE_O) zero_rows<E, DK>(sm.Q[cur], L);
      zero_rows<E, DVT>(sm.V[cur], L);
    }
    write_gates(G, w == 0 ? sc : 0.f, w == 1 ? sc : 0.f);
    __syncthreads();  // chunk c visible; every wave is done with chunk c-1

    if (c + 1 < nch) {
      if (C::NBUF == 2) issue_loads(c + 1, cur ^ 1);
      sc = load_scalars(c + 1);
    }
    transpose_tile<E, DK>(sm.KT, Kc);
    prep_a<E, DK, OUT, GATED>(sm.ps, po, Kc, Qc, G);
    __syncthreads();

    // phase B: UT inverse overlapped with Y_K = K h, Y_Q = Q h
    F32<E> hb[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) hb[kb] = bfrag<E>(hacc[2 * kb], hacc[2 * kb + 1]);
    f32x4 yk[4], yq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      F32<E> af[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) af[kb] = frag<E, DK>(Kc, prow(mt, n), kb);
      yk[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) yk[mt] = mma32(yk[mt], af[kb], hb[kb]);
    }
    prep_inv_diag<E, OUT>(sm.ps, po, G);
    if constexpr (WRITE_O) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        F32<E> af[C::KB];
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) af[kb] = frag<E, DK>(Qc, prow(mt, n), kb);
        yq[mt] = zero4();
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) yq[mt] = mma32(yq[mt], af[kb], hb[kb]);
      }
    }
    wave_lds_fence();
    prep_inv_offdiag<E, OUT>(sm.ps, po, G);
    mfma_settle();  // Y_K, Y_Q and the inverse are read after the barrier
    __syncthreads();

    // phase C
    f32x4 x[4], gm[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      gm[mt] = *reinterpret_cast<const f32x4 *>(&G.gam[prow(mt, 4 * g)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = prow(mt, 4 * g + i);
        x[mt][i] = to_f<E>(Vc[TV::off(r, 16 * w + n)]) - gm[mt][i] * yk[mt][i];
      }
    }
    F32<E> xb[2] = {bfrag<E>(x[0], x[1]), bfrag<E>(x[2], x[3])};
    f32x4 vp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const F32<E> a0 = frag<E, CH>(sm.T, prow(mt, n), 0);
      const F32<E> a1 = frag<E, CH>(sm.T, prow(mt, n), 1);
      vp[mt] = mma32(mma32(zero4(), a0, xb[0]), a1, xb[1]);
    }
    F32<E> vb[2] = {bfrag<E>(vp[0], vp[1]), bfrag<E>(vp[2], vp[3])};
    f32x4 wvp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const f32x4 wl = *reinterpret_cast<const f32x4 *>(&G.wl[prow(mt, 4 * g)]);
      wvp[mt] = wl * vp[mt];
    }
    F32<E> wb[2] = {bfrag<E>(wvp[0], wvp[1]), bfrag<E>(wvp[2], wvp[3])};
    if (WRITE_O) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const F32<E> a0 = frag<E, CH>(sm.P, prow(mt, n), 0);
        const F32<E> a1 = frag<E, CH>(sm.P, prow(mt, n), 1);
        f32x4 acc = gm[mt] * yq[mt];
        acc = mma32(mma32(acc, a0, vb[0]), a1, vb[1]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[mt][i] = to_e<E>(acc[i]);
      }
      prevL = L;
      prev_r0 = row_base + (size_t)c * CH;
    }
    const float glast = G.gam[CH - 1];
#pragma unroll
    for (int mt = 0; mt < C::MTK; ++mt) {
      const F32<E> a0 = frag<E, CH>(sm.KT, prow(mt, n), 0);
      const F32<E> a1 = frag<E, CH>(sm.KT, prow(mt, n), 1);
      hacc[mt] = mma32(mma32(hacc[mt] * glast, a0, wb[0]), a1, wb[1]);
    }
    mfma_settle();  // the state is read again across the loop edge
    if (C::NBUF == 1 && c + 1 < nch) {
      __syncthreads();  // single buffer: every wave is done reading chunk c
      issue_loads(c + 1, 0);
    }
  }

  if (WRITE_O && nch > 0) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = prow(mt, 4 * g + i);
        if (r < prevL) go[((prev_r0 + r) * p.H + h) * p.DV + col] = ov[mt][i];
      }
  }
  if (p.hT) {
#pragma unroll
    for (int mt = 0; mt < C::MTK; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.hT[st_base + (size_t)prow(mt, 4 * g + i) * p.DV + col] = hacc[mt][i];
  }
}

template <typename E, int DK, bool WRITE_O>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  const size_t smem = sizeof(FwdSmem<E, DK>);
  auto kern = p.g ? fwd_kernel<E, DK, true, WRITE_O> : fwd_kernel<E, DK, false, WRITE_O>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.N * p.H * p.ntiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), smem, stream, p);
  return hipGetLastError();
}

size_t fwd_ref_smem_bytes(int dtype, int DK) {
  return (dtype == 0 && DK == 64) ? sizeof(FwdSmem<float, 64>) : 0;  // fp32 needs d_k == 64 to fit LDS
}

// fp32 inputs, d_k = 64 (the state-storing variant is bf16 only)
hipError_t launch_fwd_ref(const FwdParams &p, int dtype, int DK, bool store_states, bool write_o,
                          hipStream_t stream) {
  if (dtype != 0 || DK != 64 || store_states) return hipErrorInvalidValue;
  return write_o ? launch_fwd_t<float, 64, true>(p, stream) : launch_fwd_t<float, 64, false>(p, stream);
}

}  // namespace dn
