// Fused chunkwise forward pass of the (gated) delta rule for gfx950.
//
// One workgroup (4 waves) owns one (sequence, head, 64-wide d_v tile) and walks
// that sequence's 64-token chunks in order, keeping its slice of the state
// h = S^T (d_k x 64, fp32) in registers the whole time.  Per chunk:
//
//   load     K, Q (64 x d_k), V tile (64 x 64), beta, g -> LDS (prefetched
//            into registers one chunk ahead); b = cumsum(g), gamma = exp(b)
//   phase A  A = strictLower(diag(beta) (K K^T) * Gamma),  P = (Q K^T) * Gamma
//            (Gamma_rj = exp(b_r - b_j), j <= r), MFMA, 5 tiles per wave
//   phase B  wave 0: R = (I + A)^-1 -- 16x16 diagonal blocks by forward
//            substitution in fp32 registers, off-diagonal blocks by small MFMA
//            products R_ij = -R_ii sum_m A_im R_mj -- and T = R diag(beta);
//            meanwhile every wave forms Y_K = K h and Y_Q = Q h for its columns
//   phase C  X = V - diag(gamma) Y_K,  V' = T X,
//            O = diag(gamma) Y_Q + P V',
//            h <- gamma_64 h + K^T diag(exp(b_64 - b)) V'
//
// This is the WY/UT form of the chunk (products of Householder-like
// transitions, "Parallelizing Linear Transformers with the Delta Rule over
// Sequence Length", page 3 abstract; the UT transform is named in the Gated
// DeltaNet review thread, review 2), with the gate entering through
// cumulative decay ratios (page 1, answer W2).  Each wave owns 16 of the 64
// d_v columns for the whole state chain, so the chain needs no cross-wave
// exchange: only read-only operands (K, Q, K^T, T, P) are shared through LDS.
//
// Partial chunks are zero-padded rows (k = q = v = 0, beta = g = 0), which
// leave A, T, V', gamma_64 and the state unchanged.
#include "dn_internal.h"

namespace dn {

template <typename E, int DK>
struct FwdSmem {
  static constexpr int PAD = 16 / sizeof(E);  // 16-byte row skew
  static constexpr int LDK = DK + PAD;        // K, Q rows
  static constexpr int LD64 = 64 + PAD;       // 64-wide E matrices
  static constexpr int LDA = 64 + 4;          // fp32 A
  static constexpr int LDR = 16 + PAD;        // R diagonal blocks
  E K[CH * LDK];
  E Q[CH * LDK];
  E KT[DK * LD64];
  E V[CH * LD64];
  E T[CH * LD64];
  E P[CH * LD64];
  E Rd[4 * 16 * LDR];
  float A[CH * LDA];
  float b[CH];
  float gam[CH];
  float beta[CH];
};

template <typename E, int DK>
struct Prefetch {
  static constexpr int EPU = 16 / sizeof(E);         // elements per 16-byte unit
  static constexpr int UK = DK / EPU;                // units per K row
  static constexpr int NUK = CH * UK / NTHR;         // K units per thread
  static constexpr int UV = DVT / EPU;               // units per V row
  static constexpr int NUV = CH * UV / NTHR;         // V units per thread
  u128 k[NUK], q[NUK], v[NUV];
  float s;  // wave 0: g of row lane; wave 1: beta of row lane
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

// (seq, head, tile) of this workgroup; siblings of one (seq, head) land on one
// XCD (workgroups are dealt to the 8 XCDs round-robin) so that their shared
// K/Q reads hit the same L2.
__device__ __forceinline__ void wg_coords(int x, int pairs, int ntiles, int xcd_map, int &pair,
                                          int &tile) {
  if (xcd_map) {
    int xcd = x & 7, slot = x >> 3;
    pair = (slot / ntiles) * 8 + xcd;
    tile = slot % ntiles;
  } else {
    pair = x / ntiles;
    tile = x % ntiles;
  }
}

template <typename E, int DK>
__device__ __forceinline__ void prefetch_chunk(Prefetch<E, DK> &pf, const FwdParams &p, const SeqInfo &si,
                                               int h, int dv0, int c, int L) {
  using PF = Prefetch<E, DK>;
  const int t = threadIdx.x;
  const E *q = static_cast<const E *>(p.q);
  const E *k = static_cast<const E *>(p.k);
  const E *v = static_cast<const E *>(p.v);
  const size_t tok0 = (size_t)si.b * p.T + si.t0 + (size_t)c * CH;
#pragma unroll
  for (int i = 0; i < PF::NUK; ++i) {
    int s = t + NTHR * i, row = s / PF::UK, cu = s % PF::UK;
    if (row < L) {
      size_t off = ((tok0 + row) * p.H + h) * DK + cu * PF::EPU;
      pf.k[i] = ldg128(k + off);
      pf.q[i] = ldg128(q + off);
    } else {
      pf.k[i] = zero128();
      pf.q[i] = zero128();
    }
  }
#pragma unroll
  for (int i = 0; i < PF::NUV; ++i) {
    int s = t + NTHR * i, row = s / PF::UV, cu = s % PF::UV;
    if (row < L)
      pf.v[i] = ldg128(v + ((tok0 + row) * p.H + h) * p.DV + dv0 + cu * PF::EPU);
    else
      pf.v[i] = zero128();
  }
  const int w = t >> 6, l = t & 63;
  pf.s = 0.f;
  if (l < L) {
    size_t si_ = (tok0 + l) * p.H + h;
    if (w == 0 && p.g) pf.s = p.g[si_];
    if (w == 1) pf.s = p.beta[si_];
  }
}

template <typename E, int DK>
__device__ __forceinline__ void store_chunk(FwdSmem<E, DK> &sm, const Prefetch<E, DK> &pf) {
  using PF = Prefetch<E, DK>;
  using SM = FwdSmem<E, DK>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PF::NUK; ++i) {
    int s = t + NTHR * i, row = s / PF::UK, cu = s % PF::UK;
    *reinterpret_cast<u128 *>(&sm.K[row * SM::LDK + cu * PF::EPU]) = pf.k[i];
    *reinterpret_cast<u128 *>(&sm.Q[row * SM::LDK + cu * PF::EPU]) = pf.q[i];
    const E *ke = reinterpret_cast<const E *>(&pf.k[i]);
#pragma unroll
    for (int e = 0; e < PF::EPU; ++e) sm.KT[(cu * PF::EPU + e) * SM::LD64 + row] = ke[e];
  }
#pragma unroll
  for (int i = 0; i < PF::NUV; ++i) {
    int s = t + NTHR * i, row = s / PF::UV, cu = s % PF::UV;
    *reinterpret_cast<u128 *>(&sm.V[row * SM::LD64 + cu * PF::EPU]) = pf.v[i];
  }
  const int w = t >> 6, l = t & 63;
  if (w == 0) {
    float bsum = wave_incl_scan(pf.s);
    sm.b[l] = bsum;
    sm.gam[l] = __expf(bsum);
  } else if (w == 1) {
    sm.beta[l] = pf.s;
  }
}

// Phase A: lower tiles of K K^T (waves 0, 1) and Q K^T (waves 2, 3), scaled by
// the gate ratios; A (strict, times beta_r) in fp32, P (inclusive) in E.
template <typename E, int DK>
__device__ __forceinline__ void phase_a(FwdSmem<E, DK> &sm, bool gated) {
  using SM = FwdSmem<E, DK>;
  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const E *src = (w < 2) ? sm.K : sm.Q;
  const int rb0 = (w & 1) ? 1 : 0, rb1 = (w & 1) ? 2 : 3;
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int ti = which ? rb1 : rb0;
    F32<E> af[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) af[kb] = afrag<E>(src, SM::LDK, 16 * ti + n, kb);
    for (int tj = 0; tj <= ti; ++tj) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        acc = mma32(acc, af[kb], afrag<E>(sm.K, SM::LDK, 16 * tj + n, kb));
      const int j = 16 * tj + n;
      const float bj = sm.b[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * ti + 4 * g + e;
        const float gr = (gated && j <= r) ? __expf(sm.b[r] - bj) : 1.f;
        if (w < 2) {
          sm.A[r * SM::LDA + j] = (j < r) ? sm.beta[r] * gr * acc[e] : 0.f;
        } else {
          sm.P[r * SM::LD64 + j] = to_e<E>((j <= r) ? gr * acc[e] : 0.f);
        }
      }
    }
  }
}

// Phase B (wave 0 only): T = (I + A)^-1 diag(beta) into sm.T.
template <typename E, int DK>
__device__ __forceinline__ void invert_wave0(FwdSmem<E, DK> &sm) {
  using SM = FwdSmem<E, DK>;
  const int l = lane_id(), bi = l >> 4, c = l & 15, g = l >> 4, n = l & 15;
  // diagonal blocks: lane (bi, c) computes column c of (I + A_ii)^-1
  float Rc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    float acc = (r == c) ? 1.f : 0.f;
    const float *arow = &sm.A[(16 * bi + r) * SM::LDA + 16 * bi];
#pragma unroll
    for (int j = 0; j < r; ++j) acc -= arow[j] * Rc[j];
    Rc[r] = acc;
  }
  const float bc = sm.beta[16 * bi + c];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    sm.Rd[(bi * 16 + r) * SM::LDR + c] = to_e<E>(Rc[r]);
    sm.T[(16 * bi + r) * SM::LD64 + 16 * bi + c] = to_e<E>(Rc[r] * bc);
  }
  wave_lds_fence();
  // B fragment of diagonal block R_jj (column n, rows 4g..4g+3)
  auto bdiag = [&](int j) {
    F16<E> f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = sm.Rd[(j * 16 + 4 * g + i) * SM::LDR + n];
    return f;
  };
  auto ablk = [&](int i, int m) { return afrag16_f<E>(sm.A, SM::LDA, 16 * i + n, 16 * m); };
  auto adiag = [&](int i) { return afrag16<E>(&sm.Rd[i * 16 * SM::LDR], SM::LDR, n, 0); };
  f32x4 y;
  y = mma16(zero4(), ablk(1, 0), bdiag(0));
  const f32x4 R10 = -mma16(zero4(), adiag(1), bfrag16<E>(y));
  y = mma16(zero4(), ablk(2, 1), bdiag(1));
  const f32x4 R21 = -mma16(zero4(), adiag(2), bfrag16<E>(y));
  y = mma16(zero4(), ablk(3, 2), bdiag(2));
  const f32x4 R32 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
  y = mma16(zero4(), ablk(2, 0), bdiag(0));
  y = mma16(y, ablk(2, 1), bfrag16<E>(R10));
  const f32x4 R20 = -mma16(zero4(), adiag(2), bfrag16<E>(y));
  y = mma16(zero4(), ablk(3, 1), bdiag(1));
  y = mma16(y, ablk(3, 2), bfrag16<E>(R21));
  const f32x4 R31 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
  y = mma16(zero4(), ablk(3, 0), bdiag(0));
  y = mma16(y, ablk(3, 1), bfrag16<E>(R10));
  y = mma16(y, ablk(3, 2), bfrag16<E>(R20));
  const f32x4 R30 = -mma16(zero4(), adiag(3), bfrag16<E>(y));
  auto put = [&](int i, int j, const f32x4 &R) {
    const float bj = sm.beta[16 * j + n];
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.T[(16 * i + 4 * g + e) * SM::LD64 + 16 * j + n] = to_e<E>(R[e] * bj);
  };
  put(1, 0, R10);
  put(2, 1, R21);
  put(3, 2, R32);
  put(2, 0, R20);
  put(3, 1, R31);
  put(3, 0, R30);
}

template <typename E, int DK, bool STORE_STATES, bool WRITE_O>
__global__ __launch_bounds__(NTHR, 1) void fwd_kernel(FwdParams p) {
  using SM = FwdSmem<E, DK>;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM &sm = *reinterpret_cast<SM *>(smem_raw);
  constexpr int MT = DK / 16;  // state row tiles per wave

  int pair, tile;
  wg_coords(blockIdx.x, p.N * p.H, p.ntiles, p.xcd_map, pair, tile);
  if (pair >= p.N * p.H) return;
  const int n_seq = pair / p.H, h = pair % p.H;
  const int dv0 = tile * DVT;
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  const int nch = (si.len + CH - 1) / CH;
  const bool gated = p.g != nullptr;

  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const int col = dv0 + 16 * w + n;  // this lane's d_v column

  // zero T and P once: their upper triangles are never written again
  for (int i = threadIdx.x; i < CH * SM::LD64; i += NTHR) {
    sm.T[i] = to_e<E>(0.f);
    sm.P[i] = to_e<E>(0.f);
  }

  // state slice: rows 16*mt + 4g + e, column `col`
  f32x4 hacc[MT];
  const size_t st_base = ((size_t)n_seq * p.H + h) * DK * p.DV;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      hacc[mt][e] = p.h0 ? p.h0[st_base + (size_t)(16 * mt + 4 * g + e) * p.DV + col] : 0.f;
  }

  Prefetch<E, DK> pf;
  if (nch > 0) prefetch_chunk<E, DK>(pf, p, si, h, dv0, 0, min(CH, si.len));

  for (int c = 0; c < nch; ++c) {
    const int L = min(CH, si.len - c * CH);
    __syncthreads();
    store_chunk<E, DK>(sm, pf);
    __syncthreads();
    if (c + 1 < nch) prefetch_chunk<E, DK>(pf, p, si, h, dv0, c + 1, min(CH, si.len - (c + 1) * CH));
    if (STORE_STATES) {
      const int cg = p.chunk_base ? p.chunk_base[n_seq] + c : n_seq * p.NC + c;
      float *dst = p.states + ((size_t)cg * p.H + h) * DK * p.DV;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(16 * mt + 4 * g + e) * p.DV + col] = hacc[mt][e];
    }

    phase_a<E, DK>(sm, gated);
    __syncthreads();

    if (w == 0) invert_wave0<E, DK>(sm);
    // Y_K = K h, Y_Q = Q h for this wave's 16 columns
    F32<E> hb[DK / 32];
#pragma unroll
    for (int kb = 0; kb < DK / 32; ++kb) hb[kb] = bfrag<E>(hacc[2 * kb], hacc[2 * kb + 1]);
    f32x4 yk[4], yq[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      yk[mt] = zero4();
      yq[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        yk[mt] = mma32(yk[mt], afrag<E>(sm.K, SM::LDK, 16 * mt + n, kb), hb[kb]);
        if (WRITE_O) yq[mt] = mma32(yq[mt], afrag<E>(sm.Q, SM::LDK, 16 * mt + n, kb), hb[kb]);
      }
    }
    __syncthreads();

    // X = V - diag(gamma) Y_K
    f32x4 x[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * g + e;
        x[mt][e] = to_f<E>(sm.V[r * SM::LD64 + 16 * w + n]) - sm.gam[r] * yk[mt][e];
      }
    F32<E> xb[2];
    xb[0] = bfrag<E>(x[0], x[1]);
    xb[1] = bfrag<E>(x[2], x[3]);
    // V' = T X
    f32x4 vp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      vp[mt] = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) vp[mt] = mma32(vp[mt], afrag<E>(sm.T, SM::LD64, 16 * mt + n, kb), xb[kb]);
    }
    F32<E> vb[2];
    vb[0] = bfrag<E>(vp[0], vp[1]);
    vb[1] = bfrag<E>(vp[2], vp[3]);
    if (WRITE_O) {
      // O = diag(gamma) Y_Q + P V'
      E *o = static_cast<E *>(p.o);
      const size_t tok0 = (size_t)si.b * p.T + si.t0 + (size_t)c * CH;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = sm.gam[16 * mt + 4 * g + e] * yq[mt][e];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc = mma32(acc, afrag<E>(sm.P, SM::LD64, 16 * mt + n, kb), vb[kb]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * mt + 4 * g + e;
          if (r < L) o[((tok0 + r) * p.H + h) * p.DV + col] = to_e<E>(acc[e]);
        }
      }
    }
    // h <- gamma_64 h + K^T diag(exp(b_64 - b)) V'
    const float blast = sm.b[CH - 1];
    const float glast = sm.gam[CH - 1];
    f32x4 wv[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * mt + 4 * g + e;
        wv[mt][e] = (gated ? __expf(blast - sm.b[r]) : 1.f) * vp[mt][e];
      }
    F32<E> wb[2];
    wb[0] = bfrag<E>(wv[0], wv[1]);
    wb[1] = bfrag<E>(wv[2], wv[3]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = hacc[mt] * glast;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) acc = mma32(acc, afrag<E>(sm.KT, SM::LD64, 16 * mt + n, kb), wb[kb]);
      hacc[mt] = acc;
    }
  }

  if (p.hT) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) p.hT[st_base + (size_t)(16 * mt + 4 * g + e) * p.DV + col] = hacc[mt][e];
  }
}

template <typename E, int DK, bool STORE_STATES, bool WRITE_O>
static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
  const size_t smem = sizeof(FwdSmem<E, DK>);
  auto kern = fwd_kernel<E, DK, STORE_STATES, WRITE_O>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.N * p.H * p.ntiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), smem, stream, p);
  return hipGetLastError();
}

size_t fwd_smem_bytes(int dtype, int DK) {
  if (dtype == 1) return DK == 64 ? sizeof(FwdSmem<bf16, 64>) : sizeof(FwdSmem<bf16, 128>);
  return DK == 64 ? sizeof(FwdSmem<float, 64>) : 0;  // fp32 needs d_k == 64 to fit LDS
}

hipError_t launch_fwd(const FwdParams &p, int dtype, int DK, bool store_states, bool write_o,
                      hipStream_t stream) {
#define DN_FWD_CASE(E, D)                                                       \
  if (store_states)                                                             \
    return write_o ? launch_fwd_t<E, D, true, true>(p, stream)                  \
                   : launch_fwd_t<E, D, true, false>(p, stream);                \
  return write_o ? launch_fwd_t<E, D, false, true>(p, stream)                   \
                 : launch_fwd_t<E, D, false, false>(p, stream);
  if (dtype == 1) {
    if (DK == 64) { DN_FWD_CASE(bf16, 64) }
    DN_FWD_CASE(bf16, 128)
  }
  if (DK == 64) { DN_FWD_CASE(float, 64) }
  return hipErrorInvalidValue;
#undef DN_FWD_CASE
}

}  // namespace dn
