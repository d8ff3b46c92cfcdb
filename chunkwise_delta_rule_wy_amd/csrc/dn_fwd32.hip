// Fused chunkwise forward pass with 32-token chunks (bf16 inputs, d_k 64 or
// 128): the chunk-size variant of the 64-token kernel in dn_fwd.hip, for the
// chunk-size trade-off the DeltaNet rebuttal discusses (page 1, answers Q1 and
// Q2: a smaller chunk costs less WY/UT work per chunk and more chunk steps).
//
// The organisation is that of the 64-token kernel: one workgroup per
// (sequence, head, 64-wide d_v tile), four chain waves (16 state columns each,
// state h = S^T in registers, scaled by a per-chunk scalar) and four prep
// waves one chunk ahead, one barrier per step.  Its LDS footprint is half the
// 64-token kernel's, so the direct global->LDS loads run three chunks ahead
// (a four-slot ring) instead of two.  A chunk has two 16-token blocks, so
//
//   prep   waves 0, 1  diagonal block v of M = strictLower((K K^T) * Gamma)
//                      and T_vv = (I + diag(beta) M_vv)^-1 diag(beta) by fp32
//                      forward substitution (four lanes per column)
//          wave 2      -M_10 and P_10
//          wave 3      P_00 and P_11
//          (P = (Q K^T) * Gamma, Gamma_rj = exp(b_r - b_j) for j <= r)
//   chain  Y_K = K h, Y_Q = Q h, X = V - diag(gamma) Y_K,
//          V'_0 = T_00 X_0,  V'_1 = T_11 (X_1 - M_10 V'_0),
//          O = diag(gamma) Y_Q + P V',  h <- gamma_31 h + K^T diag(w) V'
//
// with b = cumsum g inside the chunk, gamma = exp b and w_r = exp(b_31 - b_r).
// Rows past the end of a sequence are zero (k = q = v = 0, beta = g = 0),
// which leaves V' and the state unchanged.  The LDS layouts, swizzles and
// fragment conventions are the 64-token kernel's, restricted to 32 rows.
#include "dn_wy.h"

namespace dn {
namespace {

using namespace wy;

constexpr int C32 = 32;
constexpr int F32_THREADS = 512;  // four chain waves, four prep waves
constexpr int AHEAD = 3;          // chunks the loads run ahead of the chain
constexpr int NBUF32 = AHEAD + 1; // ring slots

template <int DK>
struct Lay32 {
  static constexpr int RB = 2 * DK;
  static constexpr int UNITS = DK / 8;
  static constexpr int KB = DK / 32;
  static constexpr int MT = DK / 16;
  static constexpr int KQ = C32 * RB;         // bytes of a K or Q tile
  static constexpr int VT = C32 * DVT * 2;    // bytes of a V tile
  static constexpr int DMA_KQ = KQ / 4096;    // direct loads per prep wave for a K or Q tile
  static constexpr int DMA_V = VT / 4096;
  static constexpr int S_K = 0, S_Q = KQ, S_V = 2 * KQ, S_G = 2 * KQ + VT, S_BETA = S_G + 4 * C32;
  static constexpr int SLOT = S_BETA + 4 * C32;
  // prep results of one chunk: P (rows 0..31, 64-byte rows), -M_10, T_00^T, T_11^T, gate table
  static constexpr int O_P = 0, O_M = 2048, O_TT = O_M + 512, O_CG = O_TT + 1024;
  static constexpr int OUTB = O_CG + CG_BYTES;
  static constexpr int OUT_OFF = NBUF32 * SLOT;
  static constexpr int PRIV_OFF = OUT_OFF + 2 * OUTB;
  static constexpr int TOTAL = PRIV_OFF + 4 * PRIV_BYTES;
  static_assert(DMA_KQ >= 1 && DMA_V == 1, "direct-load split");
  static_assert(SLOT % 256 == 0 && OUTB % 256 == 0, "tile alignment");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

// ---------------------------------------------------------------- prep

// Preparation of one 32-token chunk by prep wave PW (roles in the header).
// kbase, qbase: K and Q tiles; gaddr, baddr: g and beta of the chunk's rows;
// rows >= L are padding.  Wave 0 also writes the chain's gate table and
// carries the state scale in `scale`.
template <int DK, bool GATED, int PW>
__device__ __forceinline__ void prep32(const Bases &lb, uint32_t kbase, uint32_t qbase, uint32_t gaddr,
                                       uint32_t baddr, uint32_t ob, uint32_t priv, int L, float &scale) {
  using LY = Lay32<DK>;
  constexpr int KB = LY::KB;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const uint32_t pg = priv + AT_BYTES;

  if constexpr (GATED) {
    // b over the chunk's rows (lanes past the chunk carry b_31 on)
    const float gv = (l < L) ? ld<float>(gaddr + 4 * l) : 0.f;
    const float b = wave_incl_scan(gv) * LOG2E;
    const float b0 = lane_val(b, 0), b16 = lane_val(b, 16);
    const float bst = l < 16 ? b0 : b16;
    st<float>(pg + PG_BL + 4 * l, b);
    st<float>(pg + PG_RHO + 4 * l, fexp2(b - bst));
    st<float>(pg + PG_KAP + 4 * l, fexp2(b16 - b));
    if constexpr (PW == 0) {
      const float bl = lane_val(b, C32 - 1);
      const float sc = scale;
      const float t = sc * fexp2(bl);
      const bool resc = !(t >= SCALE_MIN);
      const float inv = resc ? 1.f : 1.f / t;
      st<float>(ob + LY::O_CG + CG_GS + 4 * l, fexp2(b) * sc);
      st<float>(ob + LY::O_CG + CG_WS + 4 * l, fexp2(bl - b) * inv);
      if (l == 0) {
        st<float>(ob + LY::O_CG + CG_HSCALE, resc ? t : 1.f);
        st<float>(ob + LY::O_CG + CG_SC, sc);
        st<float>(ob + LY::O_CG + CG_SNEXT, resc ? 1.f : t);
      }
      scale = resc ? 1.f : t;
    }
    wave_lds_fence();
  }

  bf16x8 kf[2][KB];  // K rows 16t + n, d_k block kb
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < 2; ++t) kf[t][kb] = ld<bf16x8>(kbase + (lb.frag ^ (64 * kb)) + 16 * t * LY::RB);

  if constexpr (PW < 2) {
    // diagonal block PW of A = strictLower(diag(beta) (K K^T) * Gamma), fp32,
    // transposed into the scratch: lane (n, g) holds k_r . k_j with
    // r = 16PW + 4g + e, j = 16PW + n
    {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[PW][kb], kf[PW][kb]);
      const f32x4 be = ld<f32x4>(baddr + 4 * (16 * PW + 4 * g));
      f32x4 mv, a;
      if constexpr (GATED) {
        const f32x4 blr = ld<f32x4>(pg + PG_BL + 4 * (16 * PW + 4 * g));
        const float blj = ld<float>(pg + PG_BL + 4 * (16 * PW + n));
#pragma unroll
        for (int e = 0; e < 4; ++e) mv[e] = acc[e] * fexp2(blr[e] - blj);
      } else {
        mv = acc;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = 4 * g + e > n && 16 * PW + 4 * g + e < L;
        a[e] = keep ? be[e] * mv[e] : 0.f;
      }
      st<f32x4>(priv + 96 * n + 16 * g, a);
    }
    // T_vv = (I + A_vv)^-1 diag(beta): lane (c, qr) = (l / 4, l % 4) holds rows
    // 4qr .. 4qr + 3 of column c; column j of A_vv is read from the scratch and
    // x_j is broadcast from its owner lane of the quad
    wave_lds_fence();
    {
      const int c = l >> 2, qr = l & 3;
      float x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = (4 * qr + k == c) ? 1.f : 0.f;
      f32x4 acol[15];
#pragma unroll
      for (int j = 0; j < 15; ++j) acol[j] = ld<f32x4>(priv + 96 * j + 16 * qr);
#pragma unroll
      for (int j = 0; j < 15; ++j) {
        const f32x4 a = acol[j];
        const float own = x[j & 3];
        const float xj = (j >> 2) == 0 ? quad_bcast<0>(own)
                       : (j >> 2) == 1 ? quad_bcast<1>(own)
                       : (j >> 2) == 2 ? quad_bcast<2>(own)
                                       : quad_bcast<3>(own);
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] -= a[k] * xj;
      }
      const float bc = (16 * PW + c < L) ? ld<float>(baddr + 4 * (16 * PW + c)) : 0.f;
      bf16x4 tv;
#pragma unroll
      for (int k = 0; k < 4; ++k) tv[k] = (__bf16)(x[k] * bc);
      st<bf16x4>(ob + LY::O_TT + 512 * PW + blk_quad(l), tv);
    }
  } else {
    // P block (TI, TJ): lane (n, g) holds q_r . k_j with r = 16TI + n,
    // j = 16TJ + 4g + e, stored into P
    auto ptile = [&](auto ti_c, auto tj_c, const bf16x8(&qf)[KB]) {
      constexpr int TI = decltype(ti_c)::value, TJ = decltype(tj_c)::value;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[TJ][kb], qf[kb]);
      f32x4 v;
      if constexpr (TI == TJ) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = n, j = 4 * g + e;
          float gam = 1.f;
          if constexpr (GATED)
            gam = fexp2(ld<float>(pg + PG_BL + 4 * (16 * TI + r)) - ld<float>(pg + PG_BL + 4 * (16 * TJ + j)));
          v[e] = (j <= r) ? acc[e] * gam : 0.f;
        }
      } else if constexpr (GATED) {
        const float rho = ld<float>(pg + PG_RHO + 4 * (16 * TI + n));
        const f32x4 kap = ld<f32x4>(pg + PG_KAP + 4 * (16 * TJ + 4 * g));
        v = acc * kap * rho;
      } else {
        v = acc;
      }
      st<bf16x4>(ob + LY::O_P + p_write<TI, TJ>(lb), cvt4(v));
    };
    auto qfrag = [&](bf16x8(&qf)[KB], int ti) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) qf[kb] = ld<bf16x8>(qbase + (lb.frag ^ (64 * kb)) + 16 * ti * LY::RB);
    };
    bf16x8 qa[KB];
    if constexpr (PW == 2) {
      // -M_10: lane (n, g) holds k_r . k_j with r = 16 + n, j = 4g + e
      {
        f32x4 acc = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[0][kb], kf[1][kb]);
        f32x4 v;
        if constexpr (GATED) {
          const float rho = ld<float>(pg + PG_RHO + 4 * (16 + n));
          const f32x4 kap = ld<f32x4>(pg + PG_KAP + 4 * (4 * g));
          v = acc * kap * (-rho);
        } else {
          v = -acc;
        }
        st<bf16x4>(ob + LY::O_M + lb.m, cvt4(v));
      }
      qfrag(qa, 1);
      ptile(I1{}, I0{}, qa);
    } else {
      bf16x8 qb[KB];
      qfrag(qa, 0);
      qfrag(qb, 1);
      ptile(I0{}, I0{}, qa);
      ptile(I1{}, I1{}, qb);
    }
  }
  mfma_settle();
}

// ---------------------------------------------------------------- chain

template <int DK, bool GATED, bool STORE_STATES, bool WRITE_O>
__device__ __forceinline__ void chain32(const FwdParams &p, const Bases &lb, f32x4 (&hs)[DK / 16], uint32_t slot,
                                        uint32_t ob, int L, size_t row0, int h, int col, bf16 *states_dst) {
  using LY = Lay32<DK>;
  constexpr int KB = LY::KB, MT = LY::MT;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int H = p.H, DV = p.DV;

  bf16x8 hb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) hb[kb] = bfrag<bf16>(hs[2 * kb], hs[2 * kb + 1]);

  // Y_K = K h~ (lane (n, g): row 16t + 4g + e, column 16w + n); Y_Q^T = h~^T Q^T
  f32x4 yk[2], yq[2];
  {
    bf16x8 kf[2][KB], qf[2][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t a = (lb.frag ^ (64 * kb)) + slot;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        kf[t][kb] = ld<bf16x8>(a + LY::S_K + 16 * t * LY::RB);
        if constexpr (WRITE_O) qf[t][kb] = ld<bf16x8>(a + LY::S_Q + 16 * t * LY::RB);
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      yk[t] = zero4();
      yq[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        yk[t] = mma32(yk[t], kf[t][kb], hb[kb]);
        if constexpr (WRITE_O) yq[t] = mma32(yq[t], hb[kb], qf[t][kb]);
      }
    }
  }
  // X = V - diag(gamma s_c) Y_K
  f32x4 x[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const bf16x4 vr = ld_tr(slot + LY::S_V + 16 * t * 128 + lb.vtr);
    const f32x4 gm = GATED ? ld<f32x4>(ob + LY::O_CG + CG_GS + 4 * (16 * t + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) x[t][e] = bf2f(vr[e]) - gm[e] * yk[t][e];
  }
  // V'_0 = T_00 X_0, V'_1 = T_11 (X_1 - M_10 V'_0)
  f32x4 vp[2];
  bf16x4 vb[2];
  vp[0] = mma16(zero4(), ld_tr(ob + LY::O_TT + lb.btr), cvt4(x[0]));
  vb[0] = cvt4(vp[0]);
  {
    const f32x4 acc = mma16(x[1], ld<bf16x4>(ob + LY::O_M + lb.m), vb[0]);
    vp[1] = mma16(zero4(), ld_tr(ob + LY::O_TT + 512 + lb.btr), cvt4(acc));
    vb[1] = cvt4(vp[1]);
  }
  // O^T = diag(gamma s_c) Y_Q^T + V'^T P^T: lane (n, g) holds O[16nt + n][16w + 4g + e]
  // the output tiles are stored after the state update (as in the 64-token kernel)
  bf16x4 obuf[2];
  if constexpr (WRITE_O) {
    const bf16x8 va = cat(vb[0], vb[1]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 acc = yq[nt];
      if constexpr (GATED) acc = acc * ld<float>(ob + LY::O_CG + CG_GS + 4 * (16 * nt + n));
      acc = mma32(acc, va, ld<bf16x8>(ob + LY::O_P + p_read(lb, nt, 0)));
      obuf[nt] = cvt4(acc);
    }
  }
  // the state at the chunk start, h = s_c h~, as S = h^T in bf16 (the layout
  // of the 64-token kernel's stored states, one state per 32-token chunk)
  if constexpr (STORE_STATES) {
    const float sc = GATED ? ld<float>(ob + LY::O_CG + CG_SC) : 1.f;
    bf16 *dst = states_dst + (size_t)col * DK + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      *reinterpret_cast<bf16x8 *>(dst + 32 * kb) = bfrag<bf16>(hs[2 * kb] * sc, hs[2 * kb + 1] * sc);
  }
  // h~ <- h~ + K^T diag(w / s_{c+1}) V'   (after h~ *= gamma_31 s_c on a rescale)
  bf16x8 wb;
  {
    f32x4 w0 = vp[0], w1 = vp[1];
    if constexpr (GATED) {
      w0 = w0 * ld<f32x4>(ob + LY::O_CG + CG_WS + 4 * (4 * g));
      w1 = w1 * ld<f32x4>(ob + LY::O_CG + CG_WS + 4 * (16 + 4 * g));
    }
    wb = cat(cvt4(w0), cvt4(w1));
  }
  if constexpr (GATED) {
    const float hsc = ld<float>(ob + LY::O_CG + CG_HSCALE);
    if (hsc != 1.f) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) hs[mt] = hs[mt] * hsc;
    }
    __asm__ volatile("s_nop 4" ::: "memory");
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t a = slot + LY::S_K + 8 * (mt & 1) + (lb.ktr ^ (64 * (mt >> 1)));
    const bf16x4 lo = ld_tr(a);
    const bf16x4 hi = ld_tr(a + 16 * LY::RB);
    hs[mt] = mma32(hs[mt], cat(lo, hi), wb);
  }
  if constexpr (WRITE_O) {
    bf16 *orow = static_cast<bf16 *>(p.o) + (row0 * H + h) * (size_t)DV + (col - n) + 4 * g;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      if (16 * nt + n < L) *reinterpret_cast<bf16x4 *>(orow + (size_t)(16 * nt + n) * H * DV) = obuf[nt];
  }
  mfma_settle();  // the state is read again after the barrier
}

// ---------------------------------------------------------------- kernel

template <int DK, bool GATED, bool STORE_STATES, bool WRITE_O>
__global__ __launch_bounds__(F32_THREADS, 1) void fwd32_kernel(FwdParams p) {
  using LY = Lay32<DK>;
  constexpr int MT = LY::MT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const uint32_t sbase = (uint32_t)(uintptr_t)(lds_ptr<unsigned char>)smem_raw;

  int pair, tile;
  wg_coords(blockIdx.x, p.ntiles, p.xcd_map, pair, tile);
  if (pair >= p.N * p.H) return;
  const int n_seq = pair_seq(p.seq_order, pair / p.H), h = pair % p.H;
  const int dv0 = tile * DVT;
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  const int nch = (si.len + C32 - 1) / C32;
  const int H = p.H, DV = p.DV;

  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const bool chain = w < 4;
  const int v = w & 3;
  const int col = dv0 + 16 * v + n;
  const size_t row_base = (size_t)si.b * p.T + si.t0;
  const Bases lb = lane_bases<DK>(v, l);

  // P's upper block stays zero in both result buffers
  for (int i = threadIdx.x; i < 2 * LY::OUTB / 16; i += F32_THREADS)
    st<f32x4>(sbase + LY::OUT_OFF + 16 * i, zero4());

  // direct-load offsets of prep wave v (bytes, relative to the chunk's first row of this head)
  uint32_t koff[LY::DMA_KQ], voff;
  int krow[LY::DMA_KQ], vrow;
#pragma unroll
  for (int i = 0; i < LY::DMA_KQ; ++i) {
    const int pp = 64 * (v + 4 * i) + l;
    const int r = pp / LY::UNITS, u = (pp % LY::UNITS) ^ swz_kq<DK>(r);
    krow[i] = r;
    koff[i] = (uint32_t)r * (uint32_t)(H * DK * 2) + 16u * u;
  }
  {
    const int pp = 64 * v + l;
    const int r = pp / 8, u = (pp % 8) ^ swz_v(r);
    vrow = r;
    voff = (uint32_t)r * (uint32_t)(DV * 2) * (uint32_t)H + 16u * u;
  }
  const uint32_t soff = (uint32_t)l * (uint32_t)(H * 4);
  const char *gk = static_cast<const char *>(p.k);
  const char *gq = static_cast<const char *>(p.q);
  const char *gv = static_cast<const char *>(p.v);

  // prep waves: loads of chunk cc into its ring slot; K, Q, g, beta before V
  auto issue = [&](int cc) {
    const uint32_t slot = sbase + (uint32_t)(cc % NBUF32) * LY::SLOT;
    const int Lc = min(C32, si.len - cc * C32);
    const size_t r0 = row_base + (size_t)cc * C32;
    const char *kb_ = gk + (r0 * H + h) * (size_t)(DK * 2);
    const char *qb_ = gq + (r0 * H + h) * (size_t)(DK * 2);
    const char *vb_ = gv + ((r0 * H + h) * (size_t)DV + dv0) * 2;
    const char *sb = reinterpret_cast<const char *>(v == 0 ? p.g : p.beta) + (r0 * H + h) * 4;
    const bool scal = (v == 1) || (GATED && v == 0);
    const uint32_t sdst = slot + (v == 0 ? LY::S_G : LY::S_BETA);
#pragma unroll
    for (int i = 0; i < LY::DMA_KQ; ++i) {
      const uint32_t dst = slot + LY::S_K + 1024 * (v + 4 * i);
      if (krow[i] < Lc) {
        dma16s(kb_, koff[i], dst);
        dma16s(qb_, koff[i], dst + LY::KQ);
      }
    }
    if (scal && l < Lc) dma4(sb + soff, sdst);
    if (vrow < Lc) dma16s(vb_, voff, slot + LY::S_V + 1024 * v);
    if (Lc < C32) {
      // rows past the end are zero (the loads never write them)
      const int tp = threadIdx.x - 4 * 64;
      for (int i = Lc * LY::RB / 16 + tp; i < LY::KQ / 16; i += 4 * 64) {
        st<f32x4>(slot + LY::S_K + 16 * i, zero4());
        st<f32x4>(slot + LY::S_Q + 16 * i, zero4());
      }
      for (int i = Lc * 128 / 16 + tp; i < LY::VT / 16; i += 4 * 64) st<f32x4>(slot + LY::S_V + 16 * i, zero4());
    }
  };
  auto full = [&](int cc) { return (cc + 1) * C32 <= si.len; };

  // chain waves: state slice, lane (n, g) holds rows prow(mt, 4g + i) of column `col`
  f32x4 hs[MT];
  const size_t st_base = ((size_t)n_seq * H + h) * DK * DV;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
      hs[mt][i] = (chain && p.h0) ? p.h0[st_base + (size_t)r * DV + col] : 0.f;
    }
  float scale = 1.f;  // prep wave 0: state scale s_c of the next chunk it prepares
  // global chunk index of the sequence's first chunk (state slots)
  const int cg0 = STORE_STATES ? (p.chunk_base ? p.chunk_base[n_seq] : n_seq * p.NC) : 0;

  if (!chain) {
    for (int cc = 0; cc < AHEAD - 1 && cc < nch; ++cc) issue(cc);
    wait_vm<0>();
  }
  __syncthreads();

  // step s: the chain runs chunk s, the prep runs chunk s + 1 and loads chunk
  // s + AHEAD
  for (int s = -1; s < nch; ++s) {
    if (chain) {
      if (s >= 0) {
        const uint32_t slot = sbase + (uint32_t)(s % NBUF32) * LY::SLOT;
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(s & 1) * LY::OUTB;
        const int L = min(C32, si.len - s * C32);
        bf16 *sdst = nullptr;
        if (STORE_STATES) sdst = p.states + ((size_t)(cg0 + s) * H + h) * (size_t)DV * DK;
        chain32<DK, GATED, STORE_STATES, WRITE_O>(p, lb, hs, slot, ob, L, row_base + (size_t)s * C32, h, col,
                                                  sdst);
      }
    } else {
      if (s + AHEAD < nch) issue(s + AHEAD);
      const int c = s + 1;
      if (c < nch) {
        const uint32_t slot = sbase + (uint32_t)(c % NBUF32) * LY::SLOT;
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(c & 1) * LY::OUTB;
        const uint32_t priv = sbase + LY::PRIV_OFF + (uint32_t)v * PRIV_BYTES;
        const int L = min(C32, si.len - c * C32);
        const uint32_t ka = slot + LY::S_K, qa = slot + LY::S_Q, ga = slot + LY::S_G, ba = slot + LY::S_BETA;
        if (v == 0) prep32<DK, GATED, 0>(lb, ka, qa, ga, ba, ob, priv, L, scale);
        else if (v == 1) prep32<DK, GATED, 1>(lb, ka, qa, ga, ba, ob, priv, L, scale);
        else if (v == 2) prep32<DK, GATED, 2>(lb, ka, qa, ga, ba, ob, priv, L, scale);
        else prep32<DK, GATED, 3>(lb, ka, qa, ga, ba, ob, priv, L, scale);
      }
      // K, Q, g, beta of chunk s + 2 (and everything older) land before the
      // barrier; its V and the loads of chunk s + 3 (at most 2 DMA_KQ + 2 of
      // this wave's, all issued after them) may stay in flight
      if (s + AHEAD < nch && full(s + AHEAD)) wait_vm<2 * LY::DMA_KQ + 2>();
      else if (s + 2 < nch && full(s + 2)) wait_vm<LY::DMA_V>();
      else wait_vm<0>();
    }
    __syncthreads();
  }

  if (chain && p.hT) {
    float sN = 1.f;
    if (GATED && nch > 0)
      sN = ld<float>(sbase + LY::OUT_OFF + (uint32_t)((nch - 1) & 1) * LY::OUTB + LY::O_CG + CG_SNEXT);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
        p.hT[st_base + (size_t)r * DV + col] = hs[mt][i] * sN;
      }
  }
}

template <int DK, bool STORE_STATES, bool WRITE_O>
hipError_t launch32_t(const FwdParams &p, hipStream_t stream) {
  const size_t smem = Lay32<DK>::TOTAL;
  auto kern = p.g ? fwd32_kernel<DK, true, STORE_STATES, WRITE_O> : fwd32_kernel<DK, false, STORE_STATES, WRITE_O>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.N * p.H * p.ntiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(F32_THREADS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_c32(const FwdParams &p, int DK, bool store_states, bool write_o, hipStream_t stream) {
#define DN_FWD32_CASE(D)                                                 \
  if (store_states)                                                      \
    return write_o ? launch32_t<D, true, true>(p, stream)                \
                   : launch32_t<D, true, false>(p, stream);              \
  return write_o ? launch32_t<D, false, true>(p, stream) : hipErrorInvalidValue;
  if (DK == 64) { DN_FWD32_CASE(64) }
  if (DK == 128) { DN_FWD32_CASE(128) }
  return hipErrorInvalidValue;
#undef DN_FWD32_CASE
}

}  // namespace dn
