// Reverse sweep of the backward pass for gfx950, bf16 inputs: the gradient
// w.r.t. the state at every chunk boundary.
//
// One workgroup owns one (sequence, head, 64-wide d_v tile) and walks the
// sequence's chunks from the last to the first, with dh (the gradient w.r.t.
// the state leaving the current chunk, d_k x d_v, fp32) in registers.  Per
// chunk, with the chunk quantities of the forward pass:
//
//   store dh (bf16, transposed) for the chunk-parallel gradient kernel
//   dV' = P^T dO + diag(w) K dh
//   dX  = T^T dV' = diag(beta) R^T dV'      (block backward substitution:
//         dX_i = diag(beta_i) R_ii^T (dV'_i - sum_{m>i} M_mi^T dX_m))
//   dh <- gamma_63 dh + Q^T diag(gamma) dO - K^T diag(gamma) dX
//
// and dh0 is dh after the first chunk.  These are the adjoint of the chunk
// recurrence h <- gamma_63 h + K^T diag(w) V', V' = T (V - diag(gamma) K h),
// O = diag(gamma) Q h + P V'.
//
// The workgroup runs the forward kernel's two roles: four chain waves own
// d_v columns 16w .. 16w + 15 and run the recurrence above; four prep waves
// run one chunk ahead (in reverse order) with the shared chunk preparation
// (P^T, -M blocks, R_ii, gate tables) and issue the direct loads of K, Q, dO,
// g, beta two chunks ahead into a three-slot ring.  dh is carried scaled,
// dh = s dh~, so that the decay costs no work on it (the scale restarts at 1
// when it would fall below 2^-30), like the forward state.
//
// The kernel takes the number NB of 16-token blocks per chunk as a template
// argument: 4 (64-token chunks) or 2 (32-token chunks, which use the first
// half of every token-indexed buffer; every product of a block with index
// >= NB is left out at compile time).
#include "dn_wy.h"

namespace dn {
namespace {

using namespace wy;

constexpr int SCAN_THREADS = 512;  // four chain waves, four prep waves
constexpr int NBUF = 3;

// dO tile swizzle: conflict free for transposed reads of rows 32kb + 8g + 4hh + e
// (P^T dO) and of rows 32kb + 16hh + 4g + e (the update's B operand)
__device__ __forceinline__ int swz_sd(int r) { return (r & 2) | ((((r >> 2) ^ (r >> 3)) & 1) << 2); }

template <int DK>
struct SLay {
  static constexpr int RB = 2 * DK, KB = DK / 32, MT = DK / 16, UNITS = DK / 8;
  static constexpr int KQ = CH * RB, DT = CH * DVT * 2;
  static constexpr int DMA_KQ = KQ / 4096, DMA_D = DT / 4096;
  static constexpr int S_K = 0, S_Q = KQ, S_D = 2 * KQ, S_G = 2 * KQ + DT, S_BETA = S_G + 4 * CH;
  static constexpr int SLOT = S_BETA + 4 * CH;
  using RS = Res<MODE_SCAN>;
  static constexpr int OUTB = RS::BYTES;
  static constexpr int OUT_OFF = NBUF * SLOT;
  static constexpr int PRIV_OFF = OUT_OFF + 2 * OUTB;
  static constexpr int TOTAL = PRIV_OFF + 4 * PRIV_BYTES;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static_assert(SLOT % 256 == 0 && OUTB % 256 == 0, "alignment");
};

template <int DK>
struct ScanKsw {
  uint32_t frag_base;
  __device__ __forceinline__ uint32_t frag(int t, int kb) const { return (frag_base ^ (64 * kb)) + 16 * t * 2 * DK; }
};

// ---------------------------------------------------------------- chain

template <int DK, bool GATED, int NB>
__device__ __forceinline__ void chain_chunk(const Bases &lb, f32x4 (&hs)[DK / 16], uint32_t slot, uint32_t ob,
                                            const uint32_t (&dtr)[2], const uint32_t (&dpr)[2], bf16 *dst) {
  using LY = SLay<DK>;
  using RS = Res<MODE_SCAN>;
  constexpr int KB = LY::KB, MT = LY::MT;
  constexpr int NKB = NB / 2;  // 32-token contraction blocks of the chunk
  const int l = lane_id(), g = l >> 4;
  const uint32_t cgt = ob + RS::O_CG;

  // the gradient w.r.t. the state leaving the chunk, dh = s dh~, as dS = dh^T in bf16
  {
    const float sc = GATED ? ld<float>(cgt + CG_SC) : 1.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      *reinterpret_cast<bf16x8 *>(dst + 32 * kb) = bfrag<bf16>(hs[2 * kb] * sc, hs[2 * kb + 1] * sc);
  }
  bf16x8 hb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) hb[kb] = bfrag<bf16>(hs[2 * kb], hs[2 * kb + 1]);

  // dV' = diag(w s) K dh~ + P^T dO (lane (n, g): row 16t + 4g + e, column 16w + n)
  f32x4 dvp[NB];
  {
    bf16x8 kf[NB][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t a = (lb.frag ^ (64 * kb)) + slot + LY::S_K;
#pragma unroll
      for (int t = 0; t < NB; ++t) kf[t][kb] = ld<bf16x8>(a + 16 * t * LY::RB);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      f32x4 yd = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yd = mma32(yd, kf[t][kb], hb[kb]);
      dvp[t] = GATED ? yd * ld<f32x4>(cgt + CG_WS + 4 * (16 * t + 4 * g)) : yd;
    }
  }
  bf16x8 dob[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
    dob[kb] = cat(ld_tr(slot + LY::S_D + 32 * kb * 128 + dtr[0]), ld_tr(slot + LY::S_D + 32 * kb * 128 + dtr[1]));
#pragma unroll
  for (int t = 0; t < NB; ++t)
#pragma unroll
    for (int kb = t >> 1; kb < NKB; ++kb) dvp[t] = mma32(dvp[t], ld<bf16x8>(ob + RS::O_P + pt_frag(t, kb, l)), dob[kb]);

  // dh~ <- dh~ + Q^T diag(gamma / s) dO - K^T diag(gamma / s) dX (after dh~ *= gamma_63 s on a restart):
  // the restart scale and the dO term first (neither depends on dX), the dX term after the substitution;
  // contraction slot 8g + s of block kb is token 32kb + 16(s/4) + 4g + s%4
  if constexpr (GATED) {
    const float hsc = ld<float>(cgt + CG_HSCALE);
    if (hsc != 1.f) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) hs[mt] = hs[mt] * hsc;
    }
    __asm__ volatile("s_nop 4" ::: "memory");
  }
  {
    bf16x8 bo[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      bf16x4 part[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const bf16x4 d = ld_tr(slot + LY::S_D + 32 * kb * 128 + dpr[hh]);
        if constexpr (GATED) {
          const f32x4 gs = ld<f32x4>(cgt + CG_GS + 4 * (32 * kb + 16 * hh + 4 * g));
          f32x4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = bf2f(d[e]) * gs[e];
          part[hh] = cvt4(f);
        } else {
          part[hh] = d;
        }
      }
      bo[kb] = cat(part[0], part[1]);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = hs[mt];
      const uint32_t aoff = 8 * (mt & 1) + (lb.ktr ^ (64 * (mt >> 1)));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const uint32_t r0 = 32 * kb * LY::RB, r1 = (32 * kb + 16) * LY::RB;
        const bf16x8 qt = cat(ld_tr(slot + LY::S_Q + aoff + r0), ld_tr(slot + LY::S_Q + aoff + r1));
        acc = mma32(acc, qt, bo[kb]);
      }
      hs[mt] = acc;
    }
  }

  // dX_i = diag(beta_i) R_ii^T (dV'_i - sum_{m>i} M_mi^T dX_m)
  f32x4 dx[NB];
  bf16x4 dxb[NB];
#pragma unroll
  for (int i = NB - 1; i >= 0; --i) {
    f32x4 acc = dvp[i];
#pragma unroll
    for (int m = i + 1; m < NB; ++m) acc = mma16(acc, ld_tr(ob + RS::O_M + 512 * m_block(m, i) + lb.btr), dxb[m]);
    const f32x4 y = mma16(zero4(), ld<bf16x4>(ob + RS::O_TT + 512 * i + lb.m), cvt4(acc));
    dx[i] = y * ld<f32x4>(slot + LY::S_BETA + 4 * (16 * i + 4 * g));
    dxb[i] = cvt4(dx[i]);
  }
  bf16x8 bx[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    f32x4 x0 = -dx[2 * kb], x1 = -dx[2 * kb + 1];
    if constexpr (GATED) {
      x0 = x0 * ld<f32x4>(cgt + CG_GS + 4 * (32 * kb + 4 * g));
      x1 = x1 * ld<f32x4>(cgt + CG_GS + 4 * (32 * kb + 16 + 4 * g));
    }
    bx[kb] = cat(cvt4(x0), cvt4(x1));
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x4 acc = hs[mt];
    const uint32_t aoff = 8 * (mt & 1) + (lb.ktr ^ (64 * (mt >> 1)));
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const uint32_t r0 = 32 * kb * LY::RB, r1 = (32 * kb + 16) * LY::RB;
      const bf16x8 kt = cat(ld_tr(slot + LY::S_K + aoff + r0), ld_tr(slot + LY::S_K + aoff + r1));
      acc = mma32(acc, kt, bx[kb]);
    }
    hs[mt] = acc;
  }
  mfma_settle();  // the state gradient is read again after the barrier
}

// ---------------------------------------------------------------- kernel

template <int DK, bool GATED, int NB>
__global__ __launch_bounds__(SCAN_THREADS, 1) void scan_bf16_kernel(BwdParams p) {
  using LY = SLay<DK>;
  constexpr int MT = LY::MT;
  constexpr int CHN = 16 * NB;               // tokens per chunk (64 or 32)
  constexpr int NKQ = LY::DMA_KQ * NB / 4;   // direct loads per prep wave of a chunk's K (or Q) rows
  constexpr int ND = LY::DMA_D * NB / 4;     // ... and of its dO rows
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const uint32_t sbase = (uint32_t)(uintptr_t)(lds_ptr<unsigned char>)smem_raw;

  int pair, tile;
  wg_coords(blockIdx.x, p.ntiles, p.xcd_map, pair, tile);
  if (pair >= p.N * p.H) return;
  const int n_seq = pair_seq(p.seq_order, pair / p.H), h = pair % p.H;
  const int dv0 = tile * DVT;
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  const int nch = (si.len + CHN - 1) / CHN;
  const int H = p.H, DV = p.DV;

  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4, e4 = (l >> 2) & 3, q4 = l & 3;
  const bool chain = w < 4;
  const int v = w & 3;
  const int col = dv0 + 16 * v + n;
  const size_t row_base = (size_t)si.b * p.T + si.t0;
  const Bases lb = lane_bases<DK>(v, l);
  uint32_t dtr[2], dpr[2];  // dO transposed reads: natural rows (P^T dO), paired rows (update)
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g + 4 * hh + e4, r2 = 16 * hh + 4 * g + e4;
    dtr[hh] = r * 128 + 16 * ((2 * v + (q4 >> 1)) ^ swz_sd(r)) + 8 * (q4 & 1);
    dpr[hh] = r2 * 128 + 16 * ((2 * v + (q4 >> 1)) ^ swz_sd(r2)) + 8 * (q4 & 1);
  }

  // P^T above the diagonal stays zero in both result buffers
  for (int i = threadIdx.x; i < 2 * LY::OUTB / 16; i += SCAN_THREADS) st<f32x4>(sbase + LY::OUT_OFF + 16 * i, zero4());

  // direct-load offsets of prep wave v
  uint32_t koff[LY::DMA_KQ], doff[LY::DMA_D];
  int krow[LY::DMA_KQ], drow[LY::DMA_D];
#pragma unroll
  for (int i = 0; i < LY::DMA_KQ; ++i) {
    const int pp = 64 * (v + 4 * i) + l;
    const int r = pp / LY::UNITS, u = (pp % LY::UNITS) ^ swz_kq<DK>(r);
    krow[i] = r;
    koff[i] = (uint32_t)r * (uint32_t)(H * DK * 2) + 16u * u;
  }
#pragma unroll
  for (int i = 0; i < LY::DMA_D; ++i) {
    const int pp = 64 * (v + 4 * i) + l;
    const int r = pp / 8, u = (pp % 8) ^ swz_sd(r);
    drow[i] = r;
    doff[i] = (uint32_t)r * (uint32_t)(DV * 2) * (uint32_t)H + 16u * u;
  }
  const uint32_t soff = (uint32_t)l * (uint32_t)(H * 4);
  const char *gk = static_cast<const char *>(p.k);
  const char *gq = static_cast<const char *>(p.q);
  const char *gdo = static_cast<const char *>(p.dO);

  // chunk of order o (o = 0 is the last chunk) and its ring slot
  auto chunk_of = [&](int o) { return nch - 1 - o; };
  auto slot_of = [&](int o) { return sbase + (uint32_t)(o % NBUF) * LY::SLOT; };
  // loads of order o in four parts issued between the prep stages (K, g and
  // beta; K; Q; dO: dO last); a partial chunk loads everything in part 0
  auto issue = [&](int o, int part) {
    const int cc = chunk_of(o);
    const uint32_t slot = slot_of(o);
    const int Lc = min(CHN, si.len - cc * CHN);
    const size_t r0 = row_base + (size_t)cc * CHN;
    const char *kb_ = gk + (r0 * H + h) * (size_t)(DK * 2);
    const char *qb_ = gq + (r0 * H + h) * (size_t)(DK * 2);
    const char *db_ = gdo + ((r0 * H + h) * (size_t)DV + dv0) * 2;
    const float *sp = v == 0 ? p.g : p.beta;
    const bool scal = (v == 1) || (GATED && v == 0);
    const uint32_t sdst = slot + (v == 0 ? LY::S_G : LY::S_BETA);
    if (Lc == CHN) {
      // load i of a prep wave covers rows below CHN exactly when i < NKQ (ND)
      constexpr int KH = (NKQ + 1) / 2;
      if (part == 0) {
#pragma unroll
        for (int i = 0; i < KH; ++i) dma16s(kb_, koff[i], slot + LY::S_K + 1024 * (v + 4 * i));
        // one lane per row of the chunk: with 32-token chunks lanes 32 .. 63
        // would read the rows after it, past the end of the last chunk
        if (scal && (NB == 4 || l < CHN)) dma4(reinterpret_cast<const char *>(sp + r0 * H + h) + soff, sdst);
      } else if (part == 1) {
#pragma unroll
        for (int i = KH; i < NKQ; ++i) dma16s(kb_, koff[i], slot + LY::S_K + 1024 * (v + 4 * i));
      } else if (part == 2) {
#pragma unroll
        for (int i = 0; i < NKQ; ++i) dma16s(qb_, koff[i], slot + LY::S_Q + 1024 * (v + 4 * i));
      } else {
#pragma unroll
        for (int i = 0; i < ND; ++i) dma16s(db_, doff[i], slot + LY::S_D + 1024 * (v + 4 * i));
      }
    } else if (part == 0) {
#pragma unroll
      for (int i = 0; i < LY::DMA_KQ; ++i) {
        const uint32_t dst = slot + LY::S_K + 1024 * (v + 4 * i);
        if (krow[i] < Lc) {
          dma16s(kb_, koff[i], dst);
          dma16s(qb_, koff[i], dst + LY::KQ);
        }
      }
      if (scal && l < Lc) dma4(reinterpret_cast<const char *>(sp + r0 * H + h) + soff, sdst);
#pragma unroll
      for (int i = 0; i < LY::DMA_D; ++i)
        if (drow[i] < Lc) dma16s(db_, doff[i], slot + LY::S_D + 1024 * (v + 4 * i));
      // rows past the end are zero (the loads never write them)
      const int tp = threadIdx.x - 4 * 64;
      for (int i = Lc * LY::RB / 16 + tp; i < LY::KQ / 16; i += 4 * 64) {
        st<f32x4>(slot + LY::S_K + 16 * i, zero4());
        st<f32x4>(slot + LY::S_Q + 16 * i, zero4());
      }
      for (int i = Lc * 128 / 16 + tp; i < LY::DT / 16; i += 4 * 64) st<f32x4>(slot + LY::S_D + 16 * i, zero4());
      if (tp < CHN && tp >= Lc) {
        st<float>(slot + LY::S_G + 4 * tp, 0.f);
        st<float>(slot + LY::S_BETA + 4 * tp, 0.f);
      }
    }
  };
  auto full = [&](int o) { return (chunk_of(o) + 1) * CHN <= si.len; };

  // chain waves: dh~ slice, lane (n, g) holds rows prow(mt, 4g + i) of column `col`
  f32x4 hs[MT];
  const size_t st_base = ((size_t)n_seq * H + h) * DK * DV;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
      hs[mt][i] = (chain && p.dhT) ? p.dhT[st_base + (size_t)r * DV + col] : 0.f;
    }
  float scale = 1.f;  // prep wave 0: scale of dh entering the next chunk it prepares
  // global chunk index of the sequence's first chunk (state slots)
  const int cg0 = p.chunk_base ? p.chunk_base[n_seq] : n_seq * p.NC;

  if (!chain) {
    if (nch > 0)
      for (int part = 0; part < 4; ++part) issue(0, part);
    wait_vm<0>();
  }
  __syncthreads();

  // step s: the chain runs order s, the prep order s + 1, the loads order s + 2
  for (int s = -1; s < nch; ++s) {
    if (chain) {
      if (s >= 0) {
        const int c = chunk_of(s);
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(s & 1) * LY::OUTB;
        bf16 *dst = p.dstates + (((size_t)(cg0 + c) * H + h) * DV + col) * DK + 8 * g;
        chain_chunk<DK, GATED, NB>(lb, hs, slot_of(s), ob, dtr, dpr, dst);
      }
    } else {
      const bool iss_now = s + 2 < nch;
      auto iss = [&](int part) {
        if (iss_now) issue(s + 2, part);
      };
      const int o = s + 1;
      if (o < nch) {
        const int c = chunk_of(o);
        const uint32_t slot = slot_of(o);
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(o & 1) * LY::OUTB;
        const uint32_t priv = sbase + LY::PRIV_OFF + (uint32_t)v * PRIV_BYTES;
        const int L = min(CHN, si.len - c * CHN);
        const ScanKsw<DK> ksw{lb.frag};
        const uint32_t ka = slot + LY::S_K, qa = slot + LY::S_Q, ga = slot + LY::S_G, ba = slot + LY::S_BETA;
        if (v == 0) prep_chunk<DK, GATED, true, MODE_SCAN, 0, NB>(lb, ka, qa, ga, ba, ob, priv, L, scale, ksw, iss);
        else if (v == 1) prep_chunk<DK, GATED, true, MODE_SCAN, 1, NB>(lb, ka, qa, ga, ba, ob, priv, L, scale, ksw, iss);
        else if (v == 2) prep_chunk<DK, GATED, true, MODE_SCAN, 2, NB>(lb, ka, qa, ga, ba, ob, priv, L, scale, ksw, iss);
        else prep_chunk<DK, GATED, true, MODE_SCAN, 3, NB>(lb, ka, qa, ga, ba, ob, priv, L, scale, ksw, iss);
      }
      // K, Q, g, beta of order s + 2 (and everything older) land before the
      // barrier; its dO may stay in flight until the next one
      if (s + 2 < nch && full(s + 2)) wait_vm<ND>();
      else wait_vm<0>();
    }
    __syncthreads();
  }

  if (chain && p.dh0) {
    float s0 = 1.f;
    if (GATED && nch > 0)
      s0 = ld<float>(sbase + LY::OUT_OFF + (uint32_t)((nch - 1) & 1) * LY::OUTB + Res<MODE_SCAN>::O_CG + CG_SNEXT);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
        p.dh0[st_base + (size_t)r * DV + col] = hs[mt][i] * s0;
      }
  }
}

template <int DK, int NB>
hipError_t launch_t(const BwdParams &p, hipStream_t stream) {
  const size_t smem = SLay<DK>::TOTAL;
  auto kern = p.g ? scan_bf16_kernel<DK, true, NB> : scan_bf16_kernel<DK, false, NB>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.N * p.H * p.ntiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(SCAN_THREADS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_scan(const BwdParams &p, int DK, hipStream_t stream) {
  if (p.chunk == 32) {
    if (DK == 64) return launch_t<64, 2>(p, stream);
    if (DK == 128) return launch_t<128, 2>(p, stream);
    return hipErrorInvalidValue;
  }
  if (DK == 64) return launch_t<64, 4>(p, stream);
  if (DK == 128) return launch_t<128, 4>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dn
