// Fused chunkwise forward pass of the (gated) delta rule for gfx950, bf16
// inputs (d_k 64 or 128).
//
// One workgroup owns one (sequence, head, 64-wide d_v tile) and walks the
// sequence's 64-token chunks in order.  It runs eight waves in two roles,
// two waves per SIMD, so that one wave's stalls are filled by the other:
//
//   chain waves 0..3  wave w owns d_v columns 16w .. 16w + 15 of the tile and
//                     keeps its d_k x 16 slice of the state h = S^T (fp32) in
//                     registers; per chunk it runs the state recurrence.
//   prep waves 4..7   run one chunk ahead: they issue the direct loads, build
//                     the gate tables and everything of a chunk that does not
//                     depend on the state.
//
// For chunk c (b = cumsum g inside the chunk, gamma = exp b,
// Gamma_rj = exp(b_r - b_j) for j <= r, w_r = exp(b_63 - b_r)):
//
//   prep   the lower 16 x 16 blocks of M = strictLower((K K^T) * Gamma) and
//          P = (Q K^T) * Gamma (MFMA); prep wave v inverts diagonal block v:
//          T_vv = (I + diag(beta) M_vv)^-1 diag(beta) by fp32 forward
//          substitution, four lanes per column.
//   chain  Y_K = K h, Y_Q = Q h;
//          V' = (I + diag(beta) M)^-1 diag(beta) (V - diag(gamma) Y_K), by
//          block forward substitution over the four 16-token blocks,
//            V'_i = T_ii (X_i - sum_{m<i} M_im V'_m);
//          O = diag(gamma) Y_Q + P V';
//          h <- gamma_63 h + K^T diag(w) V'.
//
// This is the chunk's WY/UT form ("Parallelizing Linear Transformers with the
// Delta Rule over Sequence Length": products of Householder-like transitions
// in WY form, page 3 abstract; the UT transform named in the Gated DeltaNet
// review thread, review 2), with the gate entering through cumulative decay
// ratios (page 1, answer W2).  The (I + A)^-1 of the UT transform is formed
// only on its diagonal blocks; the block substitution applies the rest to the
// chain wave's 16 columns directly.
//
// Scaled state.  The chain keeps h~ with h = s_c h~, s_c a per-chunk scalar,
// so that the decay gamma_63 costs no work on the state:
// h~ <- h~ + K^T diag(w / s_{c+1}) V' with s_{c+1} = gamma_63 s_c; when
// s_{c+1} would fall below 2^-30 the chunk instead multiplies h~ by
// gamma_63 s_c and restarts with s = 1.  gamma s_c scales Y_K and Y_Q.
//
// Data movement.  K, Q, V and the chunk's g and beta arrive by direct
// global->LDS loads into a three-slot ring, two chunks ahead of the chain
// (one ahead of the prep).  Every LDS matrix uses an XOR swizzle of its
// 16-byte units chosen so that each access pattern is conflict free on the
// 64-bank LDS (the transposed K reads of the state update carry a two-way
// conflict that no unit swizzle removes), with a lane's address one
// precomputed base XOR a constant plus an immediate offset.  K^T operands are
// read with the LDS transpose load.  The prep's results for chunk c sit in one
// of two buffers chosen by the parity of c.
//
// Row orders.  Token tiles are natural (tile t = tokens 16t .. 16t + 15).
// Tiles of the state slice hold d_k rows prow(mt, m) = 32(mt/2) + 8(m/4) +
// 4(mt%2) + m%4, so that two stacked state tiles are the B operand of K h.
// Within a 32-token block the MFMA contraction slot 8g + s stands for token
// 16(s/4) + 4g + s%4 (two stacked natural accumulator tiles); P is stored with
// its columns permuted to match.
//
// Partial chunks are zero rows (k = q = v = 0, beta = g = 0), which leave V'
// and the state unchanged.
#include "dn_wy.h"

namespace dn {
namespace {

using namespace wy;

constexpr int FWD_THREADS = 512;  // four chain waves, four prep waves
constexpr int NBUF = 3;           // ring slots

template <int DK>
struct Lay {
  static constexpr int RB = 2 * DK;          // bytes of a K or Q row
  static constexpr int UNITS = DK / 8;       // 16-byte units of a K or Q row
  static constexpr int KB = DK / 32;         // 32-index blocks over d_k
  static constexpr int MT = DK / 16;         // 16-row tiles of a wave's state slice
  static constexpr int KQ = CH * RB;         // bytes of a K or Q tile
  static constexpr int VT = CH * DVT * 2;    // bytes of a V tile
  static constexpr int DMA_KQ = KQ / 4096;   // direct loads per prep wave for a K or Q tile
  static constexpr int DMA_V = VT / 4096;    // direct loads per prep wave for a V tile
  // ring slot
  static constexpr int S_K = 0, S_Q = KQ, S_V = 2 * KQ, S_G = 2 * KQ + VT, S_BETA = S_G + 4 * CH;
  static constexpr int SLOT = S_BETA + 4 * CH;
  // prep results of one chunk
  using RS = Res<MODE_FWD>;
  static constexpr int O_P = RS::O_P, O_M = RS::O_M, O_TT = RS::O_TT, O_CG = RS::O_CG;
  static constexpr int OUTB = RS::BYTES;
  static constexpr int OUT_OFF = NBUF * SLOT;
  static constexpr int PRIV_OFF = OUT_OFF + 2 * OUTB;  // per prep wave: A_vv^T, gate table
  static constexpr int PRIV = PRIV_BYTES;
  static constexpr int TOTAL = PRIV_OFF + 4 * PRIV;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static_assert(SLOT % 256 == 0 && OUTB % 256 == 0, "tile alignment");
};

// K / Q fragment addresses of the forward tiles
template <int DK>
struct FwdKsw {
  uint32_t frag_base;
  __device__ __forceinline__ uint32_t frag(int t, int kb) const {
    return (frag_base ^ (64 * kb)) + 16 * t * 2 * DK;
  }
};

// ---------------------------------------------------------------- chain

template <int DK, bool GATED, bool STORE_STATES, bool WRITE_O>
__device__ __forceinline__ void chain_chunk(const FwdParams &p, const Bases &lb, f32x4 (&hs)[DK / 16],
                                            uint32_t slot, uint32_t ob, int L, size_t row0, int h,
                                            int col, bf16 *states_dst) {
  using LY = Lay<DK>;
  constexpr int KB = LY::KB, MT = LY::MT;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int H = p.H, DV = p.DV;

  bf16x8 hb[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) hb[kb] = bfrag<bf16>(hs[2 * kb], hs[2 * kb + 1]);

  // Y_K = K h~ (lane (n, g): row 16t + 4g + e, column 16w + n)
  f32x4 yk[4], yq[4];
  {
    bf16x8 kf[4][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t a = (lb.frag ^ (64 * kb)) + slot + LY::S_K;
#pragma unroll
      for (int t = 0; t < 4; ++t) kf[t][kb] = ld<bf16x8>(a + 16 * t * LY::RB);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      yk[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yk[t] = mma32(yk[t], kf[t][kb], hb[kb]);
    }
  }
  // Y_Q^T = h~^T Q^T (lane (n, g): row 16t + n, column 16w + 4g + e)
  if constexpr (WRITE_O) {
    bf16x8 qf[4][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const uint32_t a = (lb.frag ^ (64 * kb)) + slot + LY::S_Q;
#pragma unroll
      for (int t = 0; t < 4; ++t) qf[t][kb] = ld<bf16x8>(a + 16 * t * LY::RB);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      yq[t] = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) yq[t] = mma32(yq[t], hb[kb], qf[t][kb]);
    }
  }

  // X = V - diag(gamma s_c) Y_K
  f32x4 x[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const bf16x4 vr = ld_tr(slot + LY::S_V + 16 * t * 128 + lb.vtr);
    const f32x4 gm = GATED ? ld<f32x4>(ob + LY::O_CG + CG_GS + 4 * (16 * t + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) x[t][e] = bf2f(vr[e]) - gm[e] * yk[t][e];
  }
  // V'_i = T_ii (X_i - sum_{m<i} M_im V'_m)
  bf16x4 vb[4];
  f32x4 vp[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 acc = x[i];
#pragma unroll
    for (int m = 0; m < i; ++m) acc = mma16(acc, ld<bf16x4>(ob + LY::O_M + 512 * m_block(i, m) + lb.m), vb[m]);
    const bf16x4 tf = ld_tr(ob + LY::O_TT + 512 * i + lb.btr);
    vp[i] = mma16(zero4(), tf, cvt4(acc));
    vb[i] = cvt4(vp[i]);
  }
  // O^T = diag(gamma s_c) Y_Q^T + V'^T P^T: lane (n, g) holds O[16nt + n][16w + 4g + e]
  // the output tiles are stored after the state update, at the end of the
  // step, when the prep waves' direct loads for the step have landed (the
  // stores then do not queue behind them; 5 % faster in the state-storing
  // variant)
  bf16x4 obuf[4];
  if constexpr (WRITE_O) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 acc = yq[nt];
      if constexpr (GATED) acc = acc * ld<float>(ob + LY::O_CG + CG_GS + 4 * (16 * nt + n));
#pragma unroll
      for (int kb = 0; kb <= (nt >> 1); ++kb)
        acc = mma32(acc, cat(vb[2 * kb], vb[2 * kb + 1]), ld<bf16x8>(ob + LY::O_P + p_read(lb, nt, kb)));
      obuf[nt] = cvt4(acc);
    }
  }
  // the state at the chunk start, h = s_c h~, as S = h^T in bf16: stored here,
  // late in the step, so that the stores do not compete with the prep waves'
  // loads, which are issued at the start of the step
  if constexpr (STORE_STATES) {
    const float sc = GATED ? ld<float>(ob + LY::O_CG + CG_SC) : 1.f;
    bf16 *dst = states_dst + (size_t)col * DK + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      *reinterpret_cast<bf16x8 *>(dst + 32 * kb) = bfrag<bf16>(hs[2 * kb] * sc, hs[2 * kb + 1] * sc);
  }
  // h~ <- h~ + K^T diag(w / s_{c+1}) V'   (after h~ *= gamma_63 s_c on a rescale)
  bf16x8 wb[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x4 w0 = vp[2 * kb], w1 = vp[2 * kb + 1];
    if constexpr (GATED) {
      w0 = w0 * ld<f32x4>(ob + LY::O_CG + CG_WS + 4 * (32 * kb + 4 * g));
      w1 = w1 * ld<f32x4>(ob + LY::O_CG + CG_WS + 4 * (32 * kb + 16 + 4 * g));
    }
    wb[kb] = cat(cvt4(w0), cvt4(w1));
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
    f32x4 acc = hs[mt];
    const uint32_t a = slot + LY::S_K + 8 * (mt & 1) + (lb.ktr ^ (64 * (mt >> 1)));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x4 lo = ld_tr(a + 32 * kb * LY::RB);
      const bf16x4 hi = ld_tr(a + (32 * kb + 16) * LY::RB);
      acc = mma32(acc, cat(lo, hi), wb[kb]);
    }
    hs[mt] = acc;
  }
  if constexpr (WRITE_O) {
    bf16 *orow = static_cast<bf16 *>(p.o) + (row0 * H + h) * (size_t)DV + (col - n) + 4 * g;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (16 * nt + n < L) *reinterpret_cast<bf16x4 *>(orow + (size_t)(16 * nt + n) * H * DV) = obuf[nt];
  }
  mfma_settle();  // the state is read again after the barrier
}

// ---------------------------------------------------------------- kernel

template <int DK, bool GATED, bool STORE_STATES, bool WRITE_O>
__global__ __launch_bounds__(FWD_THREADS, 1) void fwd_bf16_kernel(FwdParams p) {
  using LY = Lay<DK>;
  constexpr int MT = LY::MT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const uint32_t sbase = (uint32_t)(uintptr_t)(lds_ptr<unsigned char>)smem_raw;

  int pair, tile;
  wg_coords(blockIdx.x, p.ntiles, p.xcd_map, pair, tile);
  if (pair >= p.N * p.H) return;
  const int n_seq = pair_seq(p.seq_order, pair / p.H), h = pair % p.H;
  const int dv0 = tile * DVT;
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  const int nch = (si.len + CH - 1) / CH;
  const int H = p.H, DV = p.DV;

  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4;
  const bool chain = w < 4;
  const int v = w & 3;                                 // index within the role
  const int col = dv0 + 16 * v + n;                    // chain wave: this lane's d_v column
  const size_t row_base = (size_t)si.b * p.T + si.t0;  // global row of the sequence start
  const Bases lb = lane_bases<DK>(v, l);

  // P's upper blocks stay zero in both result buffers
  for (int i = threadIdx.x; i < 2 * LY::OUTB / 16; i += FWD_THREADS)
    st<f32x4>(sbase + LY::OUT_OFF + 16 * i, zero4());

  // direct-load offsets of prep wave v (bytes, relative to the chunk's first row of this head)
  uint32_t koff[LY::DMA_KQ], voff[LY::DMA_V];
  int krow[LY::DMA_KQ], vrow[LY::DMA_V];
#pragma unroll
  for (int i = 0; i < LY::DMA_KQ; ++i) {
    const int pp = 64 * (v + 4 * i) + l;
    const int r = pp / LY::UNITS, u = (pp % LY::UNITS) ^ swz_kq<DK>(r);
    krow[i] = r;
    koff[i] = (uint32_t)r * (uint32_t)(H * DK * 2) + 16u * u;
  }
#pragma unroll
  for (int i = 0; i < LY::DMA_V; ++i) {
    const int pp = 64 * (v + 4 * i) + l;
    const int r = pp / 8, u = (pp % 8) ^ swz_v(r);
    vrow[i] = r;
    voff[i] = (uint32_t)r * (uint32_t)(DV * 2) * (uint32_t)H + 16u * u;
  }
  const uint32_t soff = (uint32_t)l * (uint32_t)(H * 4);
  const char *gk = static_cast<const char *>(p.k);
  const char *gq = static_cast<const char *>(p.q);
  const char *gv = static_cast<const char *>(p.v);

  // prep waves: loads of chunk cc into its ring slot; K, Q, g, beta before V
  auto issue = [&](int cc) {
    const uint32_t slot = sbase + (uint32_t)(cc % NBUF) * LY::SLOT;
    const int Lc = min(CH, si.len - cc * CH);
    const size_t r0 = row_base + (size_t)cc * CH;
    const char *kb_ = gk + (r0 * H + h) * (size_t)(DK * 2);
    const char *qb_ = gq + (r0 * H + h) * (size_t)(DK * 2);
    const char *vb_ = gv + ((r0 * H + h) * (size_t)DV + dv0) * 2;
    const char *sb = reinterpret_cast<const char *>(v == 0 ? p.g : p.beta) + (r0 * H + h) * 4;
    const bool scal = (v == 1) || (GATED && v == 0);
    const uint32_t sdst = slot + (v == 0 ? LY::S_G : LY::S_BETA);
    if (Lc == CH) {
#pragma unroll
      for (int i = 0; i < LY::DMA_KQ; ++i) {
        const uint32_t dst = slot + LY::S_K + 1024 * (v + 4 * i);
        dma16s(kb_, koff[i], dst);
        if (WRITE_O) dma16s(qb_, koff[i], dst + LY::KQ);
      }
      if (scal) dma4(sb + soff, sdst);
#pragma unroll
      for (int i = 0; i < LY::DMA_V; ++i) dma16s(vb_, voff[i], slot + LY::S_V + 1024 * (v + 4 * i));
    } else {
#pragma unroll
      for (int i = 0; i < LY::DMA_KQ; ++i) {
        const uint32_t dst = slot + LY::S_K + 1024 * (v + 4 * i);
        if (krow[i] < Lc) dma16s(kb_, koff[i], dst);
        if (WRITE_O && krow[i] < Lc) dma16s(qb_, koff[i], dst + LY::KQ);
      }
      if (scal && l < Lc) dma4(sb + soff, sdst);
#pragma unroll
      for (int i = 0; i < LY::DMA_V; ++i)
        if (vrow[i] < Lc) dma16s(vb_, voff[i], slot + LY::S_V + 1024 * (v + 4 * i));
      // rows past the end are zero (the loads never write them)
      const int tp = threadIdx.x - 4 * 64;
      for (int i = Lc * LY::RB / 16 + tp; i < LY::KQ / 16; i += 4 * 64) {
        st<f32x4>(slot + LY::S_K + 16 * i, zero4());
        if (WRITE_O) st<f32x4>(slot + LY::S_Q + 16 * i, zero4());
      }
      for (int i = Lc * 128 / 16 + tp; i < LY::VT / 16; i += 4 * 64) st<f32x4>(slot + LY::S_V + 16 * i, zero4());
    }
  };
  auto full = [&](int cc) { return (cc + 1) * CH <= si.len; };
  // Full chunks of the plain forward: K (and g, beta) up front, Q and V from
  // the prep's stage hook (after the gate tables and after the diagonal
  // block), so that the prep waves do not stall on all of a chunk's direct
  // loads at once (the loads still land within the step).  The state-storing
  // variant issues everything up front: with its state stores in the same
  // step, the later loads measured slower.
  auto issue_k = [&](int cc) {
    const uint32_t slot = sbase + (uint32_t)(cc % NBUF) * LY::SLOT;
    const size_t r0 = row_base + (size_t)cc * CH;
    const char *kb_ = gk + (r0 * H + h) * (size_t)(DK * 2);
    const char *sb = reinterpret_cast<const char *>(v == 0 ? p.g : p.beta) + (r0 * H + h) * 4;
    const bool scal = (v == 1) || (GATED && v == 0);
    const uint32_t sdst = slot + (v == 0 ? LY::S_G : LY::S_BETA);
#pragma unroll
    for (int i = 0; i < LY::DMA_KQ; ++i) dma16s(kb_, koff[i], slot + LY::S_K + 1024 * (v + 4 * i));
    if (scal) dma4(sb + soff, sdst);
  };
  auto issue_q = [&](int cc) {
    const uint32_t slot = sbase + (uint32_t)(cc % NBUF) * LY::SLOT;
    const size_t r0 = row_base + (size_t)cc * CH;
    const char *qb_ = gq + (r0 * H + h) * (size_t)(DK * 2);
#pragma unroll
    for (int i = 0; i < LY::DMA_KQ; ++i) dma16s(qb_, koff[i], slot + LY::S_Q + 1024 * (v + 4 * i));
  };
  auto issue_v = [&](int cc) {
    const uint32_t slot = sbase + (uint32_t)(cc % NBUF) * LY::SLOT;
    const size_t r0 = row_base + (size_t)cc * CH;
    const char *vb_ = gv + ((r0 * H + h) * (size_t)DV + dv0) * 2;
#pragma unroll
    for (int i = 0; i < LY::DMA_V; ++i) dma16s(vb_, voff[i], slot + LY::S_V + 1024 * (v + 4 * i));
  };

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
    if (nch > 0) issue(0);
    wait_vm<0>();
  }
  __syncthreads();

  // step s: the chain runs chunk s, the prep runs chunk s + 1 and loads chunk s + 2
  for (int s = -1; s < nch; ++s) {
    if (chain) {
      if (s >= 0) {
        const uint32_t slot = sbase + (uint32_t)(s % NBUF) * LY::SLOT;
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(s & 1) * LY::OUTB;
        const int L = min(CH, si.len - s * CH);
        bf16 *sdst = nullptr;
        if (STORE_STATES) sdst = p.states + ((size_t)(cg0 + s) * H + h) * (size_t)DV * DK;
        chain_chunk<DK, GATED, STORE_STATES, WRITE_O>(p, lb, hs, slot, ob, L, row_base + (size_t)s * CH, h,
                                                      col, sdst);
      }
    } else {
      const bool spread = WRITE_O && !STORE_STATES && s + 2 < nch && full(s + 2);
      if (s + 2 < nch) {
        if (spread) issue_k(s + 2);
        else issue(s + 2);
      }
      const int cn = s + 2;
      auto hook = [&](int st) {
        if (spread && st == 0) issue_q(cn);
        if (spread && st == 1) issue_v(cn);
      };
      const int c = s + 1;
      if (c < nch) {
        const uint32_t slot = sbase + (uint32_t)(c % NBUF) * LY::SLOT;
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(c & 1) * LY::OUTB;
        const uint32_t priv = sbase + LY::PRIV_OFF + (uint32_t)v * LY::PRIV;
        const int L = min(CH, si.len - c * CH);
        const FwdKsw<DK> ksw{lb.frag};
        if (v == 0) prep_chunk<DK, GATED, WRITE_O, MODE_FWD, 0>(lb, slot + LY::S_K, slot + LY::S_Q, slot + LY::S_G,
                                                         slot + LY::S_BETA, ob, priv, L, scale, ksw, hook);
        else if (v == 1) prep_chunk<DK, GATED, WRITE_O, MODE_FWD, 1>(lb, slot + LY::S_K, slot + LY::S_Q, slot + LY::S_G,
                                                         slot + LY::S_BETA, ob, priv, L, scale, ksw, hook);
        else if (v == 2) prep_chunk<DK, GATED, WRITE_O, MODE_FWD, 2>(lb, slot + LY::S_K, slot + LY::S_Q, slot + LY::S_G,
                                                         slot + LY::S_BETA, ob, priv, L, scale, ksw, hook);
        else prep_chunk<DK, GATED, WRITE_O, MODE_FWD, 3>(lb, slot + LY::S_K, slot + LY::S_Q, slot + LY::S_G,
                                                         slot + LY::S_BETA, ob, priv, L, scale, ksw, hook);
      }
      // K, Q of chunk s + 2 (and everything older) land before the barrier;
      // its V may stay in flight until the next one
      if (spread && c >= nch) { issue_q(cn); issue_v(cn); }
      if (s + 2 < nch && full(s + 2)) wait_vm<LY::DMA_V>();
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
hipError_t launch_t(const FwdParams &p, hipStream_t stream) {
  const size_t smem = Lay<DK>::TOTAL;
  auto kern = p.g ? fwd_bf16_kernel<DK, true, STORE_STATES, WRITE_O>
                  : fwd_bf16_kernel<DK, false, STORE_STATES, WRITE_O>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.N * p.H * p.ntiles;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(FWD_THREADS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t fwd_smem_bytes(int dtype, int DK) {
  if (dtype == 1) return DK == 64 ? Lay<64>::TOTAL : Lay<128>::TOTAL;
  return fwd_ref_smem_bytes(dtype, DK);
}

hipError_t launch_fwd(const FwdParams &p, int dtype, int DK, bool store_states, bool write_o,
                      hipStream_t stream) {
  if (dtype != 1) return launch_fwd_ref(p, dtype, DK, store_states, write_o, stream);
#define DN_FWD_CASE(D)                                                   \
  if (store_states)                                                      \
    return write_o ? launch_t<D, true, true>(p, stream)                  \
                   : launch_t<D, true, false>(p, stream);                \
  return write_o ? launch_t<D, false, true>(p, stream)                   \
                 : launch_t<D, false, false>(p, stream);
  if (DK == 64) { DN_FWD_CASE(64) }
  if (DK == 128) { DN_FWD_CASE(128) }
  return hipErrorInvalidValue;
#undef DN_FWD_CASE
}

}  // namespace dn
