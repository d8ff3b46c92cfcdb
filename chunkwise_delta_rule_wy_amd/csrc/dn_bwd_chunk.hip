// Chunk-parallel gradients of the chunkwise (gated) delta rule for gfx950,
// bf16 inputs: one workgroup (8 waves) per (chunk, head) with all d_v
// columns, so that products contracting over d_v need no cross-workgroup sums.
//
// Inputs per chunk: K, Q, V, dO, beta, g, the state entering the chunk h and
// the gradient w.r.t. the state leaving it dh (both bf16, stored transposed:
// S = h^T and dS = dh^T, [d_v][d_k]).  With the chunk quantities of the
// forward kernel (M = strictLower((K K^T) * Gamma), A = diag(beta) M,
// R = (I + A)^-1, T = R diag(beta), P = (Q K^T) * Gamma, w_r = exp(b_63 - b_r)):
//
//   X   = V - diag(gamma) K h              V' = T X
//   dV' = P^T dO + diag(w) K dh            Y  = R^T dV',  dX = diag(beta) Y
//   dv  = dX
//   dP  = lower(dO V'^T)                   dA = -strictLower(Y V'^T)
//   dq  = diag(gamma) dO h^T + (dP * Gamma) K
//   dk  = (dP * Gamma)^T Q - diag(gamma) dX h^T + diag(w) V' dh^T + F K + F^T K,
//         F = diag(beta) dA * Gamma
//   dbeta = rowsum(X * Y) + rowsum(dA * M)
//   db_r  = gamma_r q_r . (dO h^T)_r - gamma_r k_r . (dX h^T)_r
//           - w_r k_r . (V' dh^T)_r + rowsum(E)_r - colsum(E)_r
//           + [r = 63] (sum_i w_i k_i . (V' dh^T)_i + gamma_63 <dh, h>),
//         E = dP * P + dA * A,  dg = reverse cumsum of db inside the chunk.
//
// These are the derivatives of the chunk form (an exact refactoring of the
// token recurrence).  The UT inverse is never formed beyond its diagonal
// blocks: V' and Y come from block forward / backward substitution over the
// four 16-token blocks, and dA = -strictLower(R^T dT R^T) with dT = dV' X^T
// equals -strictLower(Y V'^T), so no full R is needed; likewise
// sum_r R_rj dT_rj = rowsum(X * Y)_j.  This follows the backward pass by
// recomputation of "Parallelizing Linear Transformers with the Delta Rule
// over Sequence Length" (page 1, answer Q2) with the UT form of the Gated
// DeltaNet review thread (review 2).
//
// 32-token chunks (template argument NB = 2 blocks of 16 tokens instead of
// 4) use the same organisation on the first half of every token-indexed
// buffer; the row waves of tokens 32 .. 63 then only issue their share of the
// tile loads.
//
// Organisation.  d_v is walked in 32-column tiles through a two-stage
// pipeline; in step s
//   column waves 0..3  take tile s.  Wave 2c ("F") owns tile columns
//                      16c .. 16c + 15 for X = V - gamma K h and
//                      V' = R diag(beta) X; wave 2c + 1 ("B") the same
//                      columns for dV' = w K dh + P^T dO, Y = R^T dV', dX and
//                      dv.  They hand V'^T and Y^T to the row waves through
//                      one of two LDS buffers.
//   row waves 4..7     take tile s - 1: each owns 16 token rows of the
//                      products contracting over the tile's columns (dP, dA,
//                      dO h^T, Y h^T, V' dh^T), accumulated in registers over
//                      all tiles, and issues the direct loads of tile s + 2.
// R = (I + A)^-1 is formed once per chunk, in 16 x 16 blocks: the prep
// inverts the diagonal blocks by substitution, then three row waves compute
// the blocks below the diagonal (one block column each, by the block
// recurrence of the inverse of a lower-triangular matrix), so that V' and Y
// are ten independent block products per tile instead of a chain of block
// substitutions.  Wave w and wave w + 4 share a SIMD.  Each role runs its own loop with one barrier per step; the roles
// keep their own registers (a wave's state never holds another role's).
// Tiles arrive two steps ahead in a ring of four LDS buffers.  After the last
// step the row waves form dPG = dP * Gamma and F and write them transposed;
// then the row waves compute dq and their share of dk, the column waves
// dPG^T Q + F^T K, and wave 0 dbeta and dg.
#include "dn_wy.h"

namespace dn {
namespace {

using namespace wy;

constexpr int BW_THREADS = 512;  // eight waves
constexpr int TC = 32;           // d_v columns per tile

// swizzles of this kernel's tiles (linear in the row bits)
template <int DK>
__device__ __forceinline__ int swz_s(int r) {  // K, Q, S, dS (rows of 2 d_k bytes)
  if constexpr (DK == 128) return ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3);
  else return (r & 2) | (((r >> 3) & 1) << 2);
}
__device__ __forceinline__ int swz_v32(int r) { return ((r >> 2) & 1) << 1; }  // V tile, 64-byte rows
__device__ __forceinline__ int swz_d32(int r) { return ((r >> 3) & 1) << 1; }  // dO tile, 64-byte rows
__device__ __forceinline__ int swz_xn(int r) { return (((r >> 2) & 1) << 1) ^ (((r >> 3) & 1) * 3); }  // V', Y hand-over

template <int DK>
struct BLay {
  static constexpr int RB = 2 * DK, KB = DK / 32, MT = DK / 16;
  static constexpr int KQ = CH * RB;           // K, Q tile
  static constexpr int O_K = 0, O_Q = KQ;
  using RS = Res<MODE_CHUNK>;
  static constexpr int O_RES = 2 * KQ;         // prep results (the gate table holds beta too)
  static constexpr int O_BETA = O_RES + RS::BYTES;  // beta (0 past the end)
  static constexpr int O_X = O_BETA + 256;     // two hand-over buffers; the prep scratch and g, beta before
  static constexpr int XB = 8192;              // V' then Y, [64 tokens][32 columns] bf16 each
  static constexpr int O_XG = O_X + 4 * PRIV_BYTES;  // direct-load targets of g and beta
  static constexpr int O_XB = O_XG + 256;
  static constexpr int O_T = O_X + 2 * XB;     // ring of tile buffers: V, dO (64 x 32), S, dS (32 x d_k)
  static constexpr int ST = TC * RB;
  static constexpr int T_V = 0, T_DO = 4096, T_S = 8192, T_DS = 8192 + ST;
  static constexpr int TB = 8192 + 2 * ST;
  static constexpr int NBUF = 4;
  static constexpr int TOTAL = O_T + NBUF * TB;
  static constexpr int DMA_T = TB / 16 / 256;   // direct loads per row-wave lane per tile
  static constexpr int DMA_KQ = KQ / 16 / 512;  // per lane and matrix
  static constexpr int DMA_S = ST / 16 / 256;   // of S (and of dS) per row-wave lane
  // final phase, in the tile ring
  static constexpr int O_FIN = O_T;             // dPG^T, F^T (P^T layout)
  static constexpr int O_RED = O_T + 16384;     // reductions
  static constexpr int O_DKX = O_T + 20480;     // column waves' share of dk, fp32
  static_assert(O_XB + 256 <= O_X + 2 * XB, "scratch fits");
  static_assert(O_DKX + 4 * MT * 64 * 16 <= TOTAL, "final phase fits");
  static_assert(DMA_T == 2 + 2 * DMA_S, "tile = V, dO, S, dS");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int DK>
struct BwdKsw {
  uint32_t frag_base;
  __device__ __forceinline__ uint32_t frag(int t, int kb) const { return (frag_base ^ (64 * kb)) + 16 * t * 2 * DK; }
};


// Epilogues of the chunk-gradient kernel: the plain gradients; EPI_PRO folds
// the input prologue's backward into the stores (the gradients of q_in, k_in,
// b_in, x_in replace those of q, k, beta, g); EPI_LH folds in the Longhorn
// step size (beta holds eps = beta_raw / (1 + beta_raw |k|^2): dbeta becomes
// the gradient of beta_raw, deps (eps / beta_raw)^2, and dk gains
// -2 eps^2 deps k, the step size's dependence on the key).
enum : int { EPI_PLAIN = 0, EPI_PRO = 1, EPI_LH = 2 };

template <int DK, bool GATED, int EPI, int NB>
__global__ __launch_bounds__(BW_THREADS, 1) void bwd_chunk_kernel(BwdParams p) {
  constexpr bool PRO = EPI == EPI_PRO, LH = EPI == EPI_LH;
  using LY = BLay<DK>;
  using RS = Res<MODE_CHUNK>;
  constexpr int KB = LY::KB, MT = LY::MT, RB = LY::RB;
  // NB 16-token blocks per chunk: 4 (64-token chunks) or 2 (32-token chunks,
  // which use the first half of every token-indexed buffer and leave every
  // block with an index >= NB out)
  static_assert(NB == 4 || NB == 2, "64- or 32-token chunks");
  constexpr int CHN = 16 * NB;  // tokens per chunk
  constexpr int NKB = NB / 2;   // 32-token contraction blocks
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const uint32_t sb = (uint32_t)(uintptr_t)(lds_ptr<unsigned char>)smem_raw;

  const int h = blockIdx.x % p.H, cg = blockIdx.x / p.H;
  int n_seq, c;
  if (p.chunk_seq) {
    n_seq = p.chunk_seq[cg];
    if (n_seq < 0) return;
    c = cg - p.chunk_base[n_seq];
  } else {
    n_seq = cg / p.NC;
    c = cg % p.NC;
    if (n_seq >= p.N) return;
  }
  const SeqInfo si = seq_info(p.cu, n_seq, p.T);
  if (c * CHN >= si.len) return;
  const int L = min(CHN, si.len - c * CHN);
  const bool full = L == CHN;
  const int H = p.H, DV = p.DV, ntiles = p.DV / TC;
  const size_t row0 = (size_t)si.b * p.T + si.t0 + (size_t)c * CHN;  // global row of the chunk start
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = lane_id(), n = l & 15, g = l >> 4, e4 = (l >> 2) & 3, q4 = l & 3;

  // ---- lane bases
  const int sn = swz_s<DK>(n);
  const uint32_t lb_frag = n * RB + 16 * (g ^ (sn & 3)) + 64 * (sn >> 2);  // K/Q/S frag, row n
  uint32_t lb_str[2];  // S-like transposed reads, rows 8g + 4hh + e, columns 16mt + 4q
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g + 4 * hh + e4, s = swz_s<DK>(r);
    lb_str[hh] = r * RB + 8 * q4 + 32 * (s >> 1);
  }
  // hand-over buffers (V', Y as [token][column], 64-byte rows): fragment
  // reads, lane (n, g): row 16j + n, columns 8g .. 8g + 7 at 1024 j + lb_xf
  const uint32_t lb_xf = n * 64 + 16 * (g ^ swz_xn(n));
  const uint32_t lb_m = 32 * n + ((8 * g) ^ (16 * ((n >> 3) & 1)));           // 16x16 block row reads
  const int rb4 = 4 * g + e4;
  const uint32_t lb_btr = 32 * rb4 + ((8 * q4) ^ (16 * ((rb4 >> 3) & 1)));  // 16x16 block transposed reads
  Bases lb = {};
  lb.m = lb_m;
  lb.btr = lb_btr;

  const uint32_t ob = sb + LY::O_RES, cgt = ob + RS::O_CG;
  auto tbuf = [&](int j) { return sb + LY::O_T + (uint32_t)(j % LY::NBUF) * LY::TB; };
  auto xbuf = [&](int j) { return sb + LY::O_X + (uint32_t)(j & 1) * LY::XB; };
  auto gam4 = [&](int i) { return GATED ? ld<f32x4>(cgt + CG_GS + 4 * (16 * i + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f}; };
  auto w4 = [&](int i) { return GATED ? ld<f32x4>(cgt + CG_WS + 4 * (16 * i + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f}; };
  auto bet4 = [&](int i) { return ld<f32x4>(sb + LY::O_BETA + 4 * (16 * i + 4 * g)); };

  // ---- direct loads
  const char *gk = static_cast<const char *>(p.k);
  const char *gq = static_cast<const char *>(p.q);
  const char *gv = static_cast<const char *>(p.v);
  const char *gdo = static_cast<const char *>(p.dO);
  const size_t rowoff = (row0 * H + h);
  const size_t sbase_g = ((size_t)cg * H + h) * (size_t)DV;  // row of S / dS for d_v column 0
  auto issue_kq = [&]() {  // every wave
#pragma unroll
    for (int i = 0; i < LY::DMA_KQ; ++i) {
      const int u = 512 * i + 64 * w + l;
      const int r = u / (DK / 8), pos = (u % (DK / 8)) ^ swz_s<DK>(r);
      const uint32_t dst = sb + 16 * (512 * i + 64 * w);
      if (r < L) {
        dma16(gk + (rowoff + (size_t)r * H) * RB + 16 * pos, dst + LY::O_K);
        dma16(gq + (rowoff + (size_t)r * H) * RB + 16 * pos, dst + LY::O_Q);
      }
    }
    if (l < L) {
      if (w == 0 && GATED) dma4(reinterpret_cast<const char *>(p.g + rowoff) + 4u * l * H, sb + LY::O_XG);
      if (w == 1) dma4(reinterpret_cast<const char *>(p.beta + rowoff) + 4u * l * H, sb + LY::O_XB);
    }
  };
  // row waves' per-lane byte offsets of the tile loads (base + offset form)
  const int rw = w - 4;
  uint32_t vo_v, vo_d, vo_s[LY::DMA_S];
  {
    const int u = 64 * rw + l, r = u >> 2, pos = u & 3;  // V, dO: 64 rows x 64 bytes
    vo_v = (uint32_t)r * (uint32_t)(H * DV * 2) + 16u * (pos ^ swz_v32(r));
    vo_d = (uint32_t)r * (uint32_t)(H * DV * 2) + 16u * (pos ^ swz_d32(r));
#pragma unroll
    for (int i = 0; i < LY::DMA_S; ++i) {  // S, dS: 32 rows x RB bytes
      const int us = 256 * i + 64 * rw + l;
      const int rs = us / (DK / 8), ps = (us % (DK / 8)) ^ swz_s<DK>(rs);
      vo_s[i] = (uint32_t)(rs * RB + 16 * ps);
    }
  }
  const bool vrow = (64 * rw + l) / 4 < L;
  // loads per tile of this row wave in a full chunk: V, dO and its share of S,
  // dS; with 32-token chunks the waves of rows 32 .. 63 load S and dS only
  const bool vwave = NB == 4 || rw < NB;
  auto wait_tiles = [&](auto n_c) {  // at most n tiles of this wave's loads outstanding
    constexpr int NT = decltype(n_c)::value;
    if (vwave) wait_vm<NT * LY::DMA_T>();
    else wait_vm<NT * 2 * LY::DMA_S>();
  };
  auto issue_tile = [&](int j) {  // row waves: 64 lanes x DMA_T units of 16 bytes each
    const uint32_t tb = tbuf(j);
    const int dv0 = TC * j;
    if (vrow) {
      dma16s(gv + (rowoff * DV + dv0) * 2, vo_v, tb + LY::T_V + 16 * (64 * rw));
      dma16s(gdo + (rowoff * DV + dv0) * 2, vo_d, tb + LY::T_DO + 16 * (64 * rw));
    }
    const char *s0 = reinterpret_cast<const char *>(p.states + (sbase_g + dv0) * DK);
    const char *d0 = reinterpret_cast<const char *>(p.dstates + (sbase_g + dv0) * DK);
#pragma unroll
    for (int i = 0; i < LY::DMA_S; ++i) {
      dma16s(s0, vo_s[i], tb + LY::T_S + 16 * (256 * i + 64 * rw));
      dma16s(d0, vo_s[i], tb + LY::T_DS + 16 * (256 * i + 64 * rw));
    }
  };

  // ---- prologue: rows past the end of the chunk are zero
  if (!full) {
    for (int i = L * RB / 16 + threadIdx.x; i < LY::KQ / 16; i += BW_THREADS) {
      st<f32x4>(sb + LY::O_K + 16 * i, zero4());
      st<f32x4>(sb + LY::O_Q + 16 * i, zero4());
    }
    for (int buf = 0; buf < LY::NBUF; ++buf)
      for (int i = L * 64 / 16 + threadIdx.x; i < 4096 / 16; i += BW_THREADS) {
        st<f32x4>(sb + LY::O_T + buf * LY::TB + LY::T_V + 16 * i, zero4());
        st<f32x4>(sb + LY::O_T + buf * LY::TB + LY::T_DO + 16 * i, zero4());
      }
  }
  // P^T above the diagonal stays zero
  for (int i = threadIdx.x; i < RS::P_BYTES / 16; i += BW_THREADS) st<f32x4>(ob + RS::O_P + 16 * i, zero4());
  issue_kq();
  if (w >= 4) {
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    // K, Q, g, beta land before the prep; the tiles stay in flight through it
    if (!full) wait_vm<0>();
    else if (ntiles > 1) wait_tiles(I2{});
    else wait_tiles(I1{});
  } else {
    wait_vm<0>();
  }
  __syncthreads();

  // ---- prep of the chunk (M, P^T, R_ii, gates) by waves 0..3
  if (w < 4) {
    if (w == 1) st<float>(sb + LY::O_BETA + 4 * l, l < L ? ld<float>(sb + LY::O_XB + 4 * l) : 0.f);
    float dummy = 1.f;
    const BwdKsw<DK> ksw{lb_frag};
    const uint32_t priv = sb + LY::O_X + w * PRIV_BYTES;
    const uint32_t kba = sb + LY::O_K, qba = sb + LY::O_Q, ga = sb + LY::O_XG, ba = sb + LY::O_XB;
    if (w == 0) prep_chunk<DK, GATED, true, MODE_CHUNK, 0, NB>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else if (w == 1) prep_chunk<DK, GATED, true, MODE_CHUNK, 1, NB>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else if (w == 2) prep_chunk<DK, GATED, true, MODE_CHUNK, 2, NB>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else prep_chunk<DK, GATED, true, MODE_CHUNK, 3, NB>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
  }
  __syncthreads();

  // ---- the blocks of R = (I + A)^-1 below the diagonal, one block column per
  // wave (waves 4..6), from R_ii and -M (the prep's results):
  //   R_ij = R_ii diag(beta_i) sum_{m=j}^{i-1} (-M_im) R_mj,   i > j,
  // stored transposed (like R_ii^T) in the S part of the fourth tile buffer,
  // which the ring does not load before step 1 and then overwrites whole
  // (unlike its V and dO parts, whose rows past a partial chunk stay zero);
  // the column waves keep them in registers.
  const uint32_t rbuf = tbuf(3) + LY::T_S;
  static_assert(6 * 512 <= LY::ST, "R blocks fit in a state tile");
  auto rcol = [&](auto j_c) {  // straight-line per block column (MFMA results read without branches)
    constexpr int J = decltype(j_c)::value;
    bf16x4 rc[NB];  // R_mJ as B operands (lane (n, g): rows 4g .. 4g + 3 of column n)
    rc[J] = ld<bf16x4>(ob + RS::O_TT + 512 * J + lb_m);
#pragma unroll
    for (int i = J + 1; i < NB; ++i) {
      f32x4 z = zero4();
#pragma unroll
      for (int m = J; m < i; ++m) z = mma16(z, ld<bf16x4>(ob + RS::O_M + 512 * m_block(i, m) + lb_m), rc[m]);
      z = z * bet4(i);
      rc[i] = cvt4(mma16(zero4(), ld_tr(ob + RS::O_TT + 512 * i + lb_btr), cvt4(z)));
      st<bf16x4>(rbuf + 512 * m_block(i, J) + lb_m, rc[i]);
    }
    mfma_settle();
  };
  if (w == 4) rcol(I0{});
  else if constexpr (NB == 4) {
    if (w == 5) rcol(I1{});
    else if (w == 6) rcol(I2{});
  }
  // tile 0 lands before the pipeline starts; tile 1 may stay in flight
  if (w >= 4) {
    if (full && ntiles > 1) wait_tiles(I1{});
    else wait_vm<0>();
  }
  __syncthreads();

  const uint32_t red = sb + LY::O_RED, fin = sb + LY::O_FIN, dkx = sb + LY::O_DKX;

  if (w < 4) {
    // =========================== column waves ===========================
    const int cs = w >> 1;  // column set: tile columns 16cs .. 16cs + 15
    bf16x8 kf[NB][KB];      // K fragments, rows 16t + n
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int t = 0; t < NB; ++t) kf[t][kb] = ld<bf16x8>(sb + LY::O_K + (lb_frag ^ (64 * kb)) + 16 * t * RB);
    const uint32_t sfrag = (16 * cs) * RB;  // S / dS rows of the column set

    if ((w & 1) == 0) {
      // ------------------------------ F ------------------------------
      bf16x4 ra[NB * (NB + 1) / 2];  // R_im, m <= i, as A operands (transposed reads of the stored R^T blocks)
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int m = 0; m <= i; ++m)
          ra[i * (i + 1) / 2 + m] = ld_tr((m == i ? ob + RS::O_TT + 512 * i : rbuf + 512 * m_block(i, m)) + lb_btr);
      uint32_t lb_vtr, lb_ytr, lb_xw;
      {
        const int r = 4 * g + e4;  // V and Y transposed reads: rows 16t + 4g + e, columns 16cs + 4q
        lb_vtr = r * 64 + 16 * ((2 * cs + (q4 >> 1)) ^ swz_v32(r)) + 8 * (q4 & 1);
        lb_ytr = r * 64 + 16 * ((2 * cs + (q4 >> 1)) ^ swz_xn(r)) + 8 * (q4 & 1);
        // V' writes, lane (n, g): row 16i + n, columns 16cs + 4g .. + 3 at 1024 i + lb_xw
        lb_xw = n * 64 + 16 * ((2 * cs + (g >> 1)) ^ swz_xn(n)) + 8 * (g & 1);
      }
      f32x4 xp[NB], xy[NB];  // X of the previous tile; rowsum(X * Y) partials (rows 16i + 4g + e)
#pragma unroll
      for (int i = 0; i < NB; ++i) xp[i] = xy[i] = zero4();
      for (int s = 0; s <= ntiles; ++s) {
        if (s > 0) {  // rowsum(X * Y) of tile s - 1 (Y handed over by the B wave)
          const uint32_t yb = xbuf(s - 1) + 4096;
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            const bf16x4 yv = ld_tr(yb + 1024 * i + lb_ytr);
#pragma unroll
            for (int e = 0; e < 4; ++e) xy[i][e] += xp[i][e] * bf2f(yv[e]);
          }
        }
        if (s < ntiles) {
          const uint32_t tb = tbuf(s);
          bf16x8 hb[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) hb[kb] = ld<bf16x8>(tb + LY::T_S + sfrag + (lb_frag ^ (64 * kb)));
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            f32x4 yk = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) yk = mma32(yk, kf[t][kb], hb[kb]);
            const bf16x4 vr = ld_tr(tb + LY::T_V + 1024 * t + lb_vtr);
            const f32x4 gm = gam4(t);
#pragma unroll
            for (int e = 0; e < 4; ++e) xp[t][e] = bf2f(vr[e]) - gm[e] * yk[e];
          }
          // V' = R diag(beta) X, as V'_i^T = sum_{m<=i} (beta_m X_m)^T R_im^T so
          // that lane (n, g) holds columns 4g .. 4g + 3 of token 16i + n
          bf16x4 bx[NB];
#pragma unroll
          for (int m = 0; m < NB; ++m) bx[m] = cvt4(xp[m] * bet4(m));
          const uint32_t xv = xbuf(s);
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            f32x4 acc = zero4();
#pragma unroll
            for (int m = 0; m <= i; ++m) acc = mma16(acc, bx[m], ra[i * (i + 1) / 2 + m]);
            st<bf16x4>(xv + 1024 * i + lb_xw, cvt4(acc));
          }
        }
        mfma_settle();
        __syncthreads();
      }
      // rowsum(X * Y) of this wave's columns
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sm = row_sum16(xy[i][e]);
          if (n == 0) st<float>(red + 1024 + 256 * cs + 4 * (16 * i + 4 * g + e), sm);
        }
    } else {
      // ------------------------------ B ------------------------------
      bf16x8 ptf[6];        // P^T fragments (t, kb >= t / 2): (0,0) (0,1) (1,0) (1,1) (2,1) (3,1)
      bf16x4 rb[NB * (NB + 1) / 2];  // (R_mi)^T, m >= i, as A operands (rows of the stored R^T blocks), index m(m+1)/2 + i
      ptf[0] = ld<bf16x8>(ob + RS::O_P + pt_frag(0, 0, l));
      ptf[2] = ld<bf16x8>(ob + RS::O_P + pt_frag(1, 0, l));
      if constexpr (NB == 4) {
        ptf[1] = ld<bf16x8>(ob + RS::O_P + pt_frag(0, 1, l));
        ptf[3] = ld<bf16x8>(ob + RS::O_P + pt_frag(1, 1, l));
        ptf[4] = ld<bf16x8>(ob + RS::O_P + pt_frag(2, 1, l));
        ptf[5] = ld<bf16x8>(ob + RS::O_P + pt_frag(3, 1, l));
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i <= m; ++i)
          rb[m * (m + 1) / 2 + i] = ld<bf16x4>((m == i ? ob + RS::O_TT + 512 * i : rbuf + 512 * m_block(m, i)) + lb_m);
      // Y writes, lane (n, g): row 16i + n, columns 16cs + 4g .. + 3 at 1024 i + lb_xw
      const uint32_t lb_xw = n * 64 + 16 * ((2 * cs + (g >> 1)) ^ swz_xn(n)) + 8 * (g & 1);
      uint32_t lb_dtr[2];  // dO transposed reads, rows 8g + 4hh + e (+ 32 kb), columns 16cs + 4q
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r = 8 * g + 4 * hh + e4;
        lb_dtr[hh] = r * 64 + 16 * ((2 * cs + (q4 >> 1)) ^ swz_d32(r)) + 8 * (q4 & 1);
      }
      for (int s = 0; s <= ntiles; ++s) {
        if (s < ntiles) {
          const uint32_t tb = tbuf(s);
          bf16x8 dhb[KB];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb) dhb[kb] = ld<bf16x8>(tb + LY::T_DS + sfrag + (lb_frag ^ (64 * kb)));
          f32x4 dvp[NB];
#pragma unroll
          for (int t = 0; t < NB; ++t) {
            f32x4 yd = zero4();
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) yd = mma32(yd, kf[t][kb], dhb[kb]);
            dvp[t] = w4(t) * yd;
          }
          // dV' += P^T dO (token blocks kb >= t / 2)
          bf16x8 dob[NKB];
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            dob[kb] = cat(ld_tr(tb + LY::T_DO + 2048 * kb + lb_dtr[0]), ld_tr(tb + LY::T_DO + 2048 * kb + lb_dtr[1]));
          if constexpr (NB == 4) {
            dvp[0] = mma32(mma32(dvp[0], ptf[0], dob[0]), ptf[1], dob[1]);
            dvp[1] = mma32(mma32(dvp[1], ptf[2], dob[0]), ptf[3], dob[1]);
            dvp[2] = mma32(dvp[2], ptf[4], dob[1]);
            dvp[3] = mma32(dvp[3], ptf[5], dob[1]);
          } else {
            dvp[0] = mma32(dvp[0], ptf[0], dob[0]);
            dvp[1] = mma32(dvp[1], ptf[2], dob[0]);
          }
          // Y = R^T dV', as Y_i^T = sum_{m>=i} dV'_m^T R_mi so that lane (n, g)
          // holds columns 4g .. 4g + 3 of token 16i + n;  dX = diag(beta) Y = dv
          bf16x4 db16[NB];
#pragma unroll
          for (int m = 0; m < NB; ++m) db16[m] = cvt4(dvp[m]);
          float *dvb = p.dv + (row0 * H + h) * (size_t)DV + TC * s + 16 * cs + 4 * g;  // + token row
          const uint32_t yb = xbuf(s) + 4096;
#pragma unroll
          for (int i = NB - 1; i >= 0; --i) {
            f32x4 acc = zero4();
#pragma unroll
            for (int m = NB - 1; m >= i; --m) acc = mma16(acc, db16[m], rb[m * (m + 1) / 2 + i]);
            st<bf16x4>(yb + 1024 * i + lb_xw, cvt4(acc));
            const int r = 16 * i + n;
            if (r < L)
              *reinterpret_cast<f32x4 *>(dvb + (uint32_t)(r * H * DV)) = acc * ld<float>(sb + LY::O_BETA + 4 * r);
          }
        }
        mfma_settle();
        __syncthreads();
      }
    }
    __syncthreads();  // dPG^T, F^T and the reductions are complete

    // dk (column part) of token rows 16w .. 16w + 15: dPG^T Q + F^T K
    if (w < NB) {
      bf16x8 pgt[NKB], ft[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pgt[kb] = ld<bf16x8>(fin + pt_frag(w, kb, l));
        ft[kb] = ld<bf16x8>(fin + 8192 + pt_frag(w, kb, l));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 dk = zero4();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint32_t a0 = 32 * kb * RB + (lb_str[0] ^ (32 * mt)), a1 = 32 * kb * RB + (lb_str[1] ^ (32 * mt));
          const bf16x8 kt = cat(ld_tr(sb + LY::O_K + a0), ld_tr(sb + LY::O_K + a1));
          const bf16x8 qt = cat(ld_tr(sb + LY::O_Q + a0), ld_tr(sb + LY::O_Q + a1));
          dk = mma32(dk, qt, pgt[kb]);  // (dPG^T Q + F^T K)^T: lane (n, g) row 16w + n, columns 16mt + 4g ..
          dk = mma32(dk, kt, ft[kb]);
        }
        st<f32x4>(dkx + 16 * ((w * MT + mt) * 64 + l), dk);
      }
    }
    // dbeta, db -> dg (reverse cumulative sum inside the chunk)
    if (w == 0) {
      const int r = l;
      float ce = 0.f;
#pragma unroll
      for (int ww = 0; ww < NB; ++ww) ce += ld<float>(red + 256 * ww + 4 * r);
      const float xyr = ld<float>(red + 1024 + 4 * r) + ld<float>(red + 1280 + 4 * r);
      // rows past a 32-token chunk hold no token (and reductions nothing wrote)
      float db = r < CHN ? ld<float>(red + 2048 + 4 * r) + ld<float>(red + 2816 + 4 * r) - ce : 0.f;
      if (r == CHN - 1) {
        float s3t = 0.f;
#pragma unroll
        for (int ww = 0; ww < NB; ++ww) s3t += ld<float>(red + 2560 + 4 * ww);
        const float g63 = GATED ? ld<float>(cgt + CG_GS + 4 * (CHN - 1)) : 1.f;
        db += s3t + g63 * ld<float>(red + 2576);
      }
      const float incl = wave_incl_scan(db);
      const float total = lane_val(incl, 63);
      if (r < L) {
        const size_t idx = (row0 + r) * H + h;
        const float dbeta = xyr + ld<float>(red + 2304 + 4 * r);
        const float dgr = total - incl + db;  // sum_{r' >= r} db_r'
        if constexpr (PRO) {
          // beta = sigmoid(b_in): db_in = dbeta beta (1 - beta); g = -c softplus(x_in):
          // dx_in = -c sigmoid(x_in) dg
          const float bt = ld<float>(sb + LY::O_BETA + 4 * r);
          p.dbeta[idx] = dbeta * bt * (1.f - bt);
          if (GATED) p.dg[idx] = -p.gate_scale * dgr / (1.f + expf(-p.x_in[idx]));
        } else if constexpr (LH) {
          // dbeta_raw = deps / (1 + beta_raw |k|^2)^2 = deps (eps / beta_raw)^2 (deps at beta_raw = 0);
          // deps goes to the row waves for the key term
          const float br = p.beta_raw[idx], ep = ld<float>(sb + LY::O_BETA + 4 * r);
          const float ratio = br != 0.f ? ep / br : 1.f;
          p.dbeta[idx] = dbeta * ratio * ratio;
          st<float>(red + 3072 + 4 * r, dbeta);
          if (GATED) p.dg[idx] = dgr;
        } else {
          p.dbeta[idx] = dbeta;
          if (GATED) p.dg[idx] = dgr;
        }
      }
    }
    mfma_settle();
    __syncthreads();  // the column part of dk is in LDS
  } else {
    // ============================= row waves =============================
    const int rho = w == 4 ? 3 : w == 5 ? 0 : w == 6 ? 2 : 1;  // token rows 16rho .. 16rho + 15
    // with 32-token chunks the waves of rows 32 .. 63 only issue tile loads
    const bool active = NB == 4 || rho < NB;
    const bool hdh_wave = rho == 0;
    const uint32_t lb_dfrag = (16 * rho + n) * 64 + 16 * (g ^ swz_d32(n));  // dO frag, row 16rho + n
    // dP, dA: lane (n, g) holds rows 16rho + 4g + e, column 16jt + n;
    // dq1 = dO h^T, dk1 = Y h^T, dk2 = V' dh^T: row 16rho + n, columns 16mt + 4g + e
    f32x4 dP[NB], dAc[NB], dq1[MT], dk1[MT], dk2[MT];
#pragma unroll
    for (int t = 0; t < NB; ++t) dP[t] = dAc[t] = zero4();
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dq1[mt] = dk1[mt] = dk2[mt] = zero4();
    float hdh = 0.f;  // <dh, h> partial (one wave)
    for (int s = 0; s <= ntiles; ++s) {
      if (s + 2 < ntiles) issue_tile(s + 2);
      if (s > 0 && active) {
        const int j = s - 1;
        const uint32_t tb = tbuf(j), xv = xbuf(j), xyb = xbuf(j) + 4096;
        const bf16x8 dof = ld<bf16x8>(tb + LY::T_DO + lb_dfrag);
        const bf16x8 yf = ld<bf16x8>(xyb + 1024 * rho + lb_xf);
        // every token block: the blocks above the diagonal (jt > rho) are masked in the final phase
        bf16x8 vf;
#pragma unroll
        for (int jt = 0; jt < NB; ++jt) {
          const bf16x8 vt = ld<bf16x8>(xv + 1024 * jt + lb_xf);
          if (jt == rho) vf = vt;
          dP[jt] = mma32(dP[jt], dof, vt);
          dAc[jt] = mma32(dAc[jt], yf, vt);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint32_t a0 = lb_str[0] ^ (32 * mt), a1 = lb_str[1] ^ (32 * mt);
          const bf16x8 sf = cat(ld_tr(tb + LY::T_S + a0), ld_tr(tb + LY::T_S + a1));
          const bf16x8 dsf = cat(ld_tr(tb + LY::T_DS + a0), ld_tr(tb + LY::T_DS + a1));
          dq1[mt] = mma32(dq1[mt], sf, dof);
          dk1[mt] = mma32(dk1[mt], sf, yf);
          dk2[mt] = mma32(dk2[mt], dsf, vf);
          if (hdh_wave) hdh = dot8(sf, dsf, hdh);
        }
      }
      // tile s + 1 (and everything older) lands before the barrier; tile s + 2 may stay in flight
      if (s + 2 < ntiles && full) wait_tiles(I1{});
      else wait_vm<0>();
      mfma_settle();
      __syncthreads();
    }

    // ---- final phase (row wave rho: rows r = 16rho + 4g + e).  With 32-token
    // chunks the waves of rows 32 .. 63 run the next part too: their results
    // land in LDS that nothing reads (columns 32 .. 63 of dPG^T and F^T,
    // reductions of rows past the chunk, which wave 0 leaves out).
    const f32x4 bet_r = bet4(rho);
    float *const dqb = p.dq + ((row0 + 16 * rho) * H + h) * (size_t)DK;  // rows of this block (wave-uniform)
    float *const dkb = p.dk + ((row0 + 16 * rho) * H + h) * (size_t)DK;
    const f32x4 bl_r = GATED ? ld<f32x4>(cgt + CG_BL + 4 * (16 * rho + 4 * g)) : zero4();
    f32x4 erow = zero4(), dbr = zero4();
#pragma unroll
    for (int jt = 0; jt < NB; ++jt) {
      f32x4 dpg = zero4(), f = zero4();
      float ce = 0.f;
      if (jt <= rho) {
        const int jj = 16 * jt + n;
        const float blj = GATED ? ld<float>(cgt + CG_BL + 4 * jj) : 0.f;
        const bf16x4 pv = ld<bf16x4>(ob + RS::O_P + pt_quad(jt, rho, l));  // P[r][j]
        f32x4 mv;                                                          // M[r][j]
        if (jt < rho) {
          const bf16x4 mm = ld_tr(ob + RS::O_M + 512 * m_block(rho, jt) + lb_btr);
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = -bf2f(mm[e]);
        } else {
          const bf16x4 mm = ld<bf16x4>(ob + RS::O_M + 512 * (6 + rho) + lb_m);
#pragma unroll
          for (int e = 0; e < 4; ++e) mv[e] = bf2f(mm[e]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * rho + 4 * g + e;
          const float gm = GATED ? fexp2(jj <= r ? bl_r[e] - blj : 0.f) : 1.f;
          dpg[e] = (jj <= r) ? dP[jt][e] * gm : 0.f;
          const float da = (jj < r) ? -dAc[jt][e] : 0.f;
          f[e] = da * gm * bet_r[e];
          dbr[e] += da * mv[e];
          const float ev = dP[jt][e] * bf2f(pv[e]) + da * bet_r[e] * mv[e];
          erow[e] += ev;
          ce += ev;
        }
      }
      st<bf16x4>(fin + pt_quad(jt, rho, l), cvt4(dpg));
      st<bf16x4>(fin + 8192 + pt_quad(jt, rho, l), cvt4(f));
      ce = cross_row_sum(ce);
      if (g == 0) st<float>(red + 256 * rho + 4 * (16 * jt + n), ce);  // colsum(E) of these rows
    }
    // row terms: gamma_r q_r . DQ_r - gamma_r beta_r k_r . DY_r - w_r k_r . DH_r
    // (lane (n, g): token row r = 16rho + n, d_k columns 16mt + 4g .. + 3)
    const int rr = 16 * rho + n;
    const float gam_n = GATED ? ld<float>(cgt + CG_GS + 4 * rr) : 1.f;
    const float w_n = GATED ? ld<float>(cgt + CG_WS + 4 * rr) : 1.f;
    const float bet_n = ld<float>(sb + LY::O_BETA + 4 * rr);
    const uint32_t lb_qr = rr * RB + 8 * (g & 1);  // Q, K row rr, columns 16mt + 4g: + 16 ((2mt + g/2) ^ swz)
    const int sq = swz_s<DK>(n);
    float rowq = 0.f, rowk = 0.f, s3 = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint32_t a = lb_qr + 16 * ((2 * mt + (g >> 1)) ^ sq);
      const bf16x4 qv = ld<bf16x4>(sb + LY::O_Q + a);
      const bf16x4 kv = ld<bf16x4>(sb + LY::O_K + a);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rowq += bf2f(qv[e]) * dq1[mt][e];
        rowk += bf2f(kv[e]) * (bet_n * gam_n * dk1[mt][e] + w_n * dk2[mt][e]);
        s3 += bf2f(kv[e]) * dk2[mt][e];
      }
    }
    const float rt = cross_row_sum(gam_n * rowq - rowk);  // over the lane groups: all of d_k
    s3 = wave_sum(w_n * s3);
    if (g == 0) st<float>(red + 2048 + 4 * rr, rt);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float er = row_sum16(erow[e]);
      const float db = row_sum16(dbr[e]);
      if (n == 0) {
        st<float>(red + 2816 + 4 * (16 * rho + 4 * g + e), er);
        st<float>(red + 2304 + 4 * (16 * rho + 4 * g + e), db);
      }
    }
    if (l == 0) st<float>(red + 2560 + 4 * rho, s3);
    if (hdh_wave) {
      hdh = wave_sum(hdh);
      if (l == 0) st<float>(red + 2576, hdh);
    }
    mfma_settle();
    __syncthreads();  // dPG^T, F^T and the reductions are complete

    // Input prologue (PRO): q = q_in / |q_in| (likewise k) has the gradient
    // dq_in = (dq - q_in (q_in . dq) / |q_in|^2) / |q_in| (0 for a zero row).
    // The lane's 32 values of q_in and k_in (row rr, columns 16mt + 4g ..) are
    // loaded here, ahead of use; dq and dk stay in registers until |q_in|^2 and
    // q_in . dq are summed over the row's four lanes.  Rows past the chunk read
    // the chunk's first row (their results are not stored).
    bf16x4 xq[MT], xk[MT];  // unused (and removed by the compiler) without PRO
    if constexpr (PRO) {
      const size_t xrow = ((row0 + (rr < L ? rr : 0)) * H + h) * (size_t)DK + 4 * g;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        xq[mt] = *reinterpret_cast<const bf16x4 *>(static_cast<const bf16 *>(p.q_in) + xrow + 16 * mt);
        xk[mt] = *reinterpret_cast<const bf16x4 *>(static_cast<const bf16 *>(p.k_in) + xrow + 16 * mt);
      }
    }
    // (d - x (x . d) / |x|^2) / |x| over the row, in place
    auto pro_norm = [&](f32x4 (&d)[MT], const bf16x4 (&x)[MT]) {
      float sq = 0.f, pd = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xv = bf2f(x[mt][e]);
          sq += xv * xv;
          pd += xv * d[mt][e];
        }
      sq = cross_row_sum(sq);
      pd = cross_row_sum(pd);
      const float inv = sq > 0.f ? 1.f / sqrtf(sq) : 0.f, c = pd * inv * inv;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) d[mt][e] = (d[mt][e] - bf2f(x[mt][e]) * c) * inv;
    };
    // dq = diag(gamma) dO h^T + dPG K ;  dk (row part) = diag(w) V' dh^T - diag(gamma beta) Y h^T + F K,
    // as dq^T = gamma dq1^T + K^T dPG^T (and likewise dk): lane (n, g) holds row r = 16rho + n,
    // columns 16mt + 4g .. + 3, written as one 16-byte store
    f32x4 dkr[MT], dqv[MT];  // dqv: PRO only
    if (active) {
      bf16x8 pgr[NKB], fr[NKB];  // B operands: rows r of dPG and F, read transposed from dPG^T, F^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int r0 = 32 * kb + 8 * g + e4, r1 = r0 + 4;  // dPG^T rows j
        const int cc = 16 * rho + 4 * q4;                   // columns r
        const uint32_t a0 = 128 * r0 + 16 * ((cc / 8) ^ swz_p128(r0 & 15)) + 8 * ((cc % 8) / 4);
        const uint32_t a1 = 128 * r1 + 16 * ((cc / 8) ^ swz_p128(r1 & 15)) + 8 * ((cc % 8) / 4);
        pgr[kb] = cat(ld_tr(fin + a0), ld_tr(fin + a1));
        fr[kb] = cat(ld_tr(fin + 8192 + a0), ld_tr(fin + 8192 + a1));
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        f32x4 dq = gam_n * dq1[mt];
        f32x4 dk = w_n * dk2[mt] - (gam_n * bet_n) * dk1[mt];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const uint32_t a0 = 32 * kb * RB + (lb_str[0] ^ (32 * mt)), a1 = 32 * kb * RB + (lb_str[1] ^ (32 * mt));
          const bf16x8 kt = cat(ld_tr(sb + LY::O_K + a0), ld_tr(sb + LY::O_K + a1));
          dq = mma32(dq, kt, pgr[kb]);
          dk = mma32(dk, kt, fr[kb]);
        }
        dkr[mt] = dk;
        if constexpr (PRO) dqv[mt] = dq;
        else if (rr < L) *reinterpret_cast<f32x4 *>(dqb + (uint32_t)(n * H * DK + 16 * mt + 4 * g)) = dq;
      }
    }
    if constexpr (PRO) {
      if (active) {
      mfma_settle();
      pro_norm(dqv, xq);
      if (rr < L) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(dqb + (uint32_t)(n * H * DK + 16 * mt + 4 * g)) = dqv[mt];
      }
    }
    }
    mfma_settle();
    __syncthreads();  // the column part of dk is in LDS
    if (!active) {
    } else if constexpr (LH) {
      // dk += -2 eps^2 deps k (row rr; k from the chunk's K tile, columns 16mt + 4g ..)
      const float ep = ld<float>(sb + LY::O_BETA + 4 * rr);
      const float c = -2.f * ep * ep * (rr < L ? ld<float>(red + 3072 + 4 * rr) : 0.f);
      const int sk = swz_s<DK>(n);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x4 kv = ld<bf16x4>(sb + LY::O_K + rr * RB + 8 * (g & 1) + 16 * ((2 * mt + (g >> 1)) ^ sk));
        f32x4 dk = dkr[mt] + ld<f32x4>(dkx + 16 * ((rho * MT + mt) * 64 + l));
#pragma unroll
        for (int e = 0; e < 4; ++e) dk[e] += c * bf2f(kv[e]);
        if (rr < L) *reinterpret_cast<f32x4 *>(dkb + (uint32_t)(n * H * DK + 16 * mt + 4 * g)) = dk;
      }
    } else if constexpr (PRO) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) dkr[mt] = dkr[mt] + ld<f32x4>(dkx + 16 * ((rho * MT + mt) * 64 + l));
      pro_norm(dkr, xk);
      if (rr < L) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) *reinterpret_cast<f32x4 *>(dkb + (uint32_t)(n * H * DK + 16 * mt + 4 * g)) = dkr[mt];
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const f32x4 dk = dkr[mt] + ld<f32x4>(dkx + 16 * ((rho * MT + mt) * 64 + l));
        if (rr < L) *reinterpret_cast<f32x4 *>(dkb + (uint32_t)(n * H * DK + 16 * mt + 4 * g)) = dk;
      }
    }
  }
}

template <int DK>
hipError_t launch_t(const BwdParams &p, hipStream_t stream) {
  const size_t smem = BLay<DK>::TOTAL;
  // 32-token chunks: the plain gradients only
  if (p.chunk == 32 && (p.q_in || p.beta_raw)) return hipErrorInvalidValue;
  auto kern = p.chunk == 32  ? (p.g ? bwd_chunk_kernel<DK, true, EPI_PLAIN, 2> : bwd_chunk_kernel<DK, false, EPI_PLAIN, 2>)
              : p.q_in       ? (p.g ? bwd_chunk_kernel<DK, true, EPI_PRO, 4> : bwd_chunk_kernel<DK, false, EPI_PRO, 4>)
              : p.beta_raw ? (p.g ? bwd_chunk_kernel<DK, true, EPI_LH, 4> : bwd_chunk_kernel<DK, false, EPI_LH, 4>)
                           : (p.g ? bwd_chunk_kernel<DK, true, EPI_PLAIN, 4> : bwd_chunk_kernel<DK, false, EPI_PLAIN, 4>);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.total_chunks * p.H;
  if (grid == 0) return hipSuccess;
  if (p.DV % TC != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(BW_THREADS), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_chunk(const BwdParams &p, int DK, hipStream_t stream) {
  if (DK == 64) return launch_t<64>(p, stream);
  if (DK == 128) return launch_t<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dn
