// Chunk-parallel gradients of the chunkwise (gated) delta rule for gfx950,
// bf16 inputs: one workgroup (4 waves) per (chunk, head) with all d_v
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
// Per 64-wide d_v tile, wave w first owns columns 16w .. 16w + 15 (X, V',
// dV', Y, dv) and hands V'^T and Y^T to the others through LDS; then it owns
// token rows 16w .. 16w + 15 of the products contracting over the tile's d_v
// columns (dP, dA, dO h^T, Y h^T, V' dh^T), accumulated in registers over the
// tiles.  The tiles' V, dO, S and dS arrive by direct loads, one tile ahead.
#include "dn_wy.h"

namespace dn {
namespace {

using namespace wy;

// swizzles of this kernel's tiles (linear in the row bits, bit 0 never set)
template <int DK>
__device__ __forceinline__ int swz_s(int r) {  // K, Q, S, dS (rows of 2 d_k bytes)
  if constexpr (DK == 128) return ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3);
  else return (r & 2) | (((r >> 3) & 1) << 2);
}
__device__ __forceinline__ int swz_d(int r) { return (r & 2) | (((r >> 3) & 1) << 2); }          // dO
__device__ __forceinline__ int swz_x(int r) { return (((r >> 1) & 1) << 1) | ((r >> 2) & 1) | (((r >> 3) & 1) << 2); }  // V'^T, Y^T

template <int DK>
struct BLay {
  static constexpr int RB = 2 * DK, KB = DK / 32, MT = DK / 16;
  static constexpr int KQ = CH * RB;          // K, Q tile
  static constexpr int ST = CH * RB;          // S or dS tile (64 d_v rows)
  static constexpr int O_K = 0, O_Q = KQ;
  using RS = Res<MODE_CHUNK>;
  static constexpr int O_RES = 2 * KQ;         // prep results (the gate table holds beta too)
  static constexpr int O_BETA = O_RES + RS::BYTES;  // beta (0 past the end)
  static constexpr int O_X = O_BETA + 256;          // V'^T, Y^T; the prep scratch and g, beta before
  static constexpr int X_BYTES = 16384;
  static constexpr int O_XG = O_X + 4 * PRIV_BYTES;  // direct-load targets of g and beta
  static constexpr int O_XB = O_XG + 256;
  static constexpr int O_T = O_X + X_BYTES;    // two tile buffers: V, dO, S, dS
  static constexpr int T_V = 0, T_DO = 8192, T_S = 16384, T_DS = 16384 + ST;
  static constexpr int TB = 16384 + 2 * ST;
  static constexpr int TOTAL = O_T + 2 * TB;
  static constexpr int DMA_KQ = KQ / 4096, DMA_S = ST / 4096;  // direct loads per wave
  static_assert(O_XB + 256 <= O_X + X_BYTES, "scratch fits");
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
};

template <int DK>
struct BwdKsw {
  uint32_t frag_base;
  __device__ __forceinline__ uint32_t frag(int t, int kb) const { return (frag_base ^ (64 * kb)) + 16 * t * 2 * DK; }
};

// sum over the 16 lanes of a row of 16 (same lane group)
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}
// sum over the 4 lane groups (same column n)
__device__ __forceinline__ float sum4g(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

template <int DK, bool GATED>
__global__ __launch_bounds__(NTHR, 1) void bwd_chunk_kernel(BwdParams p) {
  using LY = BLay<DK>;
  using RS = Res<MODE_CHUNK>;
  constexpr int KB = LY::KB, MT = LY::MT, RB = LY::RB;
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
  if (c * CH >= si.len) return;
  const int L = min(CH, si.len - c * CH);
  const int H = p.H, DV = p.DV, ntiles = p.ntiles;
  const size_t row0 = (size_t)si.b * p.T + si.t0 + (size_t)c * CH;  // global row of the chunk start
  const int w = wave_id(), l = lane_id(), n = l & 15, g = l >> 4, e4 = (l >> 2) & 3, q4 = l & 3;

  // ---- lane bases
  const int sn = swz_s<DK>(n);
  const uint32_t lb_frag = n * RB + 16 * (g ^ (sn & 3)) + 64 * (sn >> 2);  // K/Q/S frag
  uint32_t lb_str[2];  // S-like transposed reads, rows 32kb + 8g + 4hh + e, columns 16mt + 4q
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g + 4 * hh + e4, s = swz_s<DK>(r);
    lb_str[hh] = r * RB + 8 * q4 + 32 * (s >> 1);
  }
  uint32_t lb_rtr;  // rows 16w + 4g + e, columns 16mt + 4q (K and Q reads of the db terms)
  {
    const int r = 4 * g + e4, s = swz_s<DK>(r);
    lb_rtr = (16 * w + r) * RB + 8 * q4 + 32 * (s >> 1);
  }
  uint32_t lb_dtr[2];  // dO transposed reads, rows 32kb + 8g + 4hh + e, columns 16w + 4q
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g + 4 * hh + e4, s = swz_d(r);
    lb_dtr[hh] = r * 128 + 16 * ((2 * w + (q4 >> 1)) ^ s) + 8 * (q4 & 1);
  }
  const int sdn = swz_d(n);
  const uint32_t lb_dfrag = (16 * w + n) * 128 + 16 * (g ^ (sdn & 3)) + 64 * (sdn >> 2);  // dO frag, row 16w + n
  uint32_t lb_vtr;  // V transposed reads, rows 16t + 4g + e, columns 16w + 4q
  {
    const int r = 4 * g + e4;
    lb_vtr = r * 128 + 16 * ((2 * w + (q4 >> 1)) ^ swz_v(r)) + 8 * (q4 & 1);
  }
  uint32_t lb_xw;  // V'^T / Y^T write: row 16w + n, columns 16i + 4g: 16w*128 + (lb_xw ^ 32 i)
  {
    const int s = swz_x(n);
    lb_xw = n * 128 + 32 * (s >> 1) + 16 * ((g >> 1) ^ (s & 1)) + 8 * (g & 1);
  }
  uint32_t lb_xtr[2];  // V'^T / Y^T transposed reads: rows 32kb + 8g + 4hh + e, columns 16jt + 4q
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int r = 8 * g + 4 * hh + e4, s = swz_x(r);
    lb_xtr[hh] = r * 128 + 32 * (s >> 1) + 16 * ((q4 >> 1) ^ (s & 1)) + 8 * (q4 & 1);
  }
  const uint32_t lb_m = 32 * n + ((8 * g) ^ (16 * ((n >> 3) & 1)));           // 16x16 block row reads
  const int rb4 = 4 * g + e4;
  const uint32_t lb_btr = 32 * rb4 + ((8 * q4) ^ (16 * ((rb4 >> 3) & 1)));  // 16x16 block transposed reads
  Bases lb = {};
  lb.m = lb_m;
  lb.btr = lb_btr;

  // ---- direct loads
  const char *gk = static_cast<const char *>(p.k);
  const char *gq = static_cast<const char *>(p.q);
  const char *gv = static_cast<const char *>(p.v);
  const char *gdo = static_cast<const char *>(p.dO);
  const size_t rowoff = (row0 * H + h);
  auto kq_off = [&](int i, int &row) {  // K / Q tile, load i of this wave
    const int pp = 64 * (w + 4 * i) + l;
    const int r = pp / (DK / 8), u = (pp % (DK / 8)) ^ swz_s<DK>(r);
    row = r;
    return (uint32_t)r * (uint32_t)(H * RB) + 16u * u;
  };
  auto issue_kq = [&]() {
#pragma unroll
    for (int i = 0; i < LY::DMA_KQ; ++i) {
      int r;
      const uint32_t off = kq_off(i, r);
      const uint32_t dst = sb + 1024 * (w + 4 * i);
      if (r < L) {
        dma16(gk + rowoff * RB + off, dst + LY::O_K);
        dma16(gq + rowoff * RB + off, dst + LY::O_Q);
      }
    }
    if (l < L) {
      if (w == 0 && GATED) dma4(reinterpret_cast<const char *>(p.g + rowoff) + 4u * l * H, sb + LY::O_XG);
      if (w == 1) dma4(reinterpret_cast<const char *>(p.beta + rowoff) + 4u * l * H, sb + LY::O_XB);
    }
  };
  const size_t sbase_g = ((size_t)cg * H + h) * (size_t)DV;  // row of S / dS for d_v column 0
  auto issue_tile = [&](int j, int buf) {
    const uint32_t tb = sb + LY::O_T + buf * LY::TB;
    const int dv0 = 64 * j;
#pragma unroll
    for (int i = 0; i < 2; ++i) {  // V and dO: 64 rows x 128 bytes
      const int pp = 64 * (w + 4 * i) + l;
      const int r = pp / 8, pos = pp % 8;
      if (r < L) {
        dma16(gv + ((rowoff + (size_t)r * H) * DV + dv0) * 2 + 16 * (pos ^ swz_v(r)), tb + LY::T_V + 1024 * (w + 4 * i));
        dma16(gdo + ((rowoff + (size_t)r * H) * DV + dv0) * 2 + 16 * (pos ^ swz_d(r)), tb + LY::T_DO + 1024 * (w + 4 * i));
      }
    }
    const char *s0 = reinterpret_cast<const char *>(p.states + (sbase_g + dv0) * DK);
    const char *d0 = reinterpret_cast<const char *>(p.dstates + (sbase_g + dv0) * DK);
#pragma unroll
    for (int i = 0; i < LY::DMA_S; ++i) {  // S and dS: 64 rows x RB bytes
      const int pp = 64 * (w + 4 * i) + l;
      const int r = pp / (DK / 8), u = (pp % (DK / 8)) ^ swz_s<DK>(r);
      dma16(s0 + r * RB + 16 * u, tb + LY::T_S + 1024 * (w + 4 * i));
      dma16(d0 + r * RB + 16 * u, tb + LY::T_DS + 1024 * (w + 4 * i));
    }
  };
  // rows past the end of the chunk are zero
  if (L < CH) {
    for (int i = L * RB / 16 + threadIdx.x; i < LY::KQ / 16; i += NTHR) {
      st<f32x4>(sb + LY::O_K + 16 * i, zero4());
      st<f32x4>(sb + LY::O_Q + 16 * i, zero4());
    }
    for (int buf = 0; buf < 2; ++buf)
      for (int i = L * 128 / 16 + threadIdx.x; i < 8192 / 16; i += NTHR) {
        st<f32x4>(sb + LY::O_T + buf * LY::TB + LY::T_V + 16 * i, zero4());
        st<f32x4>(sb + LY::O_T + buf * LY::TB + LY::T_DO + 16 * i, zero4());
      }
  }
  // P^T above the diagonal stays zero
  for (int i = threadIdx.x; i < RS::P_BYTES / 16; i += NTHR) st<f32x4>(sb + LY::O_RES + RS::O_P + 16 * i, zero4());
  issue_kq();
  issue_tile(0, 0);
  wait_vm<0>();
  if (ntiles > 1) issue_tile(1, 1);
  __syncthreads();

  // ---- prep of the chunk (M, P^T, R_ii, gates), one role per wave
  const uint32_t ob = sb + LY::O_RES;
  {
    if (w == 1) st<float>(sb + LY::O_BETA + 4 * l, l < L ? ld<float>(sb + LY::O_XB + 4 * l) : 0.f);
    float dummy = 1.f;
    const BwdKsw<DK> ksw{lb_frag};
    const uint32_t priv = sb + LY::O_X + w * PRIV_BYTES;
    const uint32_t kba = sb + LY::O_K, qba = sb + LY::O_Q, ga = sb + LY::O_XG, ba = sb + LY::O_XB;
    if (w == 0) prep_chunk<DK, GATED, true, MODE_CHUNK, 0>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else if (w == 1) prep_chunk<DK, GATED, true, MODE_CHUNK, 1>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else if (w == 2) prep_chunk<DK, GATED, true, MODE_CHUNK, 2>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
    else prep_chunk<DK, GATED, true, MODE_CHUNK, 3>(lb, kba, qba, ga, ba, ob, priv, L, dummy, ksw);
  }
  __syncthreads();

  // gate values of this lane's rows (column phase: rows 16i + 4g + e)
  const uint32_t cgt = ob + RS::O_CG;
  auto gam4 = [&](int i) { return GATED ? ld<f32x4>(cgt + CG_GS + 4 * (16 * i + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f}; };
  auto w4 = [&](int i) { return GATED ? ld<f32x4>(cgt + CG_WS + 4 * (16 * i + 4 * g)) : (f32x4){1.f, 1.f, 1.f, 1.f}; };
  auto bet4 = [&](int i) { return ld<f32x4>(sb + LY::O_BETA + 4 * (16 * i + 4 * g)); };

  // K fragments (rows 16t + n) stay in registers for every tile
  bf16x8 kf[4][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[t][kb] = ld<bf16x8>(sb + LY::O_K + (lb_frag ^ (64 * kb)) + 16 * t * RB);

  // accumulators over d_v (wave w: token rows 16w .. 16w + 15)
  f32x4 dP[4], dAc[4], dq1[MT], dk1[MT], dk2[MT];
#pragma unroll
  for (int t = 0; t < 4; ++t) dP[t] = dAc[t] = zero4();
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) dq1[mt] = dk1[mt] = dk2[mt] = zero4();
  f32x4 xy[4];  // rowsum(X * Y) partials: rows 16i + 4g + e of this lane's columns
#pragma unroll
  for (int i = 0; i < 4; ++i) xy[i] = zero4();
  float hdh = 0.f;  // <dh, h> partial

  const uint32_t xv = sb + LY::O_X, xy_ = sb + LY::O_X + 8192;  // V'^T, Y^T
  for (int j = 0; j < ntiles; ++j) {
    const uint32_t tb = sb + LY::O_T + (j & 1) * LY::TB;
    if (j > 0) {
      if (L == CH && j + 1 < ntiles) wait_vm<2 * LY::DMA_S + 4 + 16>(); else wait_vm<0>();
      __syncthreads();  // tile j loaded by every wave
    }
    // ---- column phase: columns 16w + n of the tile
    {
      bf16x8 hb[KB], dhb[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint32_t a = (lb_frag ^ (64 * kb)) + 16 * w * RB;
        hb[kb] = ld<bf16x8>(tb + LY::T_S + a);
        dhb[kb] = ld<bf16x8>(tb + LY::T_DS + a);
        hdh = dot8(hb[kb], dhb[kb], hdh);
      }
      f32x4 x[4], dvp[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 yk = zero4(), yd = zero4();
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          yk = mma32(yk, kf[t][kb], hb[kb]);
          yd = mma32(yd, kf[t][kb], dhb[kb]);
        }
        const bf16x4 vr = ld_tr(tb + LY::T_V + 16 * t * 128 + lb_vtr);
        const f32x4 gm = gam4(t);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[t][e] = bf2f(vr[e]) - gm[e] * yk[e];
        dvp[t] = w4(t) * yd;
      }
      // dV' += P^T dO (token blocks kb >= t / 2)
      bf16x8 dob[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        dob[kb] = cat(ld_tr(tb + LY::T_DO + 32 * kb * 128 + lb_dtr[0]), ld_tr(tb + LY::T_DO + 32 * kb * 128 + lb_dtr[1]));
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int kb = t >> 1; kb < 2; ++kb) dvp[t] = mma32(dvp[t], ld<bf16x8>(ob + RS::O_P + pt_frag(t, kb, l)), dob[kb]);
      // V'_i = R_ii diag(beta_i) (X_i - sum_{m<i} M_im V'_m)
      bf16x4 vb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc = x[i];
#pragma unroll
        for (int m = 0; m < i; ++m) acc = mma16(acc, ld<bf16x4>(ob + RS::O_M + 512 * m_block(i, m) + lb_m), vb[m]);
        acc = acc * bet4(i);
        vb[i] = cvt4(mma16(zero4(), ld_tr(ob + RS::O_TT + 512 * i + lb_btr), cvt4(acc)));
      }
      // Y_i = R_ii^T (dV'_i - sum_{m>i} M_mi^T dX_m), dX = diag(beta) Y
      f32x4 y[4];
      bf16x4 dxb[4];
#pragma unroll
      for (int i = 3; i >= 0; --i) {
        f32x4 acc = dvp[i];
#pragma unroll
        for (int m = i + 1; m < 4; ++m) acc = mma16(acc, ld_tr(ob + RS::O_M + 512 * m_block(m, i) + lb_btr), dxb[m]);
        y[i] = mma16(zero4(), ld<bf16x4>(ob + RS::O_TT + 512 * i + lb_m), cvt4(acc));
        const f32x4 dx = y[i] * bet4(i);
        dxb[i] = cvt4(dx);
        xy[i] = xy[i] + x[i] * y[i];
        // dv
        const int col = 64 * j + 16 * w + n;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + 4 * g + e;
          if (r < L) p.dv[((row0 + r) * H + h) * (size_t)DV + col] = dx[e];
        }
      }
      // hand V'^T and Y^T to the row phase
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st<bf16x4>(xv + 16 * w * 128 + (lb_xw ^ (32 * i)), vb[i]);
        st<bf16x4>(xy_ + 16 * w * 128 + (lb_xw ^ (32 * i)), cvt4(y[i]));
      }
    }
    __syncthreads();  // V'^T, Y^T complete
    // ---- row phase: token rows 16w + n
    {
      bf16x8 dof[2], yf[2], vf[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        dof[kb] = ld<bf16x8>(tb + LY::T_DO + (lb_dfrag ^ (64 * kb)));
        const uint32_t a0 = 32 * kb * 128 + (lb_xtr[0] ^ (32 * w)), a1 = 32 * kb * 128 + (lb_xtr[1] ^ (32 * w));
        yf[kb] = cat(ld_tr(xy_ + a0), ld_tr(xy_ + a1));
        vf[kb] = cat(ld_tr(xv + a0), ld_tr(xv + a1));
      }
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
        if (jt > w) break;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t a0 = 32 * kb * 128 + (lb_xtr[0] ^ (32 * jt)), a1 = 32 * kb * 128 + (lb_xtr[1] ^ (32 * jt));
          const bf16x8 vt = cat(ld_tr(xv + a0), ld_tr(xv + a1));
          dP[jt] = mma32(dP[jt], dof[kb], vt);
          dAc[jt] = mma32(dAc[jt], yf[kb], vt);
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const uint32_t a0 = 32 * kb * RB + (lb_str[0] ^ (32 * mt)), a1 = 32 * kb * RB + (lb_str[1] ^ (32 * mt));
          const bf16x8 sf = cat(ld_tr(tb + LY::T_S + a0), ld_tr(tb + LY::T_S + a1));
          const bf16x8 dsf = cat(ld_tr(tb + LY::T_DS + a0), ld_tr(tb + LY::T_DS + a1));
          dq1[mt] = mma32(dq1[mt], dof[kb], sf);
          dk1[mt] = mma32(dk1[mt], yf[kb], sf);
          dk2[mt] = mma32(dk2[mt], vf[kb], dsf);
        }
    }
    mfma_settle();
    __syncthreads();  // tile j and the hand-over buffers are free again
    if (j + 2 < ntiles) issue_tile(j + 2, j & 1);
  }

  // ---- final phase (wave w: rows r = 16w + 4g + e)
  const uint32_t fin = sb + LY::O_T;              // dPG^T and F^T, P^T layout
  const uint32_t red = sb + LY::O_T + LY::TB;     // reductions
  const f32x4 gam_r = gam4(w), w_r = w4(w), bet_r = bet4(w);
  const f32x4 bl_r = GATED ? ld<f32x4>(cgt + CG_BL + 4 * (16 * w + 4 * g)) : zero4();
  f32x4 erow = zero4(), dbr = zero4();
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    f32x4 dpg = zero4(), f = zero4();
    float ce = 0.f;
    if (jt <= w) {
      const int jj = 16 * jt + n;
      const float blj = GATED ? ld<float>(cgt + CG_BL + 4 * jj) : 0.f;
      const bf16x4 pv = ld<bf16x4>(ob + RS::O_P + pt_quad(jt, w, l));  // P[r][j]
      f32x4 mv;                                                        // M[r][j]
      if (jt < w) {
        const bf16x4 mm = ld_tr(ob + RS::O_M + 512 * m_block(w, jt) + lb_btr);
#pragma unroll
        for (int e = 0; e < 4; ++e) mv[e] = -bf2f(mm[e]);
      } else {
        const bf16x4 mm = ld<bf16x4>(ob + RS::O_M + 512 * (6 + w) + lb_m);
#pragma unroll
        for (int e = 0; e < 4; ++e) mv[e] = bf2f(mm[e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * g + e;
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
    st<bf16x4>(fin + pt_quad(jt, w, l), cvt4(dpg));
    st<bf16x4>(fin + 8192 + pt_quad(jt, w, l), cvt4(f));
    ce = sum4g(ce);
    if (g == 0) st<float>(red + 256 * w + 4 * (16 * jt + n), ce);  // colsum(E) of wave w
  }
  // rowsum(X * Y) of this wave's columns, and the scalars
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float s = sum16(xy[i][e]);
      if (n == 0) st<float>(red + 1024 + 256 * w + 4 * (16 * i + 4 * g + e), s);
    }
  hdh = wave_sum(hdh);
  // row terms: gamma_r q_r . DQ_r - gamma_r beta_r k_r . DY_r - w_r k_r . DH_r
  f32x4 rowt = zero4();
  float s3 = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const bf16x4 qv = ld_tr(sb + LY::O_Q + (lb_rtr ^ (32 * mt)));
    const bf16x4 kv = ld_tr(sb + LY::O_K + (lb_rtr ^ (32 * mt)));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float kdh = bf2f(kv[e]) * dk2[mt][e];
      rowt[e] += gam_r[e] * (bf2f(qv[e]) * dq1[mt][e] - bet_r[e] * bf2f(kv[e]) * dk1[mt][e]) - w_r[e] * kdh;
      s3 += w_r[e] * kdh;
    }
  }
  s3 = wave_sum(s3);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float rt = sum16(rowt[e] + erow[e]);
    const float db = sum16(dbr[e]);
    if (n == 0) {
      st<float>(red + 2048 + 4 * (16 * w + 4 * g + e), rt);
      st<float>(red + 2304 + 4 * (16 * w + 4 * g + e), db);
    }
  }
  if (l == 0) {
    st<float>(red + 2560 + 4 * w, s3);
    st<float>(red + 2576 + 4 * w, hdh);
  }
  __syncthreads();

  // dq = diag(gamma) dO h^T + dPG K ;
  // dk = dPG^T Q - diag(gamma beta) Y h^T + diag(w) V' dh^T + F K + F^T K
  {
    bf16x8 pgr[2], pgt[2], fr[2], ft[2];  // A operands: rows r (dPG, F), rows j (dPG^T, F^T)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // rows 16w + n of dPG: columns j = slots of kb, read transposed from dPG^T
      bf16x4 t0, t1, u0, u1;
      {
        const int r0 = 32 * kb + 8 * g + e4, r1 = r0 + 4;  // dPG^T rows j
        const int c = 16 * w + 4 * q4;                       // columns r
        const uint32_t a0 = 128 * r0 + 16 * ((c / 8) ^ swz_p128(r0 & 15)) + 8 * ((c % 8) / 4);
        const uint32_t a1 = 128 * r1 + 16 * ((c / 8) ^ swz_p128(r1 & 15)) + 8 * ((c % 8) / 4);
        t0 = ld_tr(fin + a0);
        t1 = ld_tr(fin + a1);
        u0 = ld_tr(fin + 8192 + a0);
        u1 = ld_tr(fin + 8192 + a1);
      }
      pgr[kb] = cat(t0, t1);
      fr[kb] = cat(u0, u1);
      pgt[kb] = ld<bf16x8>(fin + pt_frag(w, kb, l));
      ft[kb] = ld<bf16x8>(fin + 8192 + pt_frag(w, kb, l));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 dq = gam_r * dq1[mt];
      f32x4 dk = w_r * dk2[mt] - gam_r * bet_r * dk1[mt];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t a0 = 32 * kb * RB + (lb_str[0] ^ (32 * mt)), a1 = 32 * kb * RB + (lb_str[1] ^ (32 * mt));
        const bf16x8 kt = cat(ld_tr(sb + LY::O_K + a0), ld_tr(sb + LY::O_K + a1));
        const bf16x8 qt = cat(ld_tr(sb + LY::O_Q + a0), ld_tr(sb + LY::O_Q + a1));
        dq = mma32(dq, pgr[kb], kt);
        dk = mma32(dk, pgt[kb], qt);
        dk = mma32(dk, fr[kb], kt);
        dk = mma32(dk, ft[kb], kt);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * w + 4 * g + e;
        if (r < L) {
          const size_t o = ((row0 + r) * H + h) * (size_t)DK + 16 * mt + n;
          p.dq[o] = dq[e];
          p.dk[o] = dk[e];
        }
      }
    }
  }
  // dbeta, db -> dg (reverse cumulative sum inside the chunk)
  if (w == 0) {
    const int r = l;
    float ce = 0.f, xyr = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      ce += ld<float>(red + 256 * ww + 4 * r);
      xyr += ld<float>(red + 1024 + 256 * ww + 4 * r);
    }
    float db = ld<float>(red + 2048 + 4 * r) - ce;
    if (r == CH - 1) {
      float s3t = 0.f, hdt = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        s3t += ld<float>(red + 2560 + 4 * ww);
        hdt += ld<float>(red + 2576 + 4 * ww);
      }
      const float g63 = GATED ? ld<float>(cgt + CG_GS + 4 * (CH - 1)) : 1.f;
      db += s3t + g63 * hdt;
    }
    const float incl = wave_incl_scan(db);
    const float total = __shfl(incl, 63, 64);
    if (r < L) {
      const size_t idx = (row0 + r) * H + h;
      p.dbeta[idx] = xyr + ld<float>(red + 2304 + 4 * r);
      if (GATED) p.dg[idx] = total - incl + db;  // sum_{r' >= r} db_r'
    }
  }
}

template <int DK>
hipError_t launch_t(const BwdParams &p, hipStream_t stream) {
  const size_t smem = BLay<DK>::TOTAL;
  auto kern = p.g ? bwd_chunk_kernel<DK, true> : bwd_chunk_kernel<DK, false>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int grid = p.total_chunks * p.H;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), smem, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_chunk(const BwdParams &p, int DK, hipStream_t stream) {
  if (DK == 64) return launch_t<64>(p, stream);
  if (DK == 128) return launch_t<128>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace dn
