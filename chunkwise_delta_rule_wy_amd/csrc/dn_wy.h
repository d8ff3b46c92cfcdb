// Building blocks of the bf16 chunk kernels (forward and backward): LDS access
// helpers, the swizzled LDS layouts and the per-chunk preparation of the WY/UT
// form.
//
// LDS layouts.  Every matrix is stored in rows of 16-byte units with an XOR
// swizzle of the unit index by row bits.  The swizzles were chosen against
// the bank structure of the gfx950 LDS (64 banks of 4 bytes; a 16-byte read
// is served in four passes of 16 lanes grouped by lane bit 5 and the parity
// of lane bits 2..4, an 8-byte read in two passes of 32 consecutive lanes), so
// that the access patterns of the kernels are conflict free, and they are
// linear in the row bits, so that a lane's address is a precomputed base XOR
// a constant plus an immediate offset.
//
// Fragment reads.  A 16x16x32 MFMA operand gives lane (n, g) = (l % 16, l / 16)
// the 8 contraction indices of slots 8g .. 8g + 7: a 16-byte read of row n
// ("frag"), or two transposed reads (ds_read_b64_tr_b16) of four rows each
// when the contraction runs along the rows of the stored matrix.
#pragma once

#include <type_traits>

#include "dn_internal.h"

namespace dn {
namespace wy {

template <typename T> using lds_ptr = __attribute__((address_space(3))) T *;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T>
__device__ __forceinline__ T ld(uint32_t a) {
  return *(lds_ptr<const T>)(size_t)(a);
}
template <typename T>
__device__ __forceinline__ void st(uint32_t a, const T &v) {
  *(lds_ptr<T>)(size_t)(a) = v;
}
// transposed 4 x 16 read: the lane (4e + q) of each 16-lane group reads 4
// consecutive bf16 at its address; lane 4q + s receives element s of the
// reads of lanes q, 4 + q, 8 + q, 12 + q
__device__ __forceinline__ bf16x4 ld_tr(uint32_t a) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr<s16x4>)(size_t)(a)));
}
// Direct global -> LDS loads of 16 or 4 bytes per lane; lane l writes dst + 16 l
// (or 4 l), dst wave-uniform (it goes to M0).  They are issued from inline
// assembly on purpose: the compiler's wait insertion treats every transposed
// LDS read (ds_read_b64_tr_b16) after a direct load as dependent on it and
// waits for all outstanding vector memory operations, which would drain the
// prefetch ring on every step.  The kernels order these loads themselves with
// wait_vm<N> and barriers; the compiler's own waits for its loads and stores
// only become more conservative, since it does not count these.  The s_nop
// covers the one wait state an LDS DMA needs after M0 is written by SALU.
__device__ __forceinline__ void dma16(const void *src, uint32_t dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}
__device__ __forceinline__ void dma4(const void *src, uint32_t dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(dst) : "memory");
}
// the same with a wave-uniform base address and a 32-bit per-lane byte offset
__device__ __forceinline__ void dma16s(const void *base, uint32_t voff, uint32_t dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(dst) : "memory");
}

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }
__device__ __forceinline__ bf16x4 cvt4(const f32x4 &v) { return cvt_bf16x4(v); }
__device__ __forceinline__ bf16x8 cat(const bf16x4 &a, const bf16x4 &b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lane_val(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// dot product of two bf16 x 8 fragments, accumulated in fp32
__device__ __forceinline__ float dot8(const bf16x8 &a, const bf16x8 &b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), c, false);
  return c;
}

// value of lane S of each quad (lanes 4c .. 4c + 3)
template <int S>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_mov_dpp(__float_as_int(v), S | (S << 2) | (S << 4) | (S << 6), 0xf, 0xf, false));
}

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float SCALE_MIN = 0x1p-30f;  // smallest state scale before a restart at 1

// gate table of a chunk for the state-dependent work (fp32), byte offsets
//   forward (state h = s_c h~):    GS = gamma_r s_c, WS = w_r / s_{c+1}
//   reverse scan (dh = s_c dh~):   GS = gamma_r / s_c, WS = w_r s_{c+1}
//   chunk gradients:               GS = gamma_r, WS = w_r, BL = b_r log2(e)
// with w_r = exp(b_63 - b_r); HSCALE is the factor applied to the stored
// state before the chunk's update when the scale restarts at 1 (1: none).
constexpr int CG_GS = 0;
constexpr int CG_WS = 256;
constexpr int CG_HSCALE = 512;
constexpr int CG_SC = 516;      // scale of the state entering the chunk's update
constexpr int CG_SNEXT = 520;   // scale after it
constexpr int CG_BL = 512;
constexpr int CG_BYTES = 768;
// a prep wave's own gate table (fp32), byte offsets
constexpr int PG_BL = 0;      // b_r log2(e)
constexpr int PG_RHO = 256;   // exp(b_r - b_{16 floor(r/16)})
constexpr int PG_KAP = 512;   // [3][64]: exp(b_{16(i+1)} - b_j), used for j < 16(i+1)
constexpr int PG_BYTES = 1280;
constexpr int AT_BYTES = 1536;  // A_vv^T, fp32, 96-byte rows
constexpr int PRIV_BYTES = AT_BYTES + PG_BYTES;

// Which kernel a chunk preparation serves.
enum : int { MODE_FWD = 0, MODE_CHUNK = 1, MODE_SCAN = 2 };

// Results of the preparation of one chunk (byte offsets in a result buffer).
//   forward:  P with rows 0..31 in 64-byte rows and rows 32..63 in 128-byte
//             rows; -M_ij (i > j) in six 16 x 16 blocks; T_ii^T.
//   chunk gradients: P^T, 64 x 64 in 128-byte rows; -M_ij (i > j) in six
//             blocks and M_ii^T in four more; R_ii^T.
//   reverse scan: P^T; -M_ij (i > j); R_ii^T.
template <int MODE>
struct Res {
  static constexpr int O_P = 0;
  static constexpr int P_BYTES = MODE == MODE_FWD ? 6144 : 8192;
  static constexpr int O_M = P_BYTES;
  static constexpr int O_TT = O_M + (MODE == MODE_CHUNK ? 10 : 6) * 512;
  static constexpr int O_CG = O_TT + 2048;
  static constexpr int BYTES = O_CG + CG_BYTES;
  static_assert(BYTES % 256 == 0, "alignment");
};

// Unit swizzles (XOR on the 16-byte unit index of a row).
template <int DK>
__device__ __forceinline__ int swz_kq(int r) {  // K, Q of the forward kernel
  if constexpr (DK == 128)
    return (r & 1) | (((r >> 3) & 1) << 1) | (((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 3);
  else
    return ((r >> 1) & 1) | (((r >> 3) & 1) << 1) | (((r >> 2) & 1) << 2);
}
__device__ __forceinline__ int swz_v(int r) { return r & 6; }
__device__ __forceinline__ int swz_p128(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_p64(int r) { return 2 * ((r >> 3) & 1); }

// Per-lane LDS address bases.
struct Bases {
  uint32_t frag;  // K / Q row 16t + n, d_k block kb: 16t RB + (frag ^ 64 kb)
  uint32_t ktr;   // K^T read: (32kb + 16hh) RB + 8 (mt & 1) + (ktr ^ 64 (mt / 2))
  uint32_t vtr;   // V read (chain wave w): 16t * 128 + vtr
  uint32_t p64;   // P rows 16i + n, i < 2: 1024 i + p64 (+ 8 for the odd column block)
  uint32_t p128;  // P rows 16i + n, i >= 2: 2048 (i - 1) + (p128 ^ 64 kb) (+ 8 ...)
  uint32_t m;     // 16 x 16 block, lane (n, g) reads row n columns 4g..4g+3: block + m
  uint32_t btr;   // 16 x 16 block, transposed read (rows 4g + e, columns 4q): block + btr
};

template <int DK>
__device__ __forceinline__ Bases lane_bases(int w, int l) {
  Bases b;
  const int n = l & 15, g = l >> 4, e = (l >> 2) & 3, q = l & 3;
  constexpr int RB = 2 * DK;
  int s = swz_kq<DK>(n);
  b.frag = n * RB + 16 * (g ^ (s & 3)) + 64 * (s >> 2);
  const int r = 4 * g + e;
  s = swz_kq<DK>(r);
  b.ktr = r * RB + 16 * (q ^ (s & 3)) + 64 * (s >> 2);
  b.vtr = r * 128 + 16 * ((2 * w + (q >> 1)) ^ swz_v(r)) + 8 * (q & 1);
  b.p64 = 64 * n + 16 * (g ^ swz_p64(n));
  s = swz_p128(n);
  b.p128 = 128 * n + 16 * (g ^ (s & 3)) + 64 * (s >> 2);
  b.m = 32 * n + ((8 * g) ^ (16 * ((n >> 3) & 1)));
  b.btr = 32 * r + ((8 * q) ^ (16 * ((r >> 3) & 1)));
  return b;
}
// 16 x 16 block (32-byte rows): lane (c, qr) = (l / 4, l % 4) writes row c columns 4qr..4qr+3
__device__ __forceinline__ uint32_t blk_quad(int l) {
  const int c = l >> 2, qr = l & 3;
  return 32 * c + ((8 * qr) ^ (16 * ((c >> 3) & 1)));
}

// forward P addresses (relative to the result buffer)
template <int TI, int TJ>
__device__ __forceinline__ uint32_t p_write(const Bases &lb) {
  if constexpr (TI < 2) return TI * 1024 + lb.p64 + 8 * (TJ & 1);
  else return 2048 * (TI - 1) + (lb.p128 ^ (64 * (TJ >> 1))) + 8 * (TJ & 1);
}
__device__ __forceinline__ uint32_t p_read(const Bases &lb, int nt, int kb) {
  return nt < 2 ? nt * 1024 + lb.p64 : 2048 * (nt - 1) + (lb.p128 ^ (64 * kb));
}
// backward P^T (64 x 64, 128-byte rows, swizzle swz_p128): lane (n, g) at row
// 16a + n, columns 16b + 4g .. +3
__device__ __forceinline__ uint32_t pt_quad(int a, int b, int l) {
  const int n = l & 15, g = l >> 4, u = 2 * b + (g >> 1);
  return 128 * (16 * a + n) + 16 * (u ^ swz_p128(n)) + 8 * (g & 1);
}
// ... and lane (n, g) 16-byte fragment at row 16t + n, columns 32kb + 8g .. +7
__device__ __forceinline__ uint32_t pt_frag(int t, int kb, int l) {
  const int n = l & 15, g = l >> 4;
  return 128 * (16 * t + n) + 16 * ((4 * kb + g) ^ swz_p128(n));
}
__device__ __forceinline__ constexpr int m_block(int i, int j) { return i * (i - 1) / 2 + j; }

// Hook that lets a prep wave issue the direct loads of a later chunk between
// the stages of a preparation, so that the vector-memory path works while the
// wave computes instead of stalling it up front (stages 0..3).
struct NoIssue {
  __device__ __forceinline__ void operator()(int) const {}
};

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using I2 = std::integral_constant<int, 2>;
using I3 = std::integral_constant<int, 3>;

// Preparation of one chunk of NB 16-token blocks (NB = 4: 64 tokens; NB = 2:
// 32 tokens) by one of four waves (PW).
//
//   wave v < NB: diagonal block M_vv (fp32, into its A^T scratch) and the
//                inverse of its diagonal block by forward substitution;
//                P_vv
//   wave 0: -M_10 -M_20 -M_30    wave 1: -M_21 -M_31 -M_32
//   wave 2: P_10 P_20 P_21       wave 3: P_30 P_31 P_32
//
// (every block with an index >= NB is left out).  For NB = 2 the rows
// 32 .. 63 are outside the chunk: the gate scan adds zero over them, so the
// value of lane 63 is the chunk's last cumulative gate b_31.
//
// M = strictLower((K K^T) * Gamma), P = (Q K^T) * Gamma (lower, with the
// diagonal), A = diag(beta) M.  The forward variant stores T_vv =
// (I + A_vv)^-1 diag(beta) (transposed) and the gate table with the state
// scale carried in `scale` by wave 0; the backward variants store R_vv =
// (I + A_vv)^-1 (transposed) and P^T instead of P, the chunk-gradient one also
// M_vv^T and the plain gate table, the scan one the gate table of the scaled
// state gradient.  kbase, qbase: K and Q tiles (K-tile swizzle KSW); gaddr, baddr:
// g and beta of the chunk's rows (fp32, LDS); rows >= L are padding.
template <int DK, bool GATED, bool WRITE_P, int MODE, int PW, int NB = 4, typename KSW, typename ISS = NoIssue>
__device__ __forceinline__ void prep_chunk(const Bases &lb, uint32_t kbase, uint32_t qbase, uint32_t gaddr,
                                           uint32_t baddr, uint32_t ob, uint32_t priv, int L, float &scale,
                                           KSW ksw, ISS iss = ISS{}) {
  static_assert(NB == 4 || NB == 2, "64- or 32-token chunks");
  using RS = Res<MODE>;
  constexpr bool BWD = MODE != MODE_FWD;
  constexpr int KB = DK / 32;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const uint32_t pg = priv + AT_BYTES;

  if constexpr (GATED) {
    const float gv = (l < L) ? ld<float>(gaddr + 4 * l) : 0.f;
    const float b = wave_incl_scan(gv) * LOG2E;
    const float b0 = lane_val(b, 0), b16 = lane_val(b, 16), b32 = lane_val(b, 32), b48 = lane_val(b, 48);
    const float bst = l < 16 ? b0 : l < 32 ? b16 : l < 48 ? b32 : b48;
    st<float>(pg + PG_BL + 4 * l, b);
    st<float>(pg + PG_RHO + 4 * l, fexp2(b - bst));
    st<float>(pg + PG_KAP + 4 * l, fexp2(b16 - b));
    st<float>(pg + PG_KAP + 256 + 4 * l, fexp2(b32 - b));
    st<float>(pg + PG_KAP + 512 + 4 * l, fexp2(b48 - b));
    if constexpr (PW == 0) {
      const float b63 = lane_val(b, 63);
      if constexpr (MODE == MODE_CHUNK) {
        st<float>(ob + RS::O_CG + CG_GS + 4 * l, fexp2(b));
        st<float>(ob + RS::O_CG + CG_WS + 4 * l, fexp2(b63 - b));
        st<float>(ob + RS::O_CG + CG_BL + 4 * l, b);
      } else {
        // the state (forward) or state gradient (scan) of scale sc is multiplied by
        // gamma_63 in this chunk's update: t is the next scale unless it restarts
        const float sc = scale;
        const float t = sc * fexp2(b63);
        const bool resc = !(t >= SCALE_MIN);
        const float inv = resc ? 1.f : 1.f / t;
        if constexpr (MODE == MODE_FWD) {
          st<float>(ob + RS::O_CG + CG_GS + 4 * l, fexp2(b) * sc);
          st<float>(ob + RS::O_CG + CG_WS + 4 * l, fexp2(b63 - b) * inv);
        } else {
          st<float>(ob + RS::O_CG + CG_GS + 4 * l, fexp2(b) * inv);
          st<float>(ob + RS::O_CG + CG_WS + 4 * l, fexp2(b63 - b) * sc);
        }
        if (l == 0) {
          st<float>(ob + RS::O_CG + CG_HSCALE, resc ? t : 1.f);
          st<float>(ob + RS::O_CG + CG_SC, sc);
          st<float>(ob + RS::O_CG + CG_SNEXT, resc ? 1.f : t);
        }
        scale = resc ? 1.f : t;
      }
    }
    wave_lds_fence();
  }
  iss(0);

  bf16x8 kf[NB][KB];  // K rows 16t + n, d_k block kb
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int t = 0; t < NB; ++t) kf[t][kb] = ld<bf16x8>(kbase + ksw.frag(t, kb));

  // Diagonal block PW of A = strictLower(diag(beta) (K K^T) * Gamma), fp32,
  // transposed into the scratch.  Lane (n, g) holds k_r . k_j with
  // r = 16PW + 4g + e, j = 16PW + n.
  if constexpr (PW < NB) {
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
      mv[e] = keep ? mv[e] : 0.f;
      a[e] = keep ? be[e] * mv[e] : 0.f;
    }
    st<f32x4>(priv + 96 * n + 16 * g, a);
    if constexpr (MODE == MODE_CHUNK) st<bf16x4>(ob + RS::O_M + 512 * (6 + PW) + lb.m, cvt4(mv));  // M_vv^T row n
  }

  iss(1);

  // Block (TI, TJ) of -M below the diagonal: lane (n, g) holds k_r . k_j with
  // r = 16TI + n, j = 16TJ + 4g + e.
  auto mtile = [&](auto ti_c, auto tj_c) {
    constexpr int TI = decltype(ti_c)::value, TJ = decltype(tj_c)::value;
    if constexpr (TI < NB) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[TJ][kb], kf[TI][kb]);
    f32x4 v;
    if constexpr (GATED) {
      const float rho = ld<float>(pg + PG_RHO + 4 * (16 * TI + n));
      const f32x4 kap = ld<f32x4>(pg + PG_KAP + 256 * (TI - 1) + 4 * (16 * TJ + 4 * g));
      v = acc * kap * (-rho);
    } else {
      v = -acc;
    }
    st<bf16x4>(ob + RS::O_M + 512 * m_block(TI, TJ) + lb.m, cvt4(v));
    }
  };
  // in the scan, wave 0 (which also keeps the scale bookkeeping) hands block
  // (3, 0) to wave 2, the prep wave with the least other work there
  if constexpr (PW == 0) {
    mtile(I1{}, I0{});
    mtile(I2{}, I0{});
    if constexpr (MODE != MODE_SCAN) mtile(I3{}, I0{});
  } else if constexpr (PW == 1) {
    mtile(I2{}, I1{});
    mtile(I3{}, I1{});
    mtile(I3{}, I2{});
  } else if constexpr (PW == 2 && MODE == MODE_SCAN) {
    mtile(I3{}, I0{});
  }

  iss(2);

  if constexpr (WRITE_P) {
    // P block (TI, TJ), TJ <= TI.  Forward: lane (n, g) holds q_r . k_j with
    // r = 16TI + n, j = 16TJ + 4g + e, stored into P.  Backward: lane (n, g)
    // holds q_r . k_j with r = 16TI + 4g + e, j = 16TJ + n, stored into P^T.
    auto ptile = [&](auto ti_c, auto tj_c, const bf16x8(&qf)[KB]) {
      constexpr int TI = decltype(ti_c)::value, TJ = decltype(tj_c)::value;
      if constexpr (TI < NB) {
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = BWD ? mma32(acc, qf[kb], kf[TJ][kb]) : mma32(acc, kf[TJ][kb], qf[kb]);
      f32x4 v;
      if constexpr (TI == TJ) {
        // row r, column j of the lane's element e
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = BWD ? 4 * g + e : n, j = BWD ? n : 4 * g + e;
          float gam = 1.f;
          if constexpr (GATED)
            gam = fexp2(ld<float>(pg + PG_BL + 4 * (16 * TI + r)) - ld<float>(pg + PG_BL + 4 * (16 * TJ + j)));
          v[e] = (j <= r) ? acc[e] * gam : 0.f;
        }
      } else if constexpr (GATED) {
        if constexpr (BWD) {
          const f32x4 rho = ld<f32x4>(pg + PG_RHO + 4 * (16 * TI + 4 * g));
          const float kap = ld<float>(pg + PG_KAP + 256 * (TI - 1) + 4 * (16 * TJ + n));
          v = acc * rho * kap;
        } else {
          const float rho = ld<float>(pg + PG_RHO + 4 * (16 * TI + n));
          const f32x4 kap = ld<f32x4>(pg + PG_KAP + 256 * (TI - 1) + 4 * (16 * TJ + 4 * g));
          v = acc * kap * rho;
        }
      } else {
        v = acc;
      }
      if constexpr (BWD) st<bf16x4>(ob + RS::O_P + pt_quad(TJ, TI, l), cvt4(v));
      else st<bf16x4>(ob + RS::O_P + p_write<TI, TJ>(lb), cvt4(v));
      }
    };
    auto qfrag = [&](bf16x8(&qf)[KB], int ti) {
      if (ti < NB) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) qf[kb] = ld<bf16x8>(qbase + ksw.frag(ti, kb));
      }
    };
    bf16x8 qa[KB], qb[KB];
    if constexpr (PW == 0) {
      qfrag(qa, 0);
      ptile(I0{}, I0{}, qa);
    } else if constexpr (PW == 1) {
      qfrag(qa, 1);
      ptile(I1{}, I1{}, qa);
    } else if constexpr (PW == 2) {
      qfrag(qa, 1);
      qfrag(qb, 2);
      ptile(I1{}, I0{}, qa);
      ptile(I2{}, I2{}, qb);
      ptile(I2{}, I0{}, qb);
      ptile(I2{}, I1{}, qb);
    } else {
      qfrag(qa, 3);
      ptile(I3{}, I3{}, qa);
      ptile(I3{}, I0{}, qa);
      ptile(I3{}, I1{}, qa);
      ptile(I3{}, I2{}, qa);
    }
  }

  iss(3);

  // (I + A_vv)^-1 (times diag(beta) in the forward variant): lane (c, qr) =
  // (l / 4, l % 4) holds rows 4qr .. 4qr + 3 of column c; column j of A_vv is
  // read from the scratch and x_j is broadcast from its owner lane of the quad.
  wave_lds_fence();
  if constexpr (PW < NB) {
    const int c = l >> 2, qr = l & 3;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (4 * qr + k == c) ? 1.f : 0.f;
    f32x4 acol[15];  // every column first: the chain below then waits on no LDS read
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
    float bc = 1.f;
    if constexpr (!BWD) {
      // read unconditionally (rows past the end hold stale values) and select:
      // no branch around the load, so no address register live across it
      const float bv = ld<float>(baddr + 64 * PW + 4 * c);
      bc = (16 * PW + c < L) ? bv : 0.f;
    }
    bf16x4 tv;
#pragma unroll
    for (int k = 0; k < 4; ++k) tv[k] = (__bf16)(x[k] * bc);
    st<bf16x4>(ob + RS::O_TT + 512 * PW + blk_quad(l), tv);
  }
  mfma_settle();
}

}  // namespace wy
}  // namespace dn
