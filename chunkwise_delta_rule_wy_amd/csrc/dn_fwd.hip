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
#include <type_traits>

#include "dn_internal.h"

namespace dn {
namespace {

template <typename T> using lds_ptr = __attribute__((address_space(3))) T *;
typedef short s16x4 __attribute__((ext_vector_type(4)));

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
// direct global -> LDS loads of 16 or 4 bytes per lane; lane l writes dst + 16 l (or 4 l)
__device__ __forceinline__ void dma16(const void *src, uint32_t dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr<void>)(size_t)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *src, uint32_t dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr<void>)(size_t)dst, 4, 0, 0);
}

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }
__device__ __forceinline__ bf16x4 cvt4(const f32x4 &v) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (__bf16)v[i];
  return r;
}
__device__ __forceinline__ bf16x8 cat(const bf16x4 &a, const bf16x4 &b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lane_val(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
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

constexpr int FWD_THREADS = 512;  // four chain waves, four prep waves
constexpr int NBUF = 3;           // ring slots
constexpr float LOG2E = 1.4426950408889634f;
constexpr float SCALE_MIN = 0x1p-30f;  // smallest state scale before a rescale

// chain gate table of a chunk (fp32), byte offsets
constexpr int CG_GS = 0;        // gamma_r s_c
constexpr int CG_WS = 256;      // exp(b_63 - b_r) / s_{c+1}
constexpr int CG_HSCALE = 512;  // factor on h~ before the update (1: none)
constexpr int CG_SC = 516;      // s_c
constexpr int CG_SNEXT = 520;   // s_{c+1}
constexpr int CG_BYTES = 768;
// a prep wave's own gate table (fp32), byte offsets
constexpr int PG_BL = 0;      // b_r log2(e)
constexpr int PG_RHO = 256;   // exp(b_r - b_{16 floor(r/16)})
constexpr int PG_KAP = 512;   // [3][64]: exp(b_{16(i+1)} - b_j), used for j < 16(i+1)
constexpr int PG_BYTES = 1280;
constexpr int AT_BYTES = 1536;  // A_vv^T, fp32, 96-byte rows

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
  static constexpr int O_P = 0;       // P: rows 0..31 with 64-byte rows, rows 32..63 with 128-byte rows
  static constexpr int O_M = 6144;    // -M, the six blocks below the diagonal, 16 x 32-byte rows each
  static constexpr int O_TT = 9216;   // T_ii^T, four 16 x 16 bf16 blocks
  static constexpr int O_CG = 11264;  // chain gate table
  static constexpr int OUTB = O_CG + CG_BYTES;
  static constexpr int OUT_OFF = NBUF * SLOT;
  static constexpr int PRIV_OFF = OUT_OFF + 2 * OUTB;  // per prep wave: A_vv^T, gate table
  static constexpr int PRIV = AT_BYTES + PG_BYTES;
  static constexpr int TOTAL = PRIV_OFF + 4 * PRIV;
  static_assert(TOTAL <= 160 * 1024, "LDS budget");
  static_assert(SLOT % 256 == 0 && OUTB % 256 == 0, "tile alignment");
};

// Unit swizzles (XOR on the 16-byte unit index of a row).
template <int DK>
__device__ __forceinline__ int swz_kq(int r) {
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
  uint32_t m;     // -M block (i, j): 512 (i (i - 1) / 2 + j) + m
};

template <int DK>
__device__ __forceinline__ Bases lane_bases(int w, int l) {
  using LY = Lay<DK>;
  Bases b;
  const int n = l & 15, g = l >> 4, e = (l >> 2) & 3, q = l & 3;
  int s = swz_kq<DK>(n);
  b.frag = n * LY::RB + 16 * (g ^ (s & 3)) + 64 * (s >> 2);
  const int r = 4 * g + e;
  s = swz_kq<DK>(r);
  b.ktr = r * LY::RB + 16 * (q ^ (s & 3)) + 64 * (s >> 2);
  b.vtr = r * 128 + 16 * ((2 * w + (q >> 1)) ^ swz_v(r)) + 8 * (q & 1);
  b.p64 = 64 * n + 16 * (g ^ swz_p64(n));
  s = swz_p128(n);
  b.p128 = 128 * n + 16 * (g ^ (s & 3)) + 64 * (s >> 2);
  b.m = 32 * n + ((8 * g) ^ (16 * ((n >> 3) & 1)));
  return b;
}

// P addresses (relative to the chunk's result buffer)
template <int TI, int TJ>
__device__ __forceinline__ uint32_t p_write(const Bases &lb) {
  if constexpr (TI < 2) return TI * 1024 + lb.p64 + 8 * (TJ & 1);
  else return 2048 * (TI - 1) + (lb.p128 ^ (64 * (TJ >> 1))) + 8 * (TJ & 1);
}
__device__ __forceinline__ uint32_t p_read(const Bases &lb, int nt, int kb) {
  return nt < 2 ? nt * 1024 + lb.p64 : 2048 * (nt - 1) + (lb.p128 ^ (64 * kb));
}
__device__ __forceinline__ constexpr int m_block(int i, int j) { return i * (i - 1) / 2 + j; }

using I0 = std::integral_constant<int, 0>;
using I1 = std::integral_constant<int, 1>;
using I2 = std::integral_constant<int, 2>;
using I3 = std::integral_constant<int, 3>;

// ---------------------------------------------------------------- prep

// Prep wave PW for chunk c: gate tables, its blocks of M and P, T_PW,PW.
//   every prep wave: M_vv (into its A^T scratch, then T_vv) and P_vv
//   wave 0: M_10 M_20 M_30    wave 1: M_21 M_31 M_32
//   wave 2: P_10 P_20 P_21    wave 3: P_30 P_31 P_32
// Prep wave 0 also writes the chain gate table and carries the state scale.
template <int DK, bool GATED, bool WRITE_O, int PW>
__device__ __forceinline__ void prep_chunk(const Bases &lb, uint32_t slot, uint32_t ob, uint32_t priv,
                                           int L, float &scale) {
  using LY = Lay<DK>;
  constexpr int KB = LY::KB;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const uint32_t pg = priv + AT_BYTES;

  if constexpr (GATED) {
    const float gv = (l < L) ? ld<float>(slot + LY::S_G + 4 * l) : 0.f;
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
      const float sc = scale;
      const float t = sc * fexp2(b63);
      const bool resc = !(t >= SCALE_MIN);
      const float inv = resc ? 1.f : 1.f / t;
      st<float>(ob + LY::O_CG + CG_GS + 4 * l, fexp2(b) * sc);
      st<float>(ob + LY::O_CG + CG_WS + 4 * l, fexp2(b63 - b) * inv);
      if (l == 0) {
        st<float>(ob + LY::O_CG + CG_HSCALE, resc ? t : 1.f);
        st<float>(ob + LY::O_CG + CG_SC, sc);
        st<float>(ob + LY::O_CG + CG_SNEXT, resc ? 1.f : t);
      }
      scale = resc ? 1.f : t;
    }
    wave_lds_fence();
  }

  bf16x8 kf[4][KB];  // K rows 16t + n, d_k block kb
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const uint32_t a = (lb.frag ^ (64 * kb)) + slot + LY::S_K;
#pragma unroll
    for (int t = 0; t < 4; ++t) kf[t][kb] = ld<bf16x8>(a + 16 * t * LY::RB);
  }

  // Diagonal block PW of A = strictLower(diag(beta) (K K^T) * Gamma), fp32,
  // transposed into the scratch.  Lane (n, g) holds k_r . k_j with
  // r = 16PW + 4g + e, j = 16PW + n.
  {
    f32x4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[PW][kb], kf[PW][kb]);
    const f32x4 be = ld<f32x4>(slot + LY::S_BETA + 4 * (16 * PW + 4 * g));
    f32x4 a;
    if constexpr (GATED) {
      const f32x4 blr = ld<f32x4>(pg + PG_BL + 4 * (16 * PW + 4 * g));
      const float blj = ld<float>(pg + PG_BL + 4 * (16 * PW + n));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        a[e] = (4 * g + e > n && 16 * PW + 4 * g + e < L) ? be[e] * acc[e] * fexp2(blr[e] - blj) : 0.f;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = (4 * g + e > n && 16 * PW + 4 * g + e < L) ? be[e] * acc[e] : 0.f;
    }
    st<f32x4>(priv + 96 * n + 16 * g, a);
  }

  // Block (TI, TJ) of -M below the diagonal: lane (n, g) holds k_r . k_j with
  // r = 16TI + n, j = 16TJ + 4g + e.
  auto mtile = [&](auto ti_c, auto tj_c) {
    constexpr int TI = decltype(ti_c)::value, TJ = decltype(tj_c)::value;
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
    st<bf16x4>(ob + LY::O_M + 512 * m_block(TI, TJ) + lb.m, cvt4(v));
  };
  if constexpr (PW == 0) {
    mtile(I1{}, I0{});
    mtile(I2{}, I0{});
    mtile(I3{}, I0{});
  } else if constexpr (PW == 1) {
    mtile(I2{}, I1{});
    mtile(I3{}, I1{});
    mtile(I3{}, I2{});
  }

  if constexpr (WRITE_O) {
    // P block (TI, TJ), TJ <= TI: lane (n, g) holds q_r . k_j with
    // r = 16TI + n, j = 16TJ + 4g + e.
    auto ptile = [&](auto ti_c, auto tj_c, const bf16x8(&qf)[KB]) {
      constexpr int TI = decltype(ti_c)::value, TJ = decltype(tj_c)::value;
      f32x4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) acc = mma32(acc, kf[TJ][kb], qf[kb]);
      f32x4 v;
      if constexpr (TI == TJ) {
        const float blr = GATED ? ld<float>(pg + PG_BL + 4 * (16 * TI + n)) : 0.f;
        const f32x4 blj = GATED ? ld<f32x4>(pg + PG_BL + 4 * (16 * TJ + 4 * g)) : zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (4 * g + e <= n) ? (GATED ? acc[e] * fexp2(blr - blj[e]) : acc[e]) : 0.f;
      } else if constexpr (GATED) {
        const float rho = ld<float>(pg + PG_RHO + 4 * (16 * TI + n));
        const f32x4 kap = ld<f32x4>(pg + PG_KAP + 256 * (TI - 1) + 4 * (16 * TJ + 4 * g));
        v = acc * kap * rho;
      } else {
        v = acc;
      }
      st<bf16x4>(ob + LY::O_P + p_write<TI, TJ>(lb), cvt4(v));
    };
    auto qfrag = [&](bf16x8(&qf)[KB], int ti) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        qf[kb] = ld<bf16x8>((lb.frag ^ (64 * kb)) + slot + LY::S_Q + 16 * ti * LY::RB);
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

  // T_vv = (I + A_vv)^-1 diag(beta): lane (c, qr) = (l / 4, l % 4) holds rows
  // 4qr .. 4qr + 3 of column c; column j of A_vv is read from the scratch and
  // x_j is broadcast from its owner lane of the quad.
  wave_lds_fence();
  {
    const int c = l >> 2, qr = l & 3;
    float x[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = (4 * qr + k == c) ? 1.f : 0.f;
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const f32x4 a = ld<f32x4>(priv + 96 * j + 16 * qr);
      const float own = x[j & 3];
      const float xj = (j >> 2) == 0 ? quad_bcast<0>(own)
                     : (j >> 2) == 1 ? quad_bcast<1>(own)
                     : (j >> 2) == 2 ? quad_bcast<2>(own)
                                     : quad_bcast<3>(own);
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] -= a[k] * xj;
    }
    const float bc = (16 * PW + c < L) ? ld<float>(slot + LY::S_BETA + 4 * (16 * PW + c)) : 0.f;
    bf16x4 tv;
#pragma unroll
    for (int k = 0; k < 4; ++k) tv[k] = (__bf16)(x[k] * bc);
    st<bf16x4>(ob + LY::O_TT + 512 * PW + 32 * c + 8 * qr, tv);
  }
  mfma_settle();
}

// ---------------------------------------------------------------- chain

template <int DK, bool GATED, bool STORE_STATES, bool WRITE_O>
__device__ __forceinline__ void chain_chunk(const FwdParams &p, const Bases &lb, f32x4 (&hs)[DK / 16],
                                            uint32_t slot, uint32_t ob, int L, size_t row0, int h,
                                            int col, float *states_dst) {
  using LY = Lay<DK>;
  constexpr int KB = LY::KB, MT = LY::MT;
  const int l = lane_id(), n = l & 15, g = l >> 4;
  const int H = p.H, DV = p.DV;

  if constexpr (STORE_STATES) {  // the state at the chunk start, h = s_c h~
    const float sc = GATED ? ld<float>(ob + LY::O_CG + CG_SC) : 1.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + i;
        states_dst[(size_t)r * DV + col] = hs[mt][i] * sc;
      }
  }
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
    const bf16x4 tf = ld_tr(ob + LY::O_TT + 512 * i + 8 * l);
    vp[i] = mma16(zero4(), tf, cvt4(acc));
    vb[i] = cvt4(vp[i]);
  }
  // O^T = diag(gamma s_c) Y_Q^T + V'^T P^T: lane (n, g) holds O[16nt + n][16w + 4g + e]
  if constexpr (WRITE_O) {
    bf16 *orow = static_cast<bf16 *>(p.o) + (row0 * H + h) * (size_t)DV + (col - n) + 4 * g;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      f32x4 acc = yq[nt];
      if constexpr (GATED) acc = acc * ld<float>(ob + LY::O_CG + CG_GS + 4 * (16 * nt + n));
#pragma unroll
      for (int kb = 0; kb <= (nt >> 1); ++kb)
        acc = mma32(acc, cat(vb[2 * kb], vb[2 * kb + 1]), ld<bf16x8>(ob + LY::O_P + p_read(lb, nt, kb)));
      if (16 * nt + n < L) *reinterpret_cast<bf16x4 *>(orow + (size_t)(16 * nt + n) * H * DV) = cvt4(acc);
    }
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
  const int n_seq = pair / p.H, h = pair % p.H;
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
        dma16(kb_ + koff[i], dst);
        if (WRITE_O) dma16(qb_ + koff[i], dst + LY::KQ);
      }
      if (scal) dma4(sb + soff, sdst);
#pragma unroll
      for (int i = 0; i < LY::DMA_V; ++i) dma16(vb_ + voff[i], slot + LY::S_V + 1024 * (v + 4 * i));
    } else {
#pragma unroll
      for (int i = 0; i < LY::DMA_KQ; ++i) {
        const uint32_t dst = slot + LY::S_K + 1024 * (v + 4 * i);
        if (krow[i] < Lc) dma16(kb_ + koff[i], dst);
        if (WRITE_O && krow[i] < Lc) dma16(qb_ + koff[i], dst + LY::KQ);
      }
      if (scal && l < Lc) dma4(sb + soff, sdst);
#pragma unroll
      for (int i = 0; i < LY::DMA_V; ++i)
        if (vrow[i] < Lc) dma16(vb_ + voff[i], slot + LY::S_V + 1024 * (v + 4 * i));
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
        float *sdst = nullptr;
        if (STORE_STATES) {
          const int cg = p.chunk_base ? p.chunk_base[n_seq] + s : n_seq * p.NC + s;
          sdst = p.states + ((size_t)cg * H + h) * DK * DV;
        }
        chain_chunk<DK, GATED, STORE_STATES, WRITE_O>(p, lb, hs, slot, ob, L, row_base + (size_t)s * CH, h,
                                                      col, sdst);
      }
    } else {
      if (s + 2 < nch) issue(s + 2);
      const int c = s + 1;
      if (c < nch) {
        const uint32_t slot = sbase + (uint32_t)(c % NBUF) * LY::SLOT;
        const uint32_t ob = sbase + LY::OUT_OFF + (uint32_t)(c & 1) * LY::OUTB;
        const uint32_t priv = sbase + LY::PRIV_OFF + (uint32_t)v * LY::PRIV;
        const int L = min(CH, si.len - c * CH);
        if (v == 0) prep_chunk<DK, GATED, WRITE_O, 0>(lb, slot, ob, priv, L, scale);
        else if (v == 1) prep_chunk<DK, GATED, WRITE_O, 1>(lb, slot, ob, priv, L, scale);
        else if (v == 2) prep_chunk<DK, GATED, WRITE_O, 2>(lb, slot, ob, priv, L, scale);
        else prep_chunk<DK, GATED, WRITE_O, 3>(lb, slot, ob, priv, L, scale);
      }
      // K, Q of chunk s + 2 (and everything older) land before the barrier;
      // its V may stay in flight until the next one
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
