// Device helpers shared by the gfx950 kernels: element types, MFMA wrappers
// and the operand-fragment convention.
//
// Fragment convention.  All matrix products run on 16x16 output tiles with a
// 64-lane wave; lane l belongs to column n = l % 16 and lane group g = l / 16.
// An f32 accumulator tile (f32x4) holds rows 4g + i (i = 0..3) of column n:
// this is the MFMA output layout on CDNA.
//
// A contraction block of 32 indices gives lane group g the 8 indices
// 8g .. 8g + 7 (one 16-byte bf16 read of an A row).  Which physical index each
// (group, element) slot stands for is free as long as A and B agree: the
// hardware sums over every slot.  dn_chunk.h fixes the row order of the
// accumulator tiles so that two stacked tiles are a B operand in registers.
//
// A 16-index block (16x16x16 products) gives lane group g the indices
// 4g .. 4g + 3: one accumulator tile is a B operand as is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

namespace dn {

constexpr int CH = 64;     // chunk length
constexpr int DVT = 64;    // d_v columns owned by one workgroup
constexpr int NTHR = 256;  // four waves

template <typename E> struct frag32;  // one 32-index operand fragment per lane
template <> struct frag32<bf16> { typedef bf16x8 type; };
template <> struct frag32<float> { typedef f32x8 type; };
template <typename E> struct frag16;  // one 16-index operand fragment per lane
template <> struct frag16<bf16> { typedef bf16x4 type; };
template <> struct frag16<float> { typedef f32x4 type; };

template <typename E> using F32 = typename frag32<E>::type;
template <typename E> using F16 = typename frag16<E>::type;

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// c += a * b over one 32-index block
__device__ __forceinline__ f32x4 mma32(f32x4 c, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x4 c, f32x8 a, f32x8 b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}
// c += a * b over one 16-index block
__device__ __forceinline__ f32x4 mma16(f32x4 c, bf16x4 a, bf16x4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 c, f32x4 a, f32x4 b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

template <typename E> __device__ __forceinline__ E to_e(float x) { return (E)x; }
template <typename E> __device__ __forceinline__ float to_f(E x) { return (float)x; }

// Two fp32 to two bf16 (round to nearest even) in one 32-bit word.  Packing
// through 32-bit words makes the compiler emit one v_cvt_pk_bf16_f32 per pair
// also where the result feeds an MFMA operand (element-wise bf16 vectors are
// converted one value at a time there and then merged with v_perm_b32).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2v));
}
__device__ __forceinline__ bf16x4 cvt_bf16x4(const f32x4 &v) {
  return __builtin_bit_cast(bf16x4, (u32x2){pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])});
}

// B fragment (32-index block) from two stacked accumulator tiles
template <typename E>
__device__ __forceinline__ F32<E> bfrag(const f32x4 &lo, const f32x4 &hi) {
  if constexpr (std::is_same<E, bf16>::value) {
    return __builtin_bit_cast(bf16x8, (u32x4){pk_bf16(lo[0], lo[1]), pk_bf16(lo[2], lo[3]), pk_bf16(hi[0], hi[1]),
                                              pk_bf16(hi[2], hi[3])});
  } else {
    F32<E> r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[i] = to_e<E>(lo[i]);
      r[4 + i] = to_e<E>(hi[i]);
    }
    return r;
  }
}
template <typename E>
__device__ __forceinline__ F16<E> bfrag16(const f32x4 &t) {
  if constexpr (std::is_same<E, bf16>::value) {
    return cvt_bf16x4(t);
  } else {
    F16<E> r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = to_e<E>(t[i]);
    return r;
  }
}

// Four consecutive E values from LDS (8-byte aligned for bf16, 16 for f32)
template <typename E> struct four;
template <> struct four<bf16> {
  typedef bf16x4 type;
};
template <> struct four<float> {
  typedef f32x4 type;
};

// 16 bytes of raw data
struct alignas(16) u128 {
  uint32_t w[4];
};

__device__ __forceinline__ u128 ldg128(const void *p) {
  return *reinterpret_cast<const u128 *>(p);
}
__device__ __forceinline__ u128 zero128() {
  u128 r;
  r.w[0] = r.w[1] = r.w[2] = r.w[3] = 0u;
  return r;
}

// Orders this wave's LDS accesses (other lanes' writes visible to later reads).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wait states between an MFMA and VALU / memory reads of its result when the
// two are separated by control flow.  CDNA does not interlock these reads
// against the matrix pipeline; the compiler's hazard recognizer covers
// straight-line code but has been seen to miss a taken branch between the
// producer and the reader.  24 wait states exceed the longest (16-pass) case.
__device__ __forceinline__ void mfma_settle() {
  __builtin_amdgcn_sched_barrier(0);
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Cross-lane sums on the VALU (DPP and the gfx950 lane swaps), no LDS traffic.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp0(float x) {  // lanes without a source lane read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
// sum over the 16 lanes of each row (every lane gets its row's sum)
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp0<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp0<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp0<0x124>(x);  // row_ror:4
  x += dpp0<0x128>(x);  // row_ror:8
  return x;
}
// x[l] + x[l ^ 16] + x[l ^ 32] + x[l ^ 48]
__device__ __forceinline__ float cross_row_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp0<0x111>(x);       // row_shr:1
  x += dpp0<0x112>(x);       // row_shr:2
  x += dpp0<0x114>(x);       // row_shr:4
  x += dpp0<0x118>(x);       // row_shr:8
  x += dpp0<0x142, 0xa>(x);  // row_bcast:15 into rows 1, 3
  x += dpp0<0x143, 0xc>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return cross_row_sum(row_sum16(x)); }

}  // namespace dn
