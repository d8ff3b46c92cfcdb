// Device helpers shared by the gfx950 kernels: element types, MFMA wrappers
// and the operand-fragment convention.
//
// Fragment convention.  All matrix products run on 16x16 output tiles with a
// 64-lane wave; lane l belongs to column n = l % 16 and lane group g = l / 16.
// An f32 accumulator tile (f32x4) holds rows 4g + i (i = 0..3) of column n:
// this is the MFMA output layout on CDNA.
//
// A contraction block of 32 indices is split so that lane group g owns the
// 8 indices {4g + i, 16 + 4g + i : i = 0..3}.  Two stacked accumulator tiles
// (rows 0..15 and 16..31 of a matrix whose rows are the contraction index) are
// therefore already a B operand in registers -- no shuffles, no LDS round
// trip.  The A operand is read from a row-major matrix as two 4-element runs
// per lane.  The hardware sums over every (lane group, element) pair, so any
// fixed index assignment is exact as long as A and B share it.
//
// A 16-index block (16x16x16 products) uses indices {4g + i}: one accumulator
// tile is a B operand as is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// B fragment (32-index block) from two accumulator tiles, each value scaled
template <typename E>
__device__ __forceinline__ F32<E> bfrag(const f32x4 &lo, const f32x4 &hi) {
  F32<E> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = to_e<E>(lo[i]);
    r[4 + i] = to_e<E>(hi[i]);
  }
  return r;
}
template <typename E>
__device__ __forceinline__ F16<E> bfrag16(const f32x4 &t) {
  F16<E> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_e<E>(t[i]);
  return r;
}

// Four consecutive E values from LDS (8-byte aligned for bf16, 16 for f32)
template <typename E> struct four;
template <> struct four<bf16> {
  typedef bf16x4 type;
};
template <> struct four<float> {
  typedef f32x4 type;
};

// A fragment (32-index block kb) of row `row` of a row-major LDS matrix
template <typename E>
__device__ __forceinline__ F32<E> afrag(const E *m, int ld, int row, int kb) {
  const int g = lane_id() >> 4;
  const E *p = m + row * ld + kb * 32 + 4 * g;
  typedef typename four<E>::type V4;
  V4 lo = *reinterpret_cast<const V4 *>(p);
  V4 hi = *reinterpret_cast<const V4 *>(p + 16);
  F32<E> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = lo[i];
    r[4 + i] = hi[i];
  }
  return r;
}
// A fragment (16-index block starting at column c0)
template <typename E>
__device__ __forceinline__ F16<E> afrag16(const E *m, int ld, int row, int c0) {
  const int g = lane_id() >> 4;
  typedef typename four<E>::type V4;
  V4 v = *reinterpret_cast<const V4 *>(m + row * ld + c0 + 4 * g);
  F16<E> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = v[i];
  return r;
}
// A fragment (16-index block) from an fp32 row-major LDS matrix, converted
template <typename E>
__device__ __forceinline__ F16<E> afrag16_f(const float *m, int ld, int row, int c0) {
  const int g = lane_id() >> 4;
  f32x4 v = *reinterpret_cast<const f32x4 *>(m + row * ld + c0 + 4 * g);
  F16<E> r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_e<E>(v[i]);
  return r;
}

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

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

}  // namespace dn
