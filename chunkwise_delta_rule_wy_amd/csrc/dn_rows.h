// Row-wise streaming helpers for the per-(token, head) kernels: a row of Dk
// elements is read by Dk / N lanes, 16 bytes each (N = 8 for bf16, 4 for
// fp32); the lanes of a row sit in one wave, so row sums are lane shuffles.
#pragma once

#include "dn_internal.h"

namespace dn {

constexpr int ROW_THREADS = 256;

template <typename E> struct Vec16;  // 16 bytes of a row
template <> struct Vec16<bf16> { typedef bf16x8 type; static constexpr int N = 8; };
template <> struct Vec16<float> { typedef f32x4 type; static constexpr int N = 4; };

template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) x += __shfl_xor(x, m, 64);
  return x;
}

template <typename E, int DK>
struct RowMap {
  static constexpr int PER = Vec16<E>::N;          // row elements per lane
  static constexpr int LANES = DK / PER;           // lanes per row (8 .. 32)
  static constexpr int RPB = ROW_THREADS / LANES;  // rows per workgroup
  static_assert(LANES <= 64 && 64 % LANES == 0, "a row sits in one wave");
};

template <typename E>
__device__ __forceinline__ void load_row(const E *src, float (&x)[Vec16<E>::N]) {
  const typename Vec16<E>::type v = *reinterpret_cast<const typename Vec16<E>::type *>(src);
#pragma unroll
  for (int e = 0; e < Vec16<E>::N; ++e) x[e] = to_f<E>(v[e]);
}

template <typename E>
__device__ __forceinline__ void store_row(E *dst, const float (&x)[Vec16<E>::N]) {
  typename Vec16<E>::type v;
#pragma unroll
  for (int e = 0; e < Vec16<E>::N; ++e) v[e] = to_e<E>(x[e]);
  *reinterpret_cast<typename Vec16<E>::type *>(dst) = v;
}

// fp32 row slice of N elements (N / 4 16-byte accesses)
template <int N>
__device__ __forceinline__ void load_f32(const float *src, float (&x)[N]) {
#pragma unroll
  for (int e = 0; e < N; e += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(src + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[e + i] = v[i];
  }
}
template <int N>
__device__ __forceinline__ void store_f32(float *dst, const float (&x)[N]) {
#pragma unroll
  for (int e = 0; e < N; e += 4) *reinterpret_cast<f32x4 *>(dst + e) = (f32x4){x[e], x[e + 1], x[e + 2], x[e + 3]};
}

}  // namespace dn
