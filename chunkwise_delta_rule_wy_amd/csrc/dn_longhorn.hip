// Longhorn step size (Gated DeltaNet review thread, Table 1, row "Longhorn",
// with the caption's scalar beta): the delta-rule update at
//
//   eps = beta / (1 + beta s),   s = |k|^2,
//
// per (token, head), and its backward:
//
//   dbeta = deps / (1 + beta s)^2,   dk += deps * (-2 beta^2 / (1 + beta s)^2) k.
//
// The recurrence itself runs in the chunkwise kernels with beta := eps.  Both
// kernels read each key row once, 16 bytes per lane (Dk / 8 lanes for bf16,
// Dk / 4 for fp32), and are bound by HBM bandwidth; the squared norm is a sum
// over the row's lanes, which sit in one wave.
#include "dn_rows.h"

namespace dn {
namespace {

template <typename E, int DK>
__global__ __launch_bounds__(ROW_THREADS) void eps_kernel(const E *__restrict__ k, const float *__restrict__ beta,
                                                         float *__restrict__ eps, int64_t rows) {
  using RM = RowMap<E, DK>;
  const int64_t row = (int64_t)blockIdx.x * RM::RPB + threadIdx.x / RM::LANES;
  const int sub = threadIdx.x % RM::LANES;
  float s = 0.f;
  if (row < rows) {
    const typename Vec16<E>::type kv =
        *reinterpret_cast<const typename Vec16<E>::type *>(k + row * DK + sub * RM::PER);
#pragma unroll
    for (int e = 0; e < RM::PER; ++e) {
      const float x = to_f<E>(kv[e]);
      s += x * x;
    }
  }
  s = group_sum<RM::LANES>(s);
  if (row < rows && sub == 0) {
    const float b = beta[row];
    eps[row] = b / (1.f + b * s);
  }
}

template <typename E, int DK>
__global__ __launch_bounds__(ROW_THREADS) void eps_bwd_kernel(const E *__restrict__ k, const float *__restrict__ beta,
                                                             const float *deps, float *dbeta, float *__restrict__ dk,
                                                             int64_t rows) {
  using RM = RowMap<E, DK>;
  const int64_t row = (int64_t)blockIdx.x * RM::RPB + threadIdx.x / RM::LANES;
  const int sub = threadIdx.x % RM::LANES;
  float kf[RM::PER];
  float s = 0.f, b = 0.f, de = 0.f;
  if (row < rows) {
    // every lane reads deps before any lane of the row writes dbeta (which may alias it)
    b = beta[row];
    de = deps[row];
    const typename Vec16<E>::type kv =
        *reinterpret_cast<const typename Vec16<E>::type *>(k + row * DK + sub * RM::PER);
#pragma unroll
    for (int e = 0; e < RM::PER; ++e) {
      kf[e] = to_f<E>(kv[e]);
      s += kf[e] * kf[e];
    }
  }
  s = group_sum<RM::LANES>(s);
  if (row >= rows) return;
  const float den = 1.f + b * s;
  const float inv2 = 1.f / (den * den);
  const float c = -2.f * b * b * de * inv2;
  float *dkr = dk + row * DK + sub * RM::PER;
#pragma unroll
  for (int e = 0; e < RM::PER; e += 4) {
    f32x4 d = *reinterpret_cast<const f32x4 *>(dkr + e);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] += c * kf[e + i];
    *reinterpret_cast<f32x4 *>(dkr + e) = d;
  }
  if (sub == 0) dbeta[row] = de * inv2;
}

template <typename E, int DK>
hipError_t launch_t(const LonghornParams &p, hipStream_t stream) {
  using RM = RowMap<E, DK>;
  const int64_t blocks = (p.rows + RM::RPB - 1) / RM::RPB;
  if (blocks == 0) return hipSuccess;
  const E *k = static_cast<const E *>(p.k);
  if (p.dk)
    hipLaunchKernelGGL((eps_bwd_kernel<E, DK>), dim3((unsigned)blocks), dim3(ROW_THREADS), 0, stream, k, p.beta,
                       p.deps, p.dbeta, p.dk, p.rows);
  else
    hipLaunchKernelGGL((eps_kernel<E, DK>), dim3((unsigned)blocks), dim3(ROW_THREADS), 0, stream, k, p.beta, p.eps,
                       p.rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_longhorn(const LonghornParams &p, int dtype, int DK, hipStream_t stream) {
  if (dtype == 1) return DK == 64 ? launch_t<bf16, 64>(p, stream) : launch_t<bf16, 128>(p, stream);
  return DK == 64 ? launch_t<float, 64>(p, stream) : launch_t<float, 128>(p, stream);
}

}  // namespace dn
