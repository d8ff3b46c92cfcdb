// Input prologue of a (Gated) DeltaNet layer, the preparation that the
// workloads apply before the recurrence, fused into one pass per
// (token, head) row, and its backward:
//
//   q = q_in / |q_in|,  k = k_in / |k_in|   (a zero row stays zero)
//   beta = sigmoid(b_in),  g = -c softplus(x_in)
//
//   dq_in = (dq - q (q . dq)) / |q_in|        (likewise dk_in; 0 for a zero row)
//   db_in = dbeta beta (1 - beta),  dx_in = -c sigmoid(x_in) dg
//
// Each row of q and k is read once (16 bytes per lane) and written once; the
// kernels are bound by HBM bandwidth.  softplus is evaluated as
// max(x, 0) + log1p(exp(-|x|)), which neither overflows nor loses the small
// tail.
#include "dn_rows.h"

namespace dn {
namespace {

__device__ __forceinline__ float softplus(float x) { return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x))); }

template <typename E, int DK>
__global__ __launch_bounds__(ROW_THREADS) void prologue_kernel(PrologueParams p) {
  using RM = RowMap<E, DK>;
  constexpr int N = RM::PER;
  const int64_t row = (int64_t)blockIdx.x * RM::RPB + threadIdx.x / RM::LANES;
  const int sub = threadIdx.x % RM::LANES;
  const bool act = row < p.rows;
  const size_t off = (size_t)row * DK + sub * N;
  float q[N], k[N], sq = 0.f, sk = 0.f;
  if (act) {
    load_row<E>(static_cast<const E *>(p.q_in) + off, q);
    load_row<E>(static_cast<const E *>(p.k_in) + off, k);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      sq += q[e] * q[e];
      sk += k[e] * k[e];
    }
  }
  sq = group_sum<RM::LANES>(sq);
  sk = group_sum<RM::LANES>(sk);
  if (!act) return;
  const float iq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f;
  const float ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    q[e] *= iq;
    k[e] *= ik;
  }
  store_row<E>(static_cast<E *>(p.q) + off, q);
  store_row<E>(static_cast<E *>(p.k) + off, k);
  if (sub == 0) {
    p.beta[row] = 1.f / (1.f + expf(-p.b_in[row]));
    if (p.x_in) p.g[row] = -p.gate_scale * softplus(p.x_in[row]);
  }
}

template <typename E, int DK>
__global__ __launch_bounds__(ROW_THREADS) void prologue_bwd_kernel(PrologueParams p) {
  using RM = RowMap<E, DK>;
  constexpr int N = RM::PER;
  const int64_t row = (int64_t)blockIdx.x * RM::RPB + threadIdx.x / RM::LANES;
  const int sub = threadIdx.x % RM::LANES;
  const bool act = row < p.rows;
  const size_t off = (size_t)row * DK + sub * N;
  float q[N], k[N], dq[N], dk[N], sq = 0.f, sk = 0.f, pq = 0.f, pk = 0.f;
  if (act) {
    load_row<E>(static_cast<const E *>(p.q_in) + off, q);
    load_row<E>(static_cast<const E *>(p.k_in) + off, k);
    load_f32<N>(p.dq + off, dq);
    load_f32<N>(p.dk + off, dk);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      sq += q[e] * q[e];
      sk += k[e] * k[e];
      pq += q[e] * dq[e];
      pk += k[e] * dk[e];
    }
  }
  sq = group_sum<RM::LANES>(sq);
  sk = group_sum<RM::LANES>(sk);
  pq = group_sum<RM::LANES>(pq);
  pk = group_sum<RM::LANES>(pk);
  if (!act) return;
  // (dx - u (u . dx)) / n with u = x / n:  (dx - x (x . dx) / n^2) / n
  const float iq = sq > 0.f ? 1.f / sqrtf(sq) : 0.f, ik = sk > 0.f ? 1.f / sqrtf(sk) : 0.f;
  const float cq = pq * iq * iq, ck = pk * ik * ik;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    dq[e] = (dq[e] - q[e] * cq) * iq;
    dk[e] = (dk[e] - k[e] * ck) * ik;
  }
  store_f32<N>(p.dq_in + off, dq);
  store_f32<N>(p.dk_in + off, dk);
  if (sub == 0) {
    const float b = 1.f / (1.f + expf(-p.b_in[row]));
    p.db_in[row] = p.dbeta[row] * b * (1.f - b);
    if (p.x_in) p.dx_in[row] = -p.gate_scale * p.dg[row] / (1.f + expf(-p.x_in[row]));
  }
}

template <typename E, int DK>
hipError_t launch_t(const PrologueParams &p, bool backward, hipStream_t stream) {
  using RM = RowMap<E, DK>;
  const int64_t blocks = (p.rows + RM::RPB - 1) / RM::RPB;
  if (blocks == 0) return hipSuccess;
  if (backward)
    hipLaunchKernelGGL((prologue_bwd_kernel<E, DK>), dim3((unsigned)blocks), dim3(ROW_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL((prologue_kernel<E, DK>), dim3((unsigned)blocks), dim3(ROW_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueParams &p, int dtype, int DK, bool backward, hipStream_t stream) {
  if (dtype == 1) return DK == 64 ? launch_t<bf16, 64>(p, backward, stream) : launch_t<bf16, 128>(p, backward, stream);
  return DK == 64 ? launch_t<float, 64>(p, backward, stream) : launch_t<float, 128>(p, backward, stream);
}

}  // namespace dn
