// One recurrent (decode) step of the gated delta rule per (batch, head):
//
//   u = h^T k,  p = h^T q               (h = S^T, d_k x d_v, fp32)
//   d = v - alpha u
//   h' = alpha h + beta k d^T           (= (alpha S (I - beta k k^T) + beta v k^T)^T)
//   o  = h'^T q = alpha p + beta (k . q) d
//
// The step reads and writes the whole state once and does ~4 flops per state
// element, so it is bound by HBM bandwidth (Gated DeltaNet review thread,
// General Response 2: recurrent inference speed is set by state size).  One
// workgroup streams a 128-column slice of one state: each thread keeps 4
// columns of d_k/8 rows in registers between the reduction and the update,
// so every state byte crosses HBM exactly twice.
#include "dn_internal.h"

namespace dn {

constexpr int STEP_COLS = 128;

template <typename E, int DK>
__global__ __launch_bounds__(NTHR) void step_kernel(StepParams p) {
  constexpr int CG = STEP_COLS / 4;  // column groups of 4
  constexpr int RG = NTHR / CG;      // row groups
  constexpr int RPT = DK / RG;       // rows per thread
  __shared__ float s_u[RG][STEP_COLS];
  __shared__ float s_p[RG][STEP_COLS];
  __shared__ float s_k[DK], s_q[DK];
  __shared__ float s_kq;

  const int nsl = (p.DV + STEP_COLS - 1) / STEP_COLS;
  const int bh = blockIdx.x / nsl, sl = blockIdx.x % nsl;
  const int t = threadIdx.x, cg = t % CG, rg = t / CG;
  const int c0 = sl * STEP_COLS + 4 * cg;
  const bool active = c0 < p.DV;

  const E *q = static_cast<const E *>(p.q) + (size_t)bh * DK;
  const E *k = static_cast<const E *>(p.k) + (size_t)bh * DK;
  const E *v = static_cast<const E *>(p.v) + (size_t)bh * p.DV;
  float *st = p.state + (size_t)bh * DK * p.DV;

  for (int i = t; i < DK; i += NTHR) {
    s_k[i] = to_f<E>(k[i]);
    s_q[i] = to_f<E>(q[i]);
  }
  f32x4 hv[RPT];
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      hv[i] = *reinterpret_cast<const f32x4 *>(st + (size_t)(rg + RG * i) * p.DV + c0);
  }
  __syncthreads();
  if (t < 64) {
    float part = 0.f;
    for (int i = t; i < DK; i += 64) part += s_k[i] * s_q[i];
    part = wave_sum(part);
    if (t == 0) s_kq = part;
  }
  f32x4 u = zero4(), pq = zero4();
  if (active) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float ki = s_k[rg + RG * i], qi = s_q[rg + RG * i];
      u += hv[i] * ki;
      pq += hv[i] * qi;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s_u[rg][4 * cg + e] = u[e];
    s_p[rg][4 * cg + e] = pq[e];
  }
  __syncthreads();
  if (!active) return;
  f32x4 ut = zero4(), pt = zero4();
#pragma unroll
  for (int r = 0; r < RG; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ut[e] += s_u[r][4 * cg + e];
      pt[e] += s_p[r][4 * cg + e];
    }
  const float alpha = p.g ? __expf(p.g[bh]) : 1.f;
  const float beta = p.beta[bh];
  f32x4 d;
#pragma unroll
  for (int e = 0; e < 4; ++e) d[e] = to_f<E>(v[c0 + e]) - alpha * ut[e];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float bk = beta * s_k[rg + RG * i];
    *reinterpret_cast<f32x4 *>(st + (size_t)(rg + RG * i) * p.DV + c0) = alpha * hv[i] + bk * d;
  }
  if (rg == 0) {
    E *o = static_cast<E *>(p.o) + (size_t)bh * p.DV;
    const float bkq = beta * s_kq;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[c0 + e] = to_e<E>(alpha * pt[e] + bkq * d[e]);
  }
}

hipError_t launch_step(const StepParams &p, int dtype, int DK, hipStream_t stream) {
  const int nsl = (p.DV + STEP_COLS - 1) / STEP_COLS;
  const int grid = p.B * p.H * nsl;
  if (grid == 0) return hipSuccess;
  if (dtype == 1) {
    if (DK == 64)
      hipLaunchKernelGGL((step_kernel<bf16, 64>), dim3(grid), dim3(NTHR), 0, stream, p);
    else
      hipLaunchKernelGGL((step_kernel<bf16, 128>), dim3(grid), dim3(NTHR), 0, stream, p);
  } else {
    if (DK == 64)
      hipLaunchKernelGGL((step_kernel<float, 64>), dim3(grid), dim3(NTHR), 0, stream, p);
    else
      hipLaunchKernelGGL((step_kernel<float, 128>), dim3(grid), dim3(NTHR), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace dn
