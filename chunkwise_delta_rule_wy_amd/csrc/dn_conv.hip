// Depthwise causal short convolution for gfx950 (the DeltaNet rebuttal,
// answer W2: the "short convolution" layers beside the token mixer) and its
// backward:
//
//   y[t, c]  = sum_{j < W} w[c, j] x[t - (W - 1) + j, c]
//   dx[p, c] = sum_{j < W} w[c, j] dy[p + (W - 1) - j, c]
//   dw[c, j] = sum_p x[p, c] dy[p + (W - 1) - j, c]
//
// over the channels c of every head (C = H D of them per token) and only
// between tokens of one sequence (zeros before a sequence's first token).
// The fused variant also L2-normalises every (token, head) row of the output,
// q = z / |z| with z the convolution (a zero row stays zero), the way the
// layer prepares q and k; its backward recomputes z from x and applies
// dz = (dq - u (u . dq)) / |z| (u = z / |z|) before the convolution's adjoint.
//
// A wave owns a run of 32 consecutive tokens and 512 consecutive channels,
// eight per lane, so that each token row is one coalesced 16-byte access per
// lane (bf16; two for fp32); the W - 1 tokens before the run (forward) or
// after it (backward) are read again by the neighbouring wave.  Everything is
// streamed once: the kernels are bound by HBM bandwidth.  In the backward pass
// the eight waves of a workgroup (eight runs, 256 tokens) leave their
// weight-gradient partials in LDS; the workgroup sums them and adds the sums
// to dw with global atomics, consecutive threads on consecutive dw entries.
#include "dn_rows.h"

namespace dn {
namespace {

constexpr int CONV_THREADS = 256;      // forward: four waves, one run each
constexpr int CONV_BWD_THREADS = 512;  // backward: eight waves, one run each
constexpr int CONV_RUN = 32;           // tokens per run
constexpr int CONV_RUNS = CONV_THREADS / 64;
constexpr int CONV_BWD_RUNS = CONV_BWD_THREADS / 64;
constexpr int CONV_LANE_CH = 8;        // channels per lane
constexpr int CONV_WAVE_CH = 64 * CONV_LANE_CH;
constexpr int CONV_BATCH = 8;          // token rows loaded ahead of use (forward)
constexpr int CONV_BWD_BATCH = 4;      // the same for the backward pass (x and dy rows)

// the sequence around token t: [st, nx)
struct SeqTrack {
  const int32_t *cu;
  int N, n;
  int64_t len, st, nx;
  __device__ void init(const ConvParams &p, int64_t t) {
    cu = p.cu;
    N = p.N;
    len = p.T;
    if (!cu) {
      st = t / len * len;
      nx = st + len;
      return;
    }
    int lo = 0, hi = N - 1;  // the last n with cu[n] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
    st = cu[n];
    nx = cu[n + 1];
  }
  __device__ void advance(int64_t t) {
    if (!cu) {
      while (t >= nx) {
        st = nx;
        nx += len;
      }
      return;
    }
    while (t >= nx && n < N - 1) {
      ++n;
      st = cu[n];
      nx = cu[n + 1];
    }
  }
};

template <typename E>
__device__ __forceinline__ void load8(const E *src, float (&x)[CONV_LANE_CH]) {
  float a[Vec16<E>::N];
#pragma unroll
  for (int h = 0; h < CONV_LANE_CH / Vec16<E>::N; ++h) {
    load_row<E>(src + h * Vec16<E>::N, a);
#pragma unroll
    for (int e = 0; e < Vec16<E>::N; ++e) x[h * Vec16<E>::N + e] = a[e];
  }
}

template <typename E>
__device__ __forceinline__ void store8(E *dst, const float (&x)[CONV_LANE_CH]) {
  float a[Vec16<E>::N];
#pragma unroll
  for (int h = 0; h < CONV_LANE_CH / Vec16<E>::N; ++h) {
#pragma unroll
    for (int e = 0; e < Vec16<E>::N; ++e) a[e] = x[h * Vec16<E>::N + e];
    store_row<E>(dst + h * Vec16<E>::N, a);
  }
}

__device__ __forceinline__ void zero8(float (&x)[CONV_LANE_CH]) {
#pragma unroll
  for (int e = 0; e < CONV_LANE_CH; ++e) x[e] = 0.f;
}

template <int W>
__device__ __forceinline__ void load_taps(const ConvParams &p, int64_t c0, bool act, float (&wt)[W][CONV_LANE_CH]) {
#pragma unroll
  for (int e = 0; e < CONV_LANE_CH; ++e)
#pragma unroll
    for (int j = 0; j < W; ++j) wt[j][e] = act ? p.w[(c0 + e) * W + j] : 0.f;
}

// NL > 0: the output rows are L2-normalised over groups of NL lanes (one head
// of 8 NL channels; a wave's 512 channels start at a multiple of 512, so the
// groups align with heads)
template <int NL>
__device__ __forceinline__ void normalise_row(float (&z)[CONV_LANE_CH]) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < CONV_LANE_CH; ++e) ss += z[e] * z[e];
  ss = group_sum<NL>(ss);
  const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
#pragma unroll
  for (int e = 0; e < CONV_LANE_CH; ++e) z[e] *= inv;
}

template <typename E, int W, int NL>
__global__ __launch_bounds__(CONV_THREADS) void conv_fwd_kernel(ConvParams p) {
  const int lane = threadIdx.x & 63, run = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.y * 64 + lane) * CONV_LANE_CH;
  const int64_t t0 = ((int64_t)blockIdx.x * CONV_RUNS + run) * CONV_RUN;
  if (t0 >= p.TT) return;  // the whole wave
  const bool act = c0 < p.C;
  const int64_t t1 = min(t0 + (int64_t)CONV_RUN, p.TT);
  const E *x = static_cast<const E *>(p.x);
  E *y = static_cast<E *>(p.y);
  float wt[W][CONV_LANE_CH];
  load_taps<W>(p, c0, act, wt);
  // hist[k] = x[t - (W - 1) + k], k < W - 1 (the tokens before t)
  float hist[W > 1 ? W - 1 : 1][CONV_LANE_CH];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) {
    const int64_t i = t0 - (W - 1) + k;
    if (act && i >= 0) load8<E>(x + i * p.C + c0, hist[k]);
    else zero8(hist[k]);
  }
  SeqTrack sq;
  sq.init(p, t0);
  for (int b = 0; b < CONV_RUN; b += CONV_BATCH) {
    float xb[CONV_BATCH][CONV_LANE_CH];
#pragma unroll
    for (int i = 0; i < CONV_BATCH; ++i) {
      const int64_t t = t0 + b + i;
      if (act && t < t1) load8<E>(x + t * p.C + c0, xb[i]);
      else zero8(xb[i]);
    }
#pragma unroll
    for (int i = 0; i < CONV_BATCH; ++i) {
      const int64_t t = t0 + b + i;
      if (t >= t1) break;
      sq.advance(t);
      // tap j (< W - 1) reads token t - (W - 1) + j: inside the sequence when j >= lim
      const int64_t lim = sq.st - t + (W - 1);
      float acc[CONV_LANE_CH];
#pragma unroll
      for (int e = 0; e < CONV_LANE_CH; ++e) acc[e] = wt[W - 1][e] * xb[i][e];
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
        if (j >= lim)
#pragma unroll
          for (int e = 0; e < CONV_LANE_CH; ++e) acc[e] += wt[j][e] * hist[j][e];
      if constexpr (NL > 0) normalise_row<NL>(acc);
      if (act) store8<E>(y + t * p.C + c0, acc);
#pragma unroll
      for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) hist[k][e] = hist[k + 1][e];
      if constexpr (W > 1) {
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) hist[W - 2][e] = xb[i][e];
      }
    }
  }
}

// weight gradient: the eight runs' partials summed in LDS, then one atomic
// add per (channel, tap) and workgroup; thread i takes entry i of the
// workgroup's contiguous slice of dw (channel i / W, tap i % W)
template <int W>
__device__ __forceinline__ void dw_flush(const ConvParams &p, float (*part)[W * CONV_LANE_CH * 64],
                                         const float (&dwa)[W][CONV_LANE_CH], int run, int lane) {
  constexpr int PART = W * CONV_LANE_CH * 64;
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int e = 0; e < CONV_LANE_CH; ++e) part[run][(j * CONV_LANE_CH + e) * 64 + lane] = dwa[j][e];
  __syncthreads();
  const int64_t cbase = (int64_t)blockIdx.y * CONV_WAVE_CH;
  for (int i = threadIdx.x; i < PART; i += CONV_BWD_THREADS) {
    const int cl = i / W, j = i % W;
    if (cbase + cl >= p.C) break;
    const int src = (j * CONV_LANE_CH + (cl % CONV_LANE_CH)) * 64 + cl / CONV_LANE_CH;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < CONV_BWD_RUNS; ++r) s += part[r][src];
    atomicAdd(p.dw + cbase * W + i, s);
  }
}

template <typename E, int W>
__global__ __launch_bounds__(CONV_BWD_THREADS) void conv_bwd_kernel(ConvParams p) {
  constexpr int PART = W * CONV_LANE_CH * 64;  // partials of one wave: [j][e][lane]
  __shared__ float part[CONV_BWD_RUNS][PART];
  const int lane = threadIdx.x & 63, run = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.y * 64 + lane) * CONV_LANE_CH;
  const int64_t t0 = ((int64_t)blockIdx.x * CONV_BWD_RUNS + run) * CONV_RUN;
  const bool act = c0 < p.C;
  float dwa[W][CONV_LANE_CH];
#pragma unroll
  for (int j = 0; j < W; ++j) zero8(dwa[j]);
  if (t0 < p.TT) {
    const int64_t t1 = min(t0 + (int64_t)CONV_RUN, p.TT);
    const E *x = static_cast<const E *>(p.x);
    float wt[W][CONV_LANE_CH];
    load_taps<W>(p, c0, act, wt);
    // fut[k] = dy[p + k], k < W: the outputs that position p feeds
    float fut[W][CONV_LANE_CH];
#pragma unroll
    for (int k = 1; k < W; ++k) {
      const int64_t i = t0 + k - 1;
      if (act && i < p.TT) load_f32<CONV_LANE_CH>(p.dy + i * p.C + c0, fut[k]);
      else zero8(fut[k]);
    }
    SeqTrack sq;
    sq.init(p, t0);
    for (int b = 0; b < CONV_RUN; b += CONV_BWD_BATCH) {
      float xb[CONV_BWD_BATCH][CONV_LANE_CH], db[CONV_BWD_BATCH][CONV_LANE_CH];
#pragma unroll
      for (int i = 0; i < CONV_BWD_BATCH; ++i) {
        const int64_t t = t0 + b + i, u = t + (W - 1);
        if (act && t < t1) load8<E>(x + t * p.C + c0, xb[i]);
        else zero8(xb[i]);
        if (act && t < t1 && u < p.TT) load_f32<CONV_LANE_CH>(p.dy + u * p.C + c0, db[i]);
        else zero8(db[i]);
      }
#pragma unroll
      for (int i = 0; i < CONV_BWD_BATCH; ++i) {
        const int64_t t = t0 + b + i;
        if (t >= t1) break;
        sq.advance(t);
#pragma unroll
        for (int k = 0; k + 1 < W; ++k)
#pragma unroll
          for (int e = 0; e < CONV_LANE_CH; ++e) fut[k][e] = fut[k + 1][e];
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) fut[W - 1][e] = db[i][e];
        // output t + k is in the sequence of t when k < lim
        const int64_t lim = sq.nx - t;
        float acc[CONV_LANE_CH];
        zero8(acc);
#pragma unroll
        for (int j = 0; j < W; ++j) {
          const int k = W - 1 - j;
          if (k < lim) {
#pragma unroll
            for (int e = 0; e < CONV_LANE_CH; ++e) {
              acc[e] += wt[j][e] * fut[k][e];
              dwa[j][e] += xb[i][e] * fut[k][e];
            }
          }
        }
        if (act) store_f32<CONV_LANE_CH>(p.dx + t * p.C + c0, acc);
      }
    }
  }
  dw_flush<W>(p, part, dwa, run, lane);
}

// Backward of the fused convolution and normalisation.  At step t the wave
// holds xf[k] = x[t + k] and dzw[k] = dz[t + k] (k < W): it recomputes z at
// u = t + W - 1 (taps x[t .. u] inside u's sequence), turns dq[u] into dz[u],
// then emits dx[t] and the dw terms of x[t] as the plain backward does.  The
// first W - 1 steps of a run (t < t0) only fill the windows.
template <typename E, int W, int NL>
__global__ __launch_bounds__(CONV_BWD_THREADS) void conv_l2_bwd_kernel(ConvParams p) {
  constexpr int PART = W * CONV_LANE_CH * 64;
  __shared__ float part[CONV_BWD_RUNS][PART];
  const int lane = threadIdx.x & 63, run = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.y * 64 + lane) * CONV_LANE_CH;
  const int64_t t0 = ((int64_t)blockIdx.x * CONV_BWD_RUNS + run) * CONV_RUN;
  const bool act = c0 < p.C;
  float dwa[W][CONV_LANE_CH];
#pragma unroll
  for (int j = 0; j < W; ++j) zero8(dwa[j]);
  if (t0 < p.TT) {
    const int64_t t1 = min(t0 + (int64_t)CONV_RUN, p.TT);
    const int64_t ts = t0 - (W - 1);  // first step
    const E *x = static_cast<const E *>(p.x);
    float wt[W][CONV_LANE_CH];
    load_taps<W>(p, c0, act, wt);
    float xf[W][CONV_LANE_CH], dzw[W][CONV_LANE_CH];
#pragma unroll
    for (int k = 0; k < W; ++k) zero8(dzw[k]);
#pragma unroll
    for (int k = 1; k < W; ++k) {  // x[ts + k - 1]: shifted to xf[k - 1] by the first step
      const int64_t i = ts + k - 1;
      if (act && i >= 0 && i < p.TT) load8<E>(x + i * p.C + c0, xf[k]);
      else zero8(xf[k]);
    }
    SeqTrack sqt, squ;
    sqt.init(p, t0);
    squ.init(p, max(ts + (W - 1), (int64_t)0));
    for (int b = 0; b < CONV_RUN + W - 1; b += CONV_BWD_BATCH) {
      float xb[CONV_BWD_BATCH][CONV_LANE_CH], qb[CONV_BWD_BATCH][CONV_LANE_CH];
#pragma unroll
      for (int i = 0; i < CONV_BWD_BATCH; ++i) {
        const int64_t t = ts + b + i, u = t + (W - 1);
        const bool in = act && t < t1 && u >= 0 && u < p.TT;
        if (in) {
          load8<E>(x + u * p.C + c0, xb[i]);
          load_f32<CONV_LANE_CH>(p.dy + u * p.C + c0, qb[i]);
        } else {
          zero8(xb[i]);
          zero8(qb[i]);
        }
      }
#pragma unroll
      for (int i = 0; i < CONV_BWD_BATCH; ++i) {
        const int64_t t = ts + b + i, u = t + (W - 1);
        if (t >= t1) break;
#pragma unroll
        for (int k = 0; k + 1 < W; ++k)
#pragma unroll
          for (int e = 0; e < CONV_LANE_CH; ++e) {
            xf[k][e] = xf[k + 1][e];
            dzw[k][e] = dzw[k + 1][e];
          }
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) xf[W - 1][e] = xb[i][e];
        // z[u] = sum_j w_j x[t + j] over the taps inside u's sequence, then dz[u]
        float z[CONV_LANE_CH], dz[CONV_LANE_CH];
        zero8(z);
        if (u >= 0 && u < p.TT) {
          squ.advance(u);
          const int64_t lo = squ.st - t;  // tap j is inside when j >= lo
#pragma unroll
          for (int j = 0; j < W; ++j)
            if (j >= lo)
#pragma unroll
              for (int e = 0; e < CONV_LANE_CH; ++e) z[e] += wt[j][e] * xf[j][e];
        }
        float ss = 0.f, pd = 0.f;
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) {
          ss += z[e] * z[e];
          pd += z[e] * qb[i][e];
        }
        ss = group_sum<NL>(ss);
        pd = group_sum<NL>(pd);
        const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
        const float cz = pd * inv * inv;
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) dz[e] = (qb[i][e] - z[e] * cz) * inv;
#pragma unroll
        for (int e = 0; e < CONV_LANE_CH; ++e) dzw[W - 1][e] = dz[e];
        if (t < t0) continue;
        sqt.advance(t);
        // dz[t + k] feeds dx[t] when t + k is in t's sequence (k < lim)
        const int64_t lim = sqt.nx - t;
        float acc[CONV_LANE_CH];
        zero8(acc);
#pragma unroll
        for (int j = 0; j < W; ++j) {
          const int k = W - 1 - j;
          if (k < lim) {
#pragma unroll
            for (int e = 0; e < CONV_LANE_CH; ++e) {
              acc[e] += wt[j][e] * dzw[k][e];
              dwa[j][e] += xf[0][e] * dzw[k][e];
            }
          }
        }
        if (act) store_f32<CONV_LANE_CH>(p.dx + t * p.C + c0, acc);
      }
    }
  }
  dw_flush<W>(p, part, dwa, run, lane);
}

__global__ __launch_bounds__(256) void conv_zero_kernel(float *dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = 0.f;
}

template <typename E, int W>
hipError_t launch_w(const ConvParams &p, bool backward, hipStream_t stream) {
  // token blocks on x (up to 2^31 - 1), channel groups of 512 on y
  const unsigned gy = (unsigned)((p.C + CONV_WAVE_CH - 1) / CONV_WAVE_CH);
  const int64_t span = (int64_t)CONV_RUN * (backward ? CONV_BWD_RUNS : CONV_RUNS);
  const dim3 grid((unsigned)((p.TT + span - 1) / span), gy);
  if (backward) {
    const int64_t n = (int64_t)p.C * W;
    hipLaunchKernelGGL(conv_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p.dw, n);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || p.TT == 0) return err;
    if (p.norm_lanes == 16)
      hipLaunchKernelGGL((conv_l2_bwd_kernel<E, W, 16>), grid, dim3(CONV_BWD_THREADS), 0, stream, p);
    else if (p.norm_lanes == 8)
      hipLaunchKernelGGL((conv_l2_bwd_kernel<E, W, 8>), grid, dim3(CONV_BWD_THREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((conv_bwd_kernel<E, W>), grid, dim3(CONV_BWD_THREADS), 0, stream, p);
  } else {
    if (p.TT == 0) return hipSuccess;
    if (p.norm_lanes == 16)
      hipLaunchKernelGGL((conv_fwd_kernel<E, W, 16>), grid, dim3(CONV_THREADS), 0, stream, p);
    else if (p.norm_lanes == 8)
      hipLaunchKernelGGL((conv_fwd_kernel<E, W, 8>), grid, dim3(CONV_THREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((conv_fwd_kernel<E, W, 0>), grid, dim3(CONV_THREADS), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_e(const ConvParams &p, bool backward, hipStream_t stream) {
  switch (p.W) {
    case 1: return launch_w<E, 1>(p, backward, stream);
    case 2: return launch_w<E, 2>(p, backward, stream);
    case 3: return launch_w<E, 3>(p, backward, stream);
    case 4: return launch_w<E, 4>(p, backward, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_conv(const ConvParams &p, int dtype, bool backward, hipStream_t stream) {
  return dtype == 1 ? launch_e<bf16>(p, backward, stream) : launch_e<float>(p, backward, stream);
}

}  // namespace dn
