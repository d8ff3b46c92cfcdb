// Machine probes for the benchmark's roofline: the HBM bandwidth a plain
// streaming copy reaches, the bf16 matrix-core rate a plain MFMA loop reaches,
// and the shader clock.  Built into its own library
// (libdnprobe.so), apart from the operation's library; bench.py times the
// launches with HIP events on the stream it passes, and takes its timing
// events from here too.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 pbf16x8 __attribute__((ext_vector_type(8)));
typedef float pf32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int PROBE_THREADS = 256;  // four waves: one per SIMD of a CU

// Each wave issues `iters` rounds of sixteen 16x16x32 bf16 MFMAs (eight independent chains)
// (16384 flops each) on register operands; the accumulators are summed into
// `sink` so that nothing is dead.
__global__ __launch_bounds__(PROBE_THREADS) void mfma_loop_kernel(int iters, float *sink) {
  const int l = threadIdx.x & 63;
  pbf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(l + i));
    b[i] = (__bf16)(0.001f * (float)(l - i));
  }
  // distinct starting values keep the eight chains distinct
  const float z = (float)l;
  pf32x4 c0 = {z, 0.f, 0.f, 0.f}, c1 = {z + 1.f, 0.f, 0.f, 0.f}, c2 = {z + 2.f, 0.f, 0.f, 0.f},
         c3 = {z + 3.f, 0.f, 0.f, 0.f}, c4 = {z + 4.f, 0.f, 0.f, 0.f}, c5 = {z + 5.f, 0.f, 0.f, 0.f},
         c6 = {z + 6.f, 0.f, 0.f, 0.f}, c7 = {z + 7.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#define DNP_MFMA(c) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0)
    DNP_MFMA(c0); DNP_MFMA(c1); DNP_MFMA(c2); DNP_MFMA(c3);
    DNP_MFMA(c4); DNP_MFMA(c5); DNP_MFMA(c6); DNP_MFMA(c7);
    DNP_MFMA(c0); DNP_MFMA(c1); DNP_MFMA(c2); DNP_MFMA(c3);
    DNP_MFMA(c4); DNP_MFMA(c5); DNP_MFMA(c6); DNP_MFMA(c7);
#undef DNP_MFMA
  }
  const pf32x4 s = c0 + c1 + c2 + c3 + c4 + c5 + c6 + c7;
  sink[blockIdx.x * PROBE_THREADS + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
}

// One wave spins until the shader-clock counter has advanced by `cycles` and
// writes the count it observed.
__global__ __launch_bounds__(64) void clock_kernel(unsigned long long cycles, unsigned long long *out) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned long long t = t0;
  while (t - t0 < cycles) {
    __builtin_amdgcn_s_sleep(1);
    t = __builtin_amdgcn_s_memtime();
  }
  if (threadIdx.x == 0) out[0] = t - t0;
}

// Streaming copy: each thread moves 16-byte units in a grid-stride loop, four
// loads in flight before their stores.
__global__ __launch_bounds__(PROBE_THREADS) void copy_kernel(const uint4 *__restrict__ src,
                                                            uint4 *__restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

// Enqueues a device copy of `bytes` (a multiple of 16; both pointers 16-byte
// aligned) with `grid` workgroups of 256 threads.  Returns 0, -1 for bad
// arguments, or the HIP error code of the launch.
int dnp_copy(const void *src, void *dst, size_t bytes, int grid, hipStream_t stream) {
  if (!src || !dst || grid <= 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return -1;
  if (bytes == 0) return 0;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(PROBE_THREADS), 0, stream, static_cast<const uint4 *>(src),
                     static_cast<uint4 *>(dst), bytes / 16);
  return (int)hipGetLastError();
}

// Flops one dnp_mfma_loop launch performs (grid workgroups of four waves).
double dnp_mfma_loop_flops(int grid, int iters) {
  return (double)grid * 4.0 * (double)iters * 16.0 * 16384.0;
}

// Enqueues the MFMA loop: `grid` workgroups of 256 threads, `iters` rounds of
// sixteen MFMAs per wave; `sink` is device memory of grid * 256 floats.
// Returns 0, or -1 for bad arguments, or the HIP error code of the launch.
int dnp_mfma_loop(int grid, int iters, float *sink, hipStream_t stream) {
  if (grid <= 0 || iters <= 0 || !sink) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(grid), dim3(PROBE_THREADS), 0, stream, iters, sink);
  return (int)hipGetLastError();
}

// Enqueues the clock probe: one wave spins for `cycles` shader-clock cycles
// (at most 2^32) and writes the observed count to out[0] (device memory).
// Returns 0, -1 for bad arguments, or the HIP error code of the launch.
int dnp_clock(unsigned long long cycles, unsigned long long *out, hipStream_t stream) {
  if (cycles == 0 || cycles > (1ull << 32) || !out) return -1;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, stream, cycles, out);
  return (int)hipGetLastError();
}

// Timing events for the benchmark: created with hipEventDisableSystemFence,
// so that recording one does not write back and invalidate the caches at
// system scope (the default event does, which slows the kernels that follow).
// Their timestamps still mark the end of the work enqueued before them on
// the stream.  Each call returns 0 or the HIP error code.
int dnp_event_create(hipEvent_t *ev) {
  if (!ev) return -1;
  return (int)hipEventCreateWithFlags(ev, hipEventDisableSystemFence);
}

int dnp_event_destroy(hipEvent_t ev) { return (int)hipEventDestroy(ev); }

int dnp_event_record(hipEvent_t ev, hipStream_t stream) { return (int)hipEventRecord(ev, stream); }

// Milliseconds between two recorded events; waits for `end` to complete.
int dnp_event_elapsed_ms(hipEvent_t start, hipEvent_t end, float *ms) {
  if (!ms) return -1;
  const hipError_t e = hipEventSynchronize(end);
  if (e != hipSuccess) return (int)e;
  return (int)hipEventElapsedTime(ms, start, end);
}

}  // extern "C"
