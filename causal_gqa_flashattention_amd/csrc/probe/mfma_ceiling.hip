// Sustained matrix-core throughput on this device, for reading the attention
// kernels' roofline: v_mfma_f32_32x32x16_bf16 back to back, two wavefronts
// per SIMD, four independent accumulators per wavefront, operands held in
// registers.  With random operand bits the chip draws more power per MFMA
// than with constant operands and lowers its clock, so the two runs bracket
// what a kernel can reach on real data.  Not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// stamps (optional): per workgroup, wave 0 records the shader-clock counter
// (s_memtime) and the fixed-rate real-time counter (s_memrealtime) before
// and after its loop, and where it ran: [6 * block] = memtime start, end,
// realtime start, end, HW_ID, XCC_ID
template <bool RANDOM>
__global__ __launch_bounds__(512) void mfma_loop(const uint4* src, float* out, int iters, uint64_t* stamps) {
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 u = RANDOM ? src[(i * 512 + threadIdx.x) % 8192] : src[0];
    const uint4 v = RANDOM ? src[(i * 512 + threadIdx.x + 4096) % 8192] : src[1];
    a[i] = __builtin_bit_cast(bf16x8, u);
    b[i] = __builtin_bit_cast(bf16x8, v);
  }
  f32x16 c[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[n][i] = 0.f;
  uint64_t t0 = 0, r0 = 0;
  if (stamps) {
    r0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) c[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + n) & 7], c[n], 0, 0, 0);
  }
  if (stamps) {
    __builtin_amdgcn_s_waitcnt(0);
    // the last products must have finished: consume every accumulator first
    const float probe = c[0][0] + c[1][0] + c[2][0] + c[3][0];
    __asm__ volatile("; wait for %0" ::"v"(probe));
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x == 0) {
      stamps[6 * blockIdx.x + 0] = t0;
      stamps[6 * blockIdx.x + 1] = t1;
      stamps[6 * blockIdx.x + 2] = r0;
      stamps[6 * blockIdx.x + 3] = r1;
      stamps[6 * blockIdx.x + 4] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
      stamps[6 * blockIdx.x + 5] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
    }
  }
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[n][i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// One wavefront reads the real-time counter until it has advanced by
// `ticks` (at most `max_iters` reads), recording both counters at the start
// and the end: [0] memtime start, [1] end, [2] real-time start, [3] end.
__global__ void counter_spin(uint64_t* stamps, uint64_t ticks, int max_iters) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  uint64_t r = r0;
  for (int i = 0; i < max_iters && r - r0 < ticks; ++i) r = __builtin_amdgcn_s_memrealtime();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (threadIdx.x == 0) {
    stamps[0] = t0;
    stamps[1] = t1;
    stamps[2] = r0;
    stamps[3] = r;
  }
}

}  // namespace

// Rates of the two counters against HIP events: one single-wavefront launch
// that spins on the real-time counter for `ticks` of it; writes the
// real-time and memtime counts per second of event time.  `stamps` is
// device scratch of 4 uint64.  Returns 0, or the HIP error code.
extern "C" int cgqa_counter_rates(uint64_t* stamps, uint64_t ticks, double* realtime_hz, double* memtime_hz) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL(counter_spin, dim3(1), dim3(64), 0, 0, stamps, (uint64_t)1000, 1 << 20);  // warm-up
  (void)hipEventRecord(e0, 0);
  hipLaunchKernelGGL(counter_spin, dim3(1), dim3(64), 0, 0, stamps, ticks, 1 << 22);
  (void)hipEventRecord(e1, 0);
  hipError_t e = hipEventSynchronize(e1);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  uint64_t h[4] = {0, 0, 0, 0};
  if (e == hipSuccess) e = hipMemcpy(h, stamps, sizeof(h), hipMemcpyDeviceToHost);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (e != hipSuccess) return (int)e;
  *realtime_hz = (double)(h[3] - h[2]) / (ms * 1e-3);
  *memtime_hz = (double)(h[1] - h[0]) / (ms * 1e-3);
  return 0;
}

// Runs the loop on `bits` (8192 x 16 bytes of operand data, device memory)
// with one 512-thread workgroup per CU (`cus` workgroups), `reps` timed
// launches after one warm-up, and writes the achieved TFLOP/s for constant
// operands and for the given operands.  `out` is device scratch of
// cus * 512 floats.  Returns 0, or the HIP error code.
extern "C" int cgqa_mfma_ceiling(const void* bits, float* out, int cus, int iters, int reps,
                                 double* tflops_constant, double* tflops_random) {
  const uint4* src = static_cast<const uint4*>(bits);
  const double flop = 2.0 * 32 * 32 * 16 * 32.0 * iters * ((double)cus * 512 / 64);
  auto run = [&](auto kern, double* res) -> int {
    hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters, (uint64_t*)nullptr);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    (void)hipEventRecord(e0, 0);
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters, (uint64_t*)nullptr);
    (void)hipEventRecord(e1, 0);
    const hipError_t e = hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e != hipSuccess) return (int)e;
    *res = flop * reps / (ms * 1e-3) / 1e12;
    return 0;
  };
  int rc = run(mfma_loop<false>, tflops_constant);
  if (rc == 0) rc = run(mfma_loop<true>, tflops_random);
  return rc;
}

// The loops of cgqa_mfma_ceiling again, each timed launch also stamping:
// for constant and for the given operands, the achieved TFLOP/s over `reps`
// launches (HIP events) and the shader clock during the last of them (the
// median over workgroups of memtime ticks per second, the real-time counter
// running at `rt_hz`).  `stamps` is device scratch of 6 * cus uint64; `host`
// host scratch of the same size, left holding the stamps of the last
// random-operand launch.  Returns 0, or the HIP error code.
extern "C" int cgqa_mfma_clock(const void* bits, float* out, uint64_t* stamps, uint64_t* host, int cus,
                               int iters, int reps, double rt_hz, double* tflops_constant, double* ghz_constant,
                               double* tflops_random, double* ghz_random) {
  const uint4* src = static_cast<const uint4*>(bits);
  const double flop = 2.0 * 32 * 32 * 16 * 32.0 * iters * ((double)cus * 512 / 64);
  auto run = [&](auto kern, double* tf, double* ghz) -> int {
    hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters, stamps);  // warm-up
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    (void)hipEventRecord(e0, 0);
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters, stamps);
    (void)hipEventRecord(e1, 0);
    hipError_t e = hipEventSynchronize(e1);
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (e == hipSuccess) e = hipMemcpy(host, stamps, sizeof(uint64_t) * 6 * cus, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return (int)e;
    std::vector<double> g;
    for (int i = 0; i < cus; ++i) {
      const double dt = (double)(host[6 * i + 1] - host[6 * i + 0]);
      const double dr = (double)(host[6 * i + 3] - host[6 * i + 2]);
      if (dr > 0) g.push_back(dt / (dr / rt_hz) / 1e9);
    }
    if (g.empty()) return 1;
    std::nth_element(g.begin(), g.begin() + g.size() / 2, g.end());
    *ghz = g[g.size() / 2];
    *tf = flop * reps / (ms * 1e-3) / 1e12;
    return 0;
  };
  int rc = run(mfma_loop<false>, tflops_constant, ghz_constant);
  if (rc == 0) rc = run(mfma_loop<true>, tflops_random, ghz_random);
  return rc;
}

// One variant of the loops above, `reps` launches back to back (constant
// operands when random == 0): a sustained load for reading the board's power
// and clock from outside.  Returns the elapsed milliseconds (HIP events), or
// a negative HIP error code.
extern "C" double cgqa_mfma_loop(const void* bits, float* out, int cus, int iters, int reps, int random) {
  const uint4* src = static_cast<const uint4*>(bits);
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0;
  (void)hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) {
    if (random)
      hipLaunchKernelGGL(mfma_loop<true>, dim3(cus), dim3(512), 0, 0, src, out, iters, (uint64_t*)nullptr);
    else
      hipLaunchKernelGGL(mfma_loop<false>, dim3(cus), dim3(512), 0, 0, src, out, iters, (uint64_t*)nullptr);
  }
  (void)hipEventRecord(e1, 0);
  const hipError_t e = hipEventSynchronize(e1);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, e0, e1);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return e == hipSuccess ? (double)ms : -(double)e;
}
