// Sustained matrix-core throughput on this device, for reading the attention
// kernels' roofline: v_mfma_f32_32x32x16_bf16 back to back, two wavefronts
// per SIMD, four independent accumulators per wavefront, operands held in
// registers.  With random operand bits the chip draws more power per MFMA
// than with constant operands and lowers its clock, so the two runs bracket
// what a kernel can reach on real data.  Not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <bool RANDOM>
__global__ __launch_bounds__(512) void mfma_loop(const uint4* src, float* out, int iters) {
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
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int n = 0; n < 4; ++n) c[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + n) & 7], c[n], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[n][i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

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
    hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
    (void)hipEventRecord(e0, 0);
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(kern, dim3(cus), dim3(512), 0, 0, src, out, iters);
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
