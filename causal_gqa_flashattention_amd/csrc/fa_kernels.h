// Kernel argument blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

// Block-sparse mask granularity: one entry per 64 query rows x 64 keys.
constexpr int kMaskBlock = 64;

// A strided [B, H, L, D] tensor of 16-bit elements: element (b, h, i, d) is
// at p + b * sb + h * sh + i * sl + d (the D elements of a row contiguous).
struct Tensor {
  uint16_t* p;
  int64_t sb, sh;
  int sl;  // row stride (checked: sl * 128 < 2^31)
  __host__ __device__ uint16_t* head(int b, int h) const { return p + b * sb + h * sh; }
};

struct FwdArgs {
  Tensor q, k, v, o;
  float* lse;
  int B, Hq, Hkv, Lq, Lk, G;
  int off;          // Lk - Lq: causal diagonal offset
  int nqt;          // number of query tiles (set by launch_fwd)
  float scale_log2; // scale * log2(e)
  const uint8_t* mask;  // block mask [ceil(Lq/64)][nkb], nonzero = kept; null: dense
  int nkb;              // ceil(Lk / 64)
};

struct DeltaArgs {
  Tensor o, dO;
  float* delta;  // [H rows of Lq] per batch entry, contiguous
  int H, Lq;
  int64_t rows;  // B * H * Lq
};

struct BwdArgs {
  Tensor q, k, v, dO, dq, dk, dv;
  const float* lse;
  const float* delta;
  int B, Hq, Hkv, Lq, Lk, G;
  int off;
  int nqt;          // query tiles (dQ kernel)
  int nkt;          // key tiles (dK/dV kernel)
  float scale;
  float scale_log2;
  const uint8_t* mask;  // block mask [ceil(Lq/64)][nkb], nonzero = kept; null: dense
  int nkb;              // ceil(Lk / 64)
};

// Each launcher enqueues on `stream` and returns hipGetLastError().  f16:
// the elements are IEEE half instead of bfloat16.
hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, bool f16, hipStream_t stream);
hipError_t launch_delta(const DeltaArgs& a, int D, bool f16, hipStream_t stream);
// which: 1 = dQ kernel, 2 = dK/dV kernel, 3 = both (dQ first).
hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int which, bool f16, hipStream_t stream);

}  // namespace cgqa
