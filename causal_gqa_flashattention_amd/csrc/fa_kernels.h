// Kernel argument blocks and host-side launchers (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cgqa {

// Block-sparse mask granularity: one entry per 64 query rows x 64 keys.
constexpr int kMaskBlock = 64;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Lq, Lk, G;
  int off;          // Lk - Lq: causal diagonal offset
  int nqt;          // number of query tiles (set by launch_fwd)
  float scale_log2; // scale * log2(e)
  const uint8_t* mask;  // block mask [ceil(Lq/64)][nkb], nonzero = kept; null: dense
  int nkb;              // ceil(Lk / 64)
};

struct DeltaArgs {
  const uint16_t* o;
  const uint16_t* dO;
  float* delta;
  int64_t rows;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const float* lse;
  const float* delta;
  const uint16_t* dO;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int B, Hq, Hkv, Lq, Lk, G;
  int off;
  int nqt;          // query tiles (dQ kernel)
  int nkt;          // key tiles (dK/dV kernel)
  float scale;
  float scale_log2;
  const uint8_t* mask;  // block mask [ceil(Lq/64)][nkb], nonzero = kept; null: dense
  int nkb;              // ceil(Lk / 64)
};

// Each launcher enqueues on `stream` and returns hipGetLastError().
hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t stream);
// which: 1 = dQ kernel, 2 = dK/dV kernel, 3 = both (dQ first).
hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int which, hipStream_t stream);

}  // namespace cgqa
