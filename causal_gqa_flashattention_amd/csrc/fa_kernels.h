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
  // Query-range split of the dK/dV kernels (nsplit > 1; needs a workspace):
  // a key tile's query-tile list is shared by up to nsplit workgroups (all of
  // them without a mask; under a mask only lists longer than `cs` entries,
  // by ceil(len / cs)), each taking every nc-th entry and writing its fp32
  // dK / dV accumulators to part; the tile's first workgroup writes nc to
  // split_cnt (0 or 1: written directly, nothing to reduce), and
  // fa_dkv_reduce_kernel adds the partials up.
  float* part;          // [B * Hkv][nkt][nsplit][2][BN][D] fp32, or null
  int* split_cnt;       // [B * Hkv][nkt]
  int nsplit, cs;       // 1 and unused without a workspace
  float ksc;            // factor from a dK accumulator to dK (the dV one is 1)
};

// Short-query path (Lq <= kShortMaxLq): the G * Lq (query head, query row)
// pairs of one key/value head form the rows of a workgroup ("packed rows",
// r = head_in_group * Lq + query), so K and V are read once per group, and
// the keys are split into `nsplit` chunks of `chunk` keys whose partial
// results go to a caller workspace and are combined by a second kernel.
constexpr int kShortMaxLq = 8;
struct SplitArgs {
  Tensor q, k, v, o, dO, dq, dk, dv;
  float* lse;           // forward: written; backward: read
  const float* delta;   // backward
  float* part;          // [B * Hkv][R][nsplit][D] fp32: partial O (unnormalised) or dQ (unscaled)
  float* part_ml;       // [B * Hkv][R][nsplit][2] fp32: partial running max (exp2 units) and sum
  int B, Hq, Hkv, Lq, Lk, G, off;
  int R, nrb, nsplit, chunk;  // packed rows per group, 128-row blocks, key chunks, keys per chunk
  float scale, scale_log2;
  // 1 (R <= 32 at D = 256): the four wavefronts of a workgroup split each
  // chunk's key tiles and write a partial each, so nsplit = 4 x chunks
  int wsplit;
};

// Each launcher enqueues on `stream` and returns hipGetLastError().  f16:
// the elements are IEEE half instead of bfloat16.
hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, bool f16, hipStream_t stream);
hipError_t launch_delta(const DeltaArgs& a, int D, bool f16, hipStream_t stream);
// which: 1 = dQ kernel, 2 = dK/dV kernel, 3 = both (dQ first).  With
// a.part set, the dK/dV kernel splits long query lists (a.nsplit, a.cs) and a
// reduction kernel follows it.
hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int which, bool f16, hipStream_t stream);
// keys per dK/dV workgroup of the split path (64 at head dim 256, else 128)
constexpr int dkv_split_keys(int D) { return D > 128 ? 64 : 128; }
// short path: split forward + combine; split dQ + reduce
hipError_t launch_fwd_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream);
hipError_t launch_dq_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream);
// short path dK/dV for R <= 64: nsplit chunks of `chunk` keys
// (a multiple of 128) per key/value head, no workspace
hipError_t launch_dkv_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream);

// The short forward's static scratch array on the current device (looked up
// once per device, then kept): its device address and size in bytes.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace cgqa
