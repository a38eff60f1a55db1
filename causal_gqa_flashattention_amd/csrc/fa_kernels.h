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
  // Query-range split of the dK/dV kernels (nsplit > 1; needs a workspace).
  // A key tile's query-tile list is shared by nc workgroups, chunk c taking
  // every nc-th entry from entry c and writing its fp32 dK / dV accumulators
  // to a slot of `part`; fa_dkv_reduce_kernel adds a tile's slots up.
  //  * Without a mask (plan == null): every list is split min(nsplit, len)
  //    ways; the grid is key tiles x nsplit; slots [B * Hkv][nkt][nsplit];
  //    chunk 0 writes nc to split_cnt.
  //  * Under a mask (plan != null): fa_dkv_count_kernel measures every key
  //    tile's list and fa_dkv_plan_kernel writes plan (int32): [0] the
  //    number of extra chunks J, [1] the chunk length cs, [2] the number of
  //    split tiles, [3 + kt] nc of tile kt (1: written directly),
  //    [3 + nkt + kt] its first slot, [3 + 2 nkt + j] extra chunk j as
  //    kt * kMaxChunks + c (c >= 1), [3 + 2 nkt + jmax + i] split tile i,
  //    [3 + 2 nkt + 2 jmax + kt] the list length of tile kt.  The grid is
  //    nextra = B * Hkv * jmax extra-chunk workgroups (first, so that long
  //    lists start early), then one workgroup per key tile for chunk 0;
  //    slots [B * Hkv][slots].
  float* part;          // fp32 partials [.][2][BN][D] (dK accumulators, then dV), or null
  int* split_cnt;       // [B * Hkv][nkt] (no mask)
  int* plan;            // (mask) see above
  int nsplit, cs;       // chunks per key tile (at most), entries per chunk
  int nextra, jmax, slots;
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
// key tiles a masked call's split plan can hold (Lk <= 262144, 64-key tiles)
constexpr int kMaxPlanTiles = 4096;
// int32 entries of a masked call's split plan
constexpr int64_t dkv_plan_ints(int64_t nkt, int64_t jmax) { return 3 + 3 * nkt + 2 * jmax; }
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
