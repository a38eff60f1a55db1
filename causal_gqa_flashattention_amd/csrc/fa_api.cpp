// C ABI of the library: argument validation and per-head-dimension dispatch.
//
// All checks run on the host before anything is enqueued; a failed check
// returns a typed status and launches nothing (no silent fallback: page
// "When the Bottleneck Moved", section 3, on unsupported cases failing with
// typed errors; runtime rather than debug-only shape/stride checks and the
// null-buffer check: page "feat(attention): complete Flash Attention VJP
// implementation", review-comment resolutions).  Supported head dimensions:
// 64, 96, 128 and 256, forward and backward (the VJP page's Metal backward
// stops at 128 for a 32 KB threadgroup-memory limit that gfx950's 160 KB LDS
// does not have).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr int kDqBM = 128;    // query rows per dQ workgroup

bool fwd_head_dim_ok(int D) { return D == 64 || D == 96 || D == 128 || D == 256; }
bool bwd_head_dim_ok(int D) { return D == 64 || D == 96 || D == 128 || D == 256; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Count of elements of a [n0, n1, n2, n3] tensor, or -1 on int64 overflow.
int64_t elems(int64_t n0, int64_t n1, int64_t n2, int64_t n3) {
  const int64_t lim = INT64_MAX / 4;
  int64_t r = 1;
  for (int64_t n : {n0, n1, n2, n3}) {
    if (n != 0 && r > lim / n) return -1;
    r *= n;
  }
  return r;
}

fa_status check_sizes(int B, int Hq, int Hkv, int Lq, int Lk, int D, bool causal) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Lq < 0 || Lk < 0) return FA_ERR_SHAPE;
  if (Hq > 0 && Hkv == 0) return FA_ERR_GQA;
  if (Hkv > 0 && Hq % Hkv != 0) return FA_ERR_GQA;
  if (Lq > 0 && Lk == 0) return FA_ERR_SHAPE;
  if (causal && Lq > Lk) return FA_ERR_CAUSAL_LQ_GT_LK;
  if (elems(B, Hq, Lq, D) < 0 || elems(B, Hkv, Lk, D) < 0) return FA_ERR_SHAPE;
  // block counts must fit a 32-bit grid dimension
  const int64_t nq = (int64_t)B * Hq * (((int64_t)Lq + 63) / 64);
  const int64_t nk = (int64_t)B * Hkv * (((int64_t)Lk + 63) / 64);
  if (nq > INT32_MAX || nk > INT32_MAX) return FA_ERR_SHAPE;
  static_assert(FA_MASK_BLOCK == cgqa::kMaskBlock, "mask granularity");
  return FA_OK;
}

fa_status check_ptr(const void* p) {
  if (p == nullptr) return FA_ERR_NULL;
  if (!aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

fa_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  return FA_OK;
}

#define FA_TRY(expr)                   \
  do {                                 \
    const fa_status st_ = (expr);      \
    if (st_ != FA_OK) return st_;      \
  } while (0)

// A strided [B, H, L, D] operand: pointer checks, then strides.  Strides of
// dimensions of extent 1 are never used and are ignored.  Every used stride
// is >= 0 and a multiple of 8 elements (16-byte rows and heads), the row
// stride is below 2^24 (tile offsets are 32-bit), and the last element's
// offset fits in int64.  An output must not overlap itself: taken in order
// of increasing stride, each dimension's stride is at least the span of the
// dimensions inside it (the D elements of a row first).
fa_status check_tensor(const fa_tensor& t, int B, int H, int L, int D, bool output) {
  FA_TRY(check_ptr(t.data));
  struct Dim { int64_t stride, extent; } dims[3] = {{t.stride_b, B}, {t.stride_h, H}, {t.stride_l, L}};
  int64_t last = D;
  for (Dim& d : dims) {
    if (d.extent <= 1) {
      d.stride = 0;
      continue;
    }
    if (d.stride < 0 || d.stride % 8 != 0) return FA_ERR_STRIDE;
    if (d.stride > (INT64_MAX / 4 - last) / (d.extent - 1)) return FA_ERR_SHAPE;
    last += d.stride * (d.extent - 1);
  }
  if (L > 1 && t.stride_l >= (int64_t{1} << 24)) return FA_ERR_STRIDE;
  if (output) {
    // insertion sort of the used dimensions by stride
    Dim used[3];
    int n = 0;
    for (const Dim& d : dims)
      if (d.extent > 1) {
        int j = n++;
        while (j > 0 && used[j - 1].stride > d.stride) {
          used[j] = used[j - 1];
          --j;
        }
        used[j] = d;
      }
    int64_t span = D;  // elements covered by the dimensions inside
    for (int j = 0; j < n; ++j) {
      if (used[j].stride < span) return FA_ERR_STRIDE;
      span = used[j].stride * used[j].extent;
    }
  }
  return FA_OK;
}

fa_tensor dense(const void* p, int H, int L, int D) {
  return fa_tensor{const_cast<void*>(p), (int64_t)H * L * D, (int64_t)L * D, (int64_t)D};
}

// (a row stride that check_tensor did not bound belongs to a dimension of
// extent <= 1 and is never used)
cgqa::Tensor to_kernel(const fa_tensor& t) {
  const int64_t sl = t.stride_l >= 0 && t.stride_l < (int64_t{1} << 24) ? t.stride_l : 0;
  return cgqa::Tensor{static_cast<uint16_t*>(t.data), t.stride_b, t.stride_h, (int)sl};
}

bool dtype_ok(fa_dtype d) { return d == FA_BF16 || d == FA_F16; }

}  // namespace

extern "C" {

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FA_ERR_SHAPE: return "invalid or overflowing sizes";
    case FA_ERR_HEAD_DIM: return "head dimension not supported by this call";
    case FA_ERR_GQA: return "query heads are not a multiple of key/value heads";
    case FA_ERR_CAUSAL_LQ_GT_LK: return "causal attention needs Lq <= Lk";
    case FA_ERR_SCALE: return "scale must be finite and positive";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_STRIDE:
      return "a stride is negative, not a multiple of 8 elements or too large, or makes an output overlap itself";
    case FA_ERR_DTYPE: return "unknown element type";
    case FA_ERR_WORKSPACE: return "workspace too small (see fa_short_workspace_bytes)";
  }
  return "unknown status";
}

const char* fa_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"

namespace {

fa_status fwd_common(const fa_tensor& q, const fa_tensor& k, const fa_tensor& v, const fa_tensor& o,
                     float* lse, int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, fa_dtype dtype, const unsigned char* block_mask, void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (!fwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (block_mask && (Lq > FA_MASK_MAX_LEN || Lk > FA_MASK_MAX_LEN)) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  if (B == 0 || Hq == 0 || Lq == 0) return FA_OK;
  for (const void* p : {(const void*)q.data, (const void*)k.data, (const void*)v.data, (const void*)o.data,
                        (const void*)lse}) FA_TRY(check_ptr(p));
  FA_TRY(check_tensor(q, B, Hq, Lq, D, false));
  FA_TRY(check_tensor(k, B, Hkv, Lk, D, false));
  FA_TRY(check_tensor(v, B, Hkv, Lk, D, false));
  FA_TRY(check_tensor(o, B, Hq, Lq, D, true));

  cgqa::FwdArgs a;
  a.q = to_kernel(q);
  a.k = to_kernel(k);
  a.v = to_kernel(v);
  a.o = to_kernel(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.G = Hq / Hkv;
  a.off = Lk - Lq;
  a.nqt = 0;  // set by the launcher from the kernel's tile height
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = reinterpret_cast<const uint8_t*>(block_mask);
  a.nkb = (Lk + cgqa::kMaskBlock - 1) / cgqa::kMaskBlock;
  const hipError_t e = cgqa::launch_fwd(a, D, causal != 0, dtype == FA_F16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status delta_common(const fa_tensor& o, const fa_tensor& dO, float* delta, int B, int H, int Lq,
                       int D, fa_dtype dtype, void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (!fwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || Lq < 0) return FA_ERR_SHAPE;
  const int64_t n = elems(B, H, Lq, D);
  if (n < 0) return FA_ERR_SHAPE;
  if (n == 0) return FA_OK;
  for (const void* p : {(const void*)o.data, (const void*)dO.data, (const void*)delta}) FA_TRY(check_ptr(p));
  FA_TRY(check_tensor(o, B, H, Lq, D, false));
  FA_TRY(check_tensor(dO, B, H, Lq, D, false));
  cgqa::DeltaArgs a;
  a.o = to_kernel(o);
  a.dO = to_kernel(dO);
  a.delta = delta;
  a.H = H;
  a.Lq = Lq;
  a.rows = (int64_t)B * H * Lq;
  if (a.rows / 8 > INT32_MAX || (int64_t)B * H > INT32_MAX) return FA_ERR_SHAPE;
  const hipError_t e = cgqa::launch_delta(a, D, dtype == FA_F16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Query-range split of the dK/dV kernel (calls with a workspace).  A key
// tile's work is its query-tile list times the group size.  Under a causal
// mask the first key tile sees every query tile, the last almost none: with
// at least two workgroups per CU the hardware's heaviest-first rounds pair
// them up, with fewer the kernel lasts as long as the first tile.  So without
// a mask, when there are fewer than 512 key-tile workgroups (two per CU),
// every list is split until there are about 1024 workgroups (at most 8
// chunks).  A block mask can hand one key tile every query tile (a sink or
// global column) while the others see few: then a planning kernel measures
// the lists on the device and splits only the long ones, with at most
// jmax = max(16, nkt / 4) extra chunks per head.
struct DkvSplit {
  int nsplit, jmax;
  size_t part_bytes, bytes;
};

DkvSplit dkv_split_plan(int B, int Hkv, int Lq, int Lk, int D, bool masked) {
  DkvSplit p{1, 0, 0, 0};
  if (B <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || !bwd_head_dim_ok(D)) return p;
  if (masked && (Lq > FA_MASK_MAX_LEN || Lk > FA_MASK_MAX_LEN)) return p;
  const int bnk = cgqa::dkv_split_keys(D);
  const int64_t nkt = ((int64_t)Lk + bnk - 1) / bnk;
  const int64_t nh = (int64_t)B * Hkv;
  const int64_t wgs = nh * nkt;
  const int64_t nqt = ((int64_t)Lq + 63) / 64;
  const size_t slot_bytes = (size_t)2 * bnk * D * sizeof(float);
  if (masked) {
    if (nqt < 2 || nkt > cgqa::kMaxPlanTiles) return p;
    const int64_t jmax = std::max<int64_t>(16, (nkt + 3) / 4);
    if (wgs + nh * jmax > INT32_MAX || nh * jmax * 8 > INT32_MAX) return p;
    p.nsplit = 8;
    p.jmax = (int)jmax;
    p.part_bytes = (size_t)(nh * 2 * jmax) * slot_bytes;
    p.bytes = p.part_bytes + (((size_t)cgqa::dkv_plan_ints(nkt, jmax) * sizeof(int) + 255) & ~(size_t)255);
    return p;
  }
  if (wgs >= 512 || wgs * 8 > INT32_MAX) return p;
  int64_t S = 2;
  while (S < 8 && wgs * S < 1024) S *= 2;
  S = std::min<int64_t>(S, nqt);
  if (S <= 1) return p;
  p.nsplit = (int)S;
  p.part_bytes = (size_t)(wgs * S) * slot_bytes;
  p.bytes = p.part_bytes + (((size_t)wgs * sizeof(int) + 255) & ~(size_t)255);
  return p;
}

// Shared body of every backward call.  which: FA_GRAD_DQ and/or FA_GRAD_DKV.
// A workspace (may be NULL) lets the dK/dV kernel split long query lists.
fa_status bwd_common(const fa_tensor& q, const fa_tensor& k, const fa_tensor& v, const float* lse,
                     const float* delta, const fa_tensor& dO, const fa_tensor& dq, const fa_tensor& dk,
                     const fa_tensor& dv, int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, fa_dtype dtype, const unsigned char* block_mask, unsigned which,
                     void* stream, bool ws_call = false, void* workspace = nullptr,
                     size_t workspace_bytes = 0) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (!bwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (block_mask && (Lq > FA_MASK_MAX_LEN || Lk > FA_MASK_MAX_LEN)) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  which &= FA_GRAD_DQ | FA_GRAD_DKV;
  if (B == 0 || Hq == 0) return FA_OK;
  // dk/dv are written whenever keys exist (zeros when there is no query row);
  // dq only when there are query rows.
  if (Lq == 0) which &= FA_GRAD_DKV;
  if (Lk == 0) which &= FA_GRAD_DQ;
  if (which == 0) return FA_OK;
  FA_TRY(check_ptr(k.data));
  FA_TRY(check_ptr(v.data));
  if (Lq > 0)
    for (const void* p : {(const void*)q.data, (const void*)lse, (const void*)delta, (const void*)dO.data}) FA_TRY(check_ptr(p));
  if (which & FA_GRAD_DQ) FA_TRY(check_ptr(dq.data));
  if (which & FA_GRAD_DKV) {
    FA_TRY(check_ptr(dk.data));
    FA_TRY(check_ptr(dv.data));
  }
  FA_TRY(check_tensor(k, B, Hkv, Lk, D, false));
  FA_TRY(check_tensor(v, B, Hkv, Lk, D, false));
  if (Lq > 0) {
    FA_TRY(check_tensor(q, B, Hq, Lq, D, false));
    FA_TRY(check_tensor(dO, B, Hq, Lq, D, false));
  }
  if (which & FA_GRAD_DQ) FA_TRY(check_tensor(dq, B, Hq, Lq, D, true));
  if (which & FA_GRAD_DKV) {
    FA_TRY(check_tensor(dk, B, Hkv, Lk, D, true));
    FA_TRY(check_tensor(dv, B, Hkv, Lk, D, true));
  }

  DkvSplit split{1, 0, 0, 0};
  if (ws_call && (which & FA_GRAD_DKV)) {
    split = dkv_split_plan(B, Hkv, Lq, Lk, D, block_mask != nullptr);
    if (split.nsplit > 1) {
      FA_TRY(check_ptr(workspace));
      if (workspace_bytes < split.bytes) return FA_ERR_WORKSPACE;
    }
  }

  cgqa::BwdArgs a{};
  a.q = to_kernel(q);
  a.k = to_kernel(k);
  a.v = to_kernel(v);
  a.dO = to_kernel(dO);
  a.dq = to_kernel(dq);
  a.dk = to_kernel(dk);
  a.dv = to_kernel(dv);
  a.lse = lse;
  a.delta = delta;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.G = Hq / Hkv;
  a.off = Lk - Lq;
  a.nqt = (Lq + kDqBM - 1) / kDqBM;
  a.nkt = 0;  // set by the launcher from the dK/dV kernel's key tile
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = reinterpret_cast<const uint8_t*>(block_mask);
  a.nkb = (Lk + cgqa::kMaskBlock - 1) / cgqa::kMaskBlock;
  a.nsplit = 1;
  if (split.nsplit > 1) {
    a.part = static_cast<float*>(workspace);
    int* tail = reinterpret_cast<int*>(static_cast<char*>(workspace) + split.part_bytes);
    a.nsplit = split.nsplit;
    if (block_mask != nullptr) {
      a.plan = tail;
      a.jmax = split.jmax;
      a.slots = 2 * split.jmax;
      a.nextra = B * Hkv * split.jmax;
    } else {
      a.split_cnt = tail;
    }
  }
  const hipError_t e = cgqa::launch_bwd(a, D, causal != 0, (int)which, dtype == FA_F16,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// Contiguous bf16 tensors of the plain calls.
struct Dense {
  int B, Hq, Hkv, Lq, Lk, D;
  fa_tensor q(const void* p) const { return dense(p, Hq, Lq, D); }
  fa_tensor kv(const void* p) const { return dense(p, Hkv, Lk, D); }
};

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return fwd_common(t.q(q), t.kv(k), t.kv(v), t.q(o), lse, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                    FA_BF16, nullptr, stream);
}

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return fwd_common(t.q(q), t.kv(k), t.kv(v), t.q(o), lse, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                    FA_BF16, block_mask, stream);
}

fa_status fa_fwd_ex(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype, block_mask, stream);
}

fa_status fa_bwd_delta(const void* o, const void* dO, float* delta,
                       int B, int H, int Lq, int D, void* stream) {
  return delta_common(dense(o, H, Lq, D), dense(dO, H, Lq, D), delta, B, H, Lq, D, FA_BF16, stream);
}

fa_status fa_bwd_delta_ex(fa_tensor o, fa_tensor dO, float* delta, int B, int H, int Lq, int D,
                          fa_dtype dtype, void* stream) {
  return delta_common(o, dO, delta, B, H, Lq, D, dtype, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const float* delta, const void* dO,
                 void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream) {
  (void)o;  // O enters the backward only through delta
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(dq), t.kv(dk), t.kv(dv),
                    B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, nullptr, FA_GRAD_DQ | FA_GRAD_DKV,
                    stream);
}

fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const float* delta, const void* dO,
                              void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream) {
  (void)o;
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(dq), t.kv(dk), t.kv(dv),
                    B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, block_mask,
                    FA_GRAD_DQ | FA_GRAD_DKV, stream);
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dO, void* dq,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                    int causal, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(dq), t.kv(nullptr),
                    t.kv(nullptr), B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, nullptr, FA_GRAD_DQ,
                    stream);
}

fa_status fa_bwd_dq_block_sparse(const void* q, const void* k, const void* v,
                                 const float* lse, const float* delta, const void* dO, void* dq,
                                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                 int causal, const unsigned char* block_mask, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(dq), t.kv(nullptr),
                    t.kv(nullptr), B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, block_mask,
                    FA_GRAD_DQ, stream);
}

fa_status fa_bwd_dkv(const void* q, const void* k, const void* v,
                     const float* lse, const float* delta, const void* dO,
                     void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(nullptr), t.kv(dk), t.kv(dv),
                    B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, nullptr, FA_GRAD_DKV, stream);
}

fa_status fa_bwd_dkv_block_sparse(const void* q, const void* k, const void* v,
                                  const float* lse, const float* delta, const void* dO,
                                  void* dk, void* dv,
                                  int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                  int causal, const unsigned char* block_mask, void* stream) {
  const Dense t{B, Hq, Hkv, Lq, Lk, D};
  return bwd_common(t.q(q), t.kv(k), t.kv(v), lse, delta, t.q(dO), t.q(nullptr), t.kv(dk), t.kv(dv),
                    B, Hq, Hkv, Lq, Lk, D, scale, causal, FA_BF16, block_mask, FA_GRAD_DKV, stream);
}

fa_status fa_bwd_ex(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                    fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, unsigned grads, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype,
                    block_mask, grads, stream);
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, int masked) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv) return 0;
  return dkv_split_plan(B, Hkv, Lq, Lk, D, masked != 0).bytes;
}

fa_status fa_bwd_ws(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                    fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, unsigned grads,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype,
                    block_mask, grads, stream, true, workspace, workspace_bytes);
}

}  // extern "C"

namespace {

// ---------------------------------------------------------------- short queries
// Work split of the short-query kernels: packed rows R = G * Lq in blocks of
// 128, keys in chunks of whole 64-key tiles.  Enough chunks that the grid is
// one round of resident workgroups on the 256 CUs of an MI355X (two per CU at
// D <= 128, one at D = 256, where a workgroup fills a CU's registers): a
// second round would repeat each workgroup's start-up and its wait for its
// first tile (measured slower at 32768 keys).  At least 256 keys per chunk so
// that a workgroup's fixed costs stay small against its loads.
struct ShortPlan {
  int R, nrb, nsplit, chunk, wsplit;
  size_t part_bytes, ml_bytes;
};

bool short_plan(int B, int Hq, int Hkv, int Lq, int Lk, int D, ShortPlan* p) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  p->R = G * Lq;
  p->nrb = (p->R + 127) / 128;
  const int64_t tiles = ((int64_t)Lk + 63) / 64;
  const int64_t groups = (int64_t)B * Hkv * p->nrb;
  // R <= 32 at D = 256: the wavefronts of a workgroup split a chunk's tiles
  // four ways, one workgroup per CU (its four K/V buffers fill the LDS), four
  // partials per chunk.  (At D = 256 the single computing wavefront of the
  // plain kernels bounds the dQ split; at D <= 128 the plain kernels, two
  // workgroups per CU with a tile in flight each, measured faster.)
  p->wsplit = p->R <= 32 && D == 256 ? 1 : 0;
  const int64_t target = p->wsplit ? 256 : (D <= 128 ? 512 : 256);  // resident workgroups
  const int64_t per_chunk = p->wsplit ? 4 : 1;  // partials per chunk
  int64_t ns = (target + groups - 1) / groups;
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, tiles / 4));
  ns = std::max<int64_t>(std::min<int64_t>(ns, 1024 / per_chunk), 1);  // the merge kernels hold <= 1024 weights
  const int64_t chunk_tiles = (tiles + ns - 1) / ns;
  p->nsplit = (int)(per_chunk * ((tiles + chunk_tiles - 1) / chunk_tiles));
  p->chunk = (int)(chunk_tiles * 64);
  const int64_t rows = (int64_t)B * Hkv * p->nsplit * p->R;
  if (groups * p->nsplit > INT32_MAX) return false;
  p->part_bytes = (size_t)rows * D * sizeof(float);
  p->ml_bytes = (size_t)rows * 2 * sizeof(float);
  return true;
}

cgqa::SplitArgs split_args(const ShortPlan& pl, void* workspace, int B, int Hq, int Hkv, int Lq, int Lk,
                           float scale) {
  cgqa::SplitArgs a{};
  a.part = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.part_bytes);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.G = Hq / Hkv; a.off = Lk - Lq;
  a.R = pl.R; a.nrb = pl.nrb; a.nsplit = pl.nsplit; a.chunk = pl.chunk; a.wsplit = pl.wsplit;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  return a;
}

fa_status check_workspace(const ShortPlan& pl, const void* workspace, size_t bytes) {
  FA_TRY(check_ptr(workspace));
  if (bytes < pl.part_bytes + pl.ml_bytes) return FA_ERR_WORKSPACE;
  return FA_OK;
}

}  // namespace

extern "C" {

static_assert(FA_SHORT_MAX_LQ == cgqa::kShortMaxLq, "short-query limit");

size_t fa_short_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D) {
  ShortPlan pl;
  if (!fwd_head_dim_ok(D) || Lq > FA_SHORT_MAX_LQ || !short_plan(B, Hq, Hkv, Lq, Lk, D, &pl)) return 0;
  return pl.part_bytes + pl.ml_bytes;
}

// The checks of fa_fwd_short, then its launch with the given workspace;
// `workspace` NULL asks for the static per-device scratch array instead.
static fa_status fwd_short_common(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                                  int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                                  fa_dtype dtype, void* workspace, size_t workspace_bytes, bool noalloc,
                                  void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (!fwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (Lq > FA_SHORT_MAX_LQ) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  if (B == 0 || Hq == 0 || Lq == 0) return FA_OK;
  for (const void* p : {(const void*)q.data, (const void*)k.data, (const void*)v.data, (const void*)o.data,
                        (const void*)lse})
    FA_TRY(check_ptr(p));
  FA_TRY(check_tensor(q, B, Hq, Lq, D, false));
  FA_TRY(check_tensor(k, B, Hkv, Lk, D, false));
  FA_TRY(check_tensor(v, B, Hkv, Lk, D, false));
  FA_TRY(check_tensor(o, B, Hq, Lq, D, true));
  ShortPlan pl;
  if (!short_plan(B, Hq, Hkv, Lq, Lk, D, &pl)) return FA_ERR_SHAPE;
  if (noalloc) {
    if (pl.part_bytes + pl.ml_bytes > cgqa::kNoAllocScratchBytes) return FA_ERR_WORKSPACE;
    if (cgqa::noalloc_scratch(&workspace) != hipSuccess) return FA_ERR_LAUNCH;
    workspace_bytes = cgqa::kNoAllocScratchBytes;
  }
  FA_TRY(check_workspace(pl, workspace, workspace_bytes));
  cgqa::SplitArgs a = split_args(pl, workspace, B, Hq, Hkv, Lq, Lk, scale);
  a.q = to_kernel(q);
  a.k = to_kernel(k);
  a.v = to_kernel(v);
  a.o = to_kernel(o);
  a.lse = lse;
  const hipError_t e = cgqa::launch_fwd_short(a, D, causal != 0, dtype == FA_F16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

fa_status fa_fwd_short(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                       int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                       fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fwd_short_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype, workspace,
                          workspace_bytes, false, stream);
}

static_assert(FA_NOALLOC_SCRATCH_BYTES == cgqa::kNoAllocScratchBytes, "static scratch size");

fa_status fa_fwd_short_noalloc(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                               int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                               fa_dtype dtype, void* stream) {
  return fwd_short_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, dtype, nullptr, 0, true,
                          stream);
}

fa_status fa_bwd_short(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                       fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                       int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                       fa_dtype dtype, unsigned grads, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!dtype_ok(dtype)) return FA_ERR_DTYPE;
  if (!bwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (Lq > FA_SHORT_MAX_LQ) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  grads &= FA_GRAD_DQ | FA_GRAD_DKV;
  if (B == 0 || Hq == 0) return FA_OK;
  if (Lq == 0) grads &= FA_GRAD_DKV;
  if (Lk == 0) grads &= FA_GRAD_DQ;
  if (grads == 0) return FA_OK;
  // every check before the first launch
  ShortPlan pl{};
  if (grads & FA_GRAD_DQ) {
    for (const void* p : {(const void*)q.data, (const void*)k.data, (const void*)v.data, (const void*)lse,
                          (const void*)delta, (const void*)dO.data, (const void*)dq.data})
      FA_TRY(check_ptr(p));
    FA_TRY(check_tensor(q, B, Hq, Lq, D, false));
    FA_TRY(check_tensor(k, B, Hkv, Lk, D, false));
    FA_TRY(check_tensor(v, B, Hkv, Lk, D, false));
    FA_TRY(check_tensor(dO, B, Hq, Lq, D, false));
    FA_TRY(check_tensor(dq, B, Hq, Lq, D, true));
    if (!short_plan(B, Hq, Hkv, Lq, Lk, D, &pl)) return FA_ERR_SHAPE;
    FA_TRY(check_workspace(pl, workspace, workspace_bytes));
  }
  // dK/dV: the key-block kernel, whose grid over keys already fills the chip
  // (its own checks run before it launches).  When every packed row sees
  // every key (one query row, or no causal mask) and the group's rows sit
  // at one stride, the G query heads of a group are handed to it as one
  // head of G * Lq rows: one pass over the group's rows instead of G
  // passes of mostly padded query tiles.  lse and delta, [B, Hq, Lq]
  // contiguous, are already laid out as [B, Hkv, G * Lq].
  if (grads & FA_GRAD_DKV) {
    const int G = Hq / Hkv;
    // a group's rows resident in one workgroup, keys streamed past them
    // (at most 64 packed rows, 32 at D = 256; row offsets within 2^30 elements)
    auto span = [&](const fa_tensor& t) {
      return (int64_t)(G - 1) * t.stride_h + (int64_t)(Lq - 1) * t.stride_l + D;
    };
    const bool stream_ok = Lq > 0 && G * Lq <= (D <= 128 ? 64 : 32) && q.stride_h >= 0 && dO.stride_h >= 0 &&
                           q.stride_l >= 0 && dO.stride_l >= 0 && span(q) < (int64_t{1} << 30) &&
                           span(dO) < (int64_t{1} << 30);
    if (stream_ok) {
      for (const void* p : {(const void*)q.data, (const void*)k.data, (const void*)v.data, (const void*)lse,
                            (const void*)delta, (const void*)dO.data, (const void*)dk.data, (const void*)dv.data})
        FA_TRY(check_ptr(p));
      FA_TRY(check_tensor(q, B, Hq, Lq, D, false));
      FA_TRY(check_tensor(k, B, Hkv, Lk, D, false));
      FA_TRY(check_tensor(v, B, Hkv, Lk, D, false));
      FA_TRY(check_tensor(dO, B, Hq, Lq, D, false));
      FA_TRY(check_tensor(dk, B, Hkv, Lk, D, true));
      FA_TRY(check_tensor(dv, B, Hkv, Lk, D, true));
      cgqa::SplitArgs s{};
      s.q = to_kernel(q);
      s.k = to_kernel(k);
      s.v = to_kernel(v);
      s.dO = to_kernel(dO);
      s.dk = to_kernel(dk);
      s.dv = to_kernel(dv);
      s.lse = const_cast<float*>(lse);
      s.delta = delta;
      s.B = B; s.Hq = Hq; s.Hkv = Hkv; s.Lq = Lq; s.Lk = Lk; s.G = G; s.off = Lk - Lq;
      s.R = G * Lq;
      // chunks of whole 128-key steps, about one round of resident workgroups
      // (two per CU where the kernel fits two, else one)
      const int64_t steps = ((int64_t)Lk + 127) / 128;
      const int64_t groups = (int64_t)B * Hkv;
      const int64_t target = D <= 128 && s.R <= 32 ? 512 : 256;
      const int64_t want = std::max<int64_t>(1, std::min<int64_t>(steps, (target + groups - 1) / groups));
      const int64_t per = (steps + want - 1) / want;
      s.chunk = (int)(per * 128);
      s.nsplit = (int)((steps + per - 1) / per);
      if (groups * s.nsplit > INT32_MAX) return FA_ERR_SHAPE;
      s.scale = scale;
      s.scale_log2 = scale * 1.4426950408889634f;
      const hipError_t e = cgqa::launch_dkv_short(s, D, causal != 0, dtype == FA_F16, static_cast<hipStream_t>(stream));
      if (e != hipSuccess) return FA_ERR_LAUNCH;
    }
    auto packed_stride = [&](const fa_tensor& t) -> int64_t {
      if (Lq == 1) return t.stride_h;
      return t.stride_h == (int64_t)Lq * t.stride_l ? t.stride_l : -1;
    };
    const int64_t rq = Lq > 0 ? packed_stride(q) : -1, ro = Lq > 0 ? packed_stride(dO) : -1;
    const bool pack = G > 1 && (Lq == 1 || !causal) && rq >= 0 && ro >= 0 && rq < (int64_t{1} << 24) &&
                      ro < (int64_t{1} << 24);
    if (stream_ok) {
      // done above
    } else if (pack) {
      const fa_tensor q2{q.data, q.stride_b, q.stride_h * G, rq};
      const fa_tensor o2{dO.data, dO.stride_b, dO.stride_h * G, ro};
      FA_TRY(bwd_common(q2, k, v, lse, delta, o2, fa_tensor{}, dk, dv, B, Hkv, Hkv, G * Lq, Lk, D, scale,
                        0, dtype, nullptr, FA_GRAD_DKV, stream));
    } else {
      FA_TRY(bwd_common(q, k, v, lse, delta, dO, fa_tensor{}, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                        dtype, nullptr, FA_GRAD_DKV, stream));
    }
  }
  if (!(grads & FA_GRAD_DQ)) return FA_OK;
  cgqa::SplitArgs a = split_args(pl, workspace, B, Hq, Hkv, Lq, Lk, scale);
  a.q = to_kernel(q);
  a.k = to_kernel(k);
  a.v = to_kernel(v);
  a.dO = to_kernel(dO);
  a.dq = to_kernel(dq);
  a.lse = const_cast<float*>(lse);
  a.delta = delta;
  const hipError_t e = cgqa::launch_dq_short(a, D, causal != 0, dtype == FA_F16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"
