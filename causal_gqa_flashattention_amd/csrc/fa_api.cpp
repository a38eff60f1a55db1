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
  }
  return "unknown status";
}

const char* fa_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"

namespace {

fa_status fwd_common(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, const unsigned char* block_mask, void* stream) {
  if (!fwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (block_mask && (Lq > FA_MASK_MAX_LEN || Lk > FA_MASK_MAX_LEN)) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  if (B == 0 || Hq == 0 || Lq == 0) return FA_OK;
  for (const void* p : {q, k, v, (const void*)o, (const void*)lse}) FA_TRY(check_ptr(p));

  cgqa::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.G = Hq / Hkv;
  a.off = Lk - Lq;
  a.nqt = 0;  // set by the launcher from the kernel's tile height
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = reinterpret_cast<const uint8_t*>(block_mask);
  a.nkb = (Lk + cgqa::kMaskBlock - 1) / cgqa::kMaskBlock;
  const hipError_t e = cgqa::launch_fwd(a, D, causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, nullptr, stream);
}

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream) {
  return fwd_common(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, causal, block_mask, stream);
}

fa_status fa_bwd_delta(const void* o, const void* dO, float* delta,
                       int B, int H, int Lq, int D, void* stream) {
  if (!fwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || Lq < 0) return FA_ERR_SHAPE;
  const int64_t n = elems(B, H, Lq, D);
  if (n < 0) return FA_ERR_SHAPE;
  if (n == 0) return FA_OK;
  for (const void* p : {o, dO, (const void*)delta}) FA_TRY(check_ptr(p));
  cgqa::DeltaArgs a;
  a.o = static_cast<const uint16_t*>(o);
  a.dO = static_cast<const uint16_t*>(dO);
  a.delta = delta;
  a.rows = (int64_t)B * H * Lq;
  if (a.rows / 8 > INT32_MAX) return FA_ERR_SHAPE;
  const hipError_t e = cgqa::launch_delta(a, D, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Shared body of fa_bwd / fa_bwd_dq / fa_bwd_dkv.  which: 1 = dQ, 2 = dK/dV.
fa_status bwd_common(const void* q, const void* k, const void* v, const float* lse,
                     const float* delta, const void* dO, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                     const unsigned char* block_mask, int which, void* stream) {
  if (!bwd_head_dim_ok(D)) return FA_ERR_HEAD_DIM;
  FA_TRY(check_sizes(B, Hq, Hkv, Lq, Lk, D, causal != 0));
  if (block_mask && (Lq > FA_MASK_MAX_LEN || Lk > FA_MASK_MAX_LEN)) return FA_ERR_SHAPE;
  FA_TRY(check_scale(scale));
  if (B == 0 || Hq == 0) return FA_OK;
  // dk/dv are written whenever keys exist (zeros when there is no query row);
  // dq only when there are query rows.
  if (Lq == 0) which &= 2;
  if (Lk == 0) which &= 1;
  if (which == 0) return FA_OK;
  FA_TRY(check_ptr(k));
  FA_TRY(check_ptr(v));
  if (Lq > 0)
    for (const void* p : {q, (const void*)lse, (const void*)delta, dO}) FA_TRY(check_ptr(p));
  if (which & 1) FA_TRY(check_ptr(dq));
  if (which & 2) {
    FA_TRY(check_ptr(dk));
    FA_TRY(check_ptr(dv));
  }

  cgqa::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.lse = lse;
  a.delta = delta;
  a.dO = static_cast<const uint16_t*>(dO);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lq = Lq; a.Lk = Lk; a.G = Hq / Hkv;
  a.off = Lk - Lq;
  a.nqt = (Lq + kDqBM - 1) / kDqBM;
  a.nkt = 0;  // set by the launcher from the dK/dV kernel's key tile
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.mask = reinterpret_cast<const uint8_t*>(block_mask);
  a.nkb = (Lk + cgqa::kMaskBlock - 1) / cgqa::kMaskBlock;
  const hipError_t e = cgqa::launch_bwd(a, D, causal != 0, which, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const float* delta, const void* dO,
                 void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream) {
  (void)o;  // O enters the backward only through delta
  return bwd_common(q, k, v, lse, delta, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                    nullptr, 3, stream);
}

fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const float* delta, const void* dO,
                              void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream) {
  (void)o;
  return bwd_common(q, k, v, lse, delta, dO, dq, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale, causal,
                    block_mask, 3, stream);
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dO, void* dq,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                    int causal, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, dq, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, D, scale,
                    causal, nullptr, 1, stream);
}

fa_status fa_bwd_dq_block_sparse(const void* q, const void* k, const void* v,
                                 const float* lse, const float* delta, const void* dO, void* dq,
                                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                 int causal, const unsigned char* block_mask, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, dq, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, D, scale,
                    causal, block_mask, 1, stream);
}

fa_status fa_bwd_dkv(const void* q, const void* k, const void* v,
                     const float* lse, const float* delta, const void* dO,
                     void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, nullptr, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale,
                    causal, nullptr, 2, stream);
}

fa_status fa_bwd_dkv_block_sparse(const void* q, const void* k, const void* v,
                                  const float* lse, const float* delta, const void* dO,
                                  void* dk, void* dv,
                                  int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                  int causal, const unsigned char* block_mask, void* stream) {
  return bwd_common(q, k, v, lse, delta, dO, nullptr, dk, dv, B, Hq, Hkv, Lq, Lk, D, scale,
                    causal, block_mask, 2, stream);
}

}  // extern "C"
