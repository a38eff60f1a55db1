/*
 * fa.h — C ABI of the causal grouped-query FlashAttention library for
 * AMD Instinct MI355X (gfx950).  Built as libcgqa_fa.so.
 *
 * The three compute calls follow the statement of the problem on the pages:
 *   - forward: scores S = scale * Q K^T with a causal mask, P = softmax(S),
 *     O = P V, saving only O and one log-sum-exp per query row
 *     (page "When the Bottleneck Moved: From Fused Cross-Entropy to
 *     FlashAttention on MLX", section 3; page "feat(attention): complete
 *     Flash Attention VJP implementation", Background);
 *   - delta precompute: delta_i = sum_d dO_id * O_id in fp32, once, outside
 *     the gradient kernels (VJP page, "Reference implementation" section and
 *     Architecture / Two-Kernel Design);
 *   - backward: a dQ kernel over query blocks and a dK/dV kernel over key
 *     blocks and key/value heads (looping over the query heads of the group,
 *     then over query blocks), both recomputing P from the saved log-sum-exp,
 *     no atomics (VJP page, Architecture / Two-Kernel Design).
 *
 * Tensor layout (plain calls): contiguous [B, H, L, D], D innermost; the
 * *_ex calls below take strided views and float16 as well.
 *   q, o, dO, dq : [B, Hq,  Lq, D]   bfloat16 (passed as raw 16-bit words)
 *   k, v, dk, dv : [B, Hkv, Lk, D]   bfloat16
 *   lse, delta   : [B, Hq,  Lq]      float32
 * The value head dimension equals the query/key head dimension.
 * Query head h reads key/value head h / (Hq / Hkv) (contiguous groups).
 *
 * Causal masking is bottom-right aligned: key j is visible to query i iff
 * j <= i + (Lk - Lq) (page "Add a fused full-attention path for head_dim 256
 * on NAX devices", Design, ragged causal inputs).  With causal = 0 every key
 * is visible.  Masked keys receive exactly zero probability.
 *
 * lse is the natural-log log-sum-exp of each query row's scaled scores:
 * lse_i = log(sum_j exp(scale * q_i . k_j)) over the visible j.
 *
 * Ownership and execution: every pointer is a DEVICE pointer owned by the
 * caller; the library allocates no memory and keeps no per-call state.
 * Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 * void*; NULL means the null stream) and nothing synchronises.  Every output
 * element is written exactly once, so outputs need no initialisation.  Calls
 * are thread-safe.  Results are bitwise reproducible run to run.
 *
 * Errors: all arguments are checked on the host before anything is
 * launched; a failed check returns a non-zero fa_status and launches
 * nothing.  There is no fallback path.  A kernel launch failure returns
 * FA_ERR_LAUNCH.  Sizes:
 *   B, Hq, Hkv, Lq, Lk >= 0 and < 2^31; B*H*L*D element counts must fit
 *   in int64; Hq % Hkv == 0 (Hkv >= 1 when Hq >= 1);
 *   D in {64, 96, 128, 256} for every call;
 *   causal requires Lq <= Lk (otherwise the first rows see no key);
 *   Lk == 0 with Lq > 0 is rejected (softmax over no keys).
 * Empty problems (B == 0, Hq == 0, or Lq == 0) are valid no-ops, except that
 * fa_bwd with Lq == 0 and Lk > 0 writes zeros to dk and dv.
 * Pointers to non-empty tensors must be non-NULL and 16-byte aligned.
 */
#ifndef CGQA_FA_H
#define CGQA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,              /* a required pointer is NULL                 */
  FA_ERR_ALIGN = 2,             /* a pointer is not 16-byte aligned           */
  FA_ERR_SHAPE = 3,             /* negative size, Lk == 0 < Lq, or overflow   */
  FA_ERR_HEAD_DIM = 4,          /* D not supported by this call               */
  FA_ERR_GQA = 5,               /* Hq not a multiple of Hkv                   */
  FA_ERR_CAUSAL_LQ_GT_LK = 6,   /* causal with Lq > Lk                        */
  FA_ERR_SCALE = 7,             /* scale not finite or not positive           */
  FA_ERR_LAUNCH = 8,            /* the HIP runtime refused a kernel launch    */
  FA_ERR_STRIDE = 9,            /* bad stride, or an output overlaps itself   */
  FA_ERR_DTYPE = 10,            /* unknown element type                       */
  FA_ERR_WORKSPACE = 11         /* workspace smaller than required            */
} fa_status;

/*
 * Forward attention.  Writes o [B,Hq,Lq,D] (bf16) and lse [B,Hq,Lq] (fp32,
 * natural log).  `scale` multiplies q.k before the softmax (usually
 * 1/sqrt(D)); it must be finite and > 0.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream);

/*
 * Delta precompute for the backward: delta[b,h,i] = sum_d f32(dO[b,h,i,d]) *
 * f32(O[b,h,i,d]), accumulated in fp32.  `H` is the number of query heads.
 */
fa_status fa_bwd_delta(const void* o, const void* dO, float* delta,
                       int B, int H, int Lq, int D, void* stream);

/*
 * Backward attention.  Given q, k, v, the saved lse (from fa_fwd) and delta
 * (from fa_bwd_delta), and the output gradient dO, writes
 *   dq [B,Hq,Lq,D], dk and dv [B,Hkv,Lk,D] (bf16).
 * dk/dv of a key/value head sum the contributions of all Hq/Hkv query heads
 * of its group.  `o` is accepted for the problem's signature; the kernels
 * read O only through delta and `o` may be NULL.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const float* delta, const void* dO,
                 void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                 int causal, void* stream);

/*
 * The two halves of fa_bwd, for callers that run them on separate streams
 * (the two gradient kernels are independent: the VJP page runs them
 * concurrently, Architecture / Two-Kernel Design).  fa_bwd_dq writes dq only;
 * fa_bwd_dkv writes dk and dv only.  Arguments, checks and errors are those
 * of fa_bwd; pointers a half does not use may be NULL.
 */
fa_status fa_bwd_dq(const void* q, const void* k, const void* v,
                    const float* lse, const float* delta, const void* dO, void* dq,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                    int causal, void* stream);
fa_status fa_bwd_dkv(const void* q, const void* k, const void* v,
                     const float* lse, const float* delta, const void* dO,
                     void* dk, void* dv,
                     int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                     int causal, void* stream);

/*
 * Block-sparse variants (page "feat(attention): complete Flash Attention VJP
 * implementation", "Sparse Block Masks": an optional uint8 mask with one
 * entry per (query tile, key tile) pair; a zero entry skips the pair).
 *
 * block_mask: DEVICE pointer, owned by the caller, uint8 row-major
 *   [ceil(Lq / FA_MASK_BLOCK)][ceil(Lk / FA_MASK_BLOCK)], one mask for every
 *   batch entry and head.  Query i may attend key j iff
 *   block_mask[(i / 64) * ceil(Lk / 64) + j / 64] != 0 and (when causal)
 *   j <= i + (Lk - Lq).  Pass the same mask to the forward and backward.
 *   NULL means no mask: the call is the plain one.  The library reads the
 *   mask on the device; its contents are not checked.
 * Tiles whose entries are all zero for a workgroup are not loaded or
 * computed.  A query row that sees no key at all gets O = 0 and
 * lse = -inf from the forward, dq = 0, and no share in dk and dv.
 * Other arguments, checks and errors are those of the plain calls; dq, dk
 * and dv are written in full (zeros where nothing is seen).  With a mask,
 * Lq and Lk may not exceed FA_MASK_MAX_LEN (each workgroup keeps its list of
 * tiles in LDS): FA_ERR_SHAPE otherwise.
 */
#define FA_MASK_BLOCK 64
#define FA_MASK_MAX_LEN 262144

fa_status fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream);

fa_status fa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const float* delta, const void* dO,
                              void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                              int causal, const unsigned char* block_mask, void* stream);

fa_status fa_bwd_dq_block_sparse(const void* q, const void* k, const void* v,
                                 const float* lse, const float* delta, const void* dO, void* dq,
                                 int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                 int causal, const unsigned char* block_mask, void* stream);

fa_status fa_bwd_dkv_block_sparse(const void* q, const void* k, const void* v,
                                  const float* lse, const float* delta, const void* dO,
                                  void* dk, void* dv,
                                  int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale,
                                  int causal, const unsigned char* block_mask, void* stream);

/*
 * General calls: element type and strided operands.
 *
 * Element type (page "feat(attention): complete Flash Attention VJP
 * implementation", summary: float16 and bfloat16 are supported): one fa_dtype
 * for q, k, v, o, dO, dq, dk and dv.  FA_F16 is IEEE binary16; the products
 * then run on the half-precision matrix instructions with fp32 accumulation,
 * and P and dS are rounded to half (RNE) as operands.  lse and delta stay
 * float32.
 *
 * Strided operands (same page, summary of params.h: the backward takes
 * gradient and input strides; review-comment resolutions: strides are
 * checked at run time): an fa_tensor is a [B, H, L, D] view whose element
 * (b, h, i, d) sits at element offset b*stride_b + h*stride_h + i*stride_l + d
 * from data.  The D elements of a row are contiguous.  This covers
 * [B, L, H, D] ("sequence-major") buffers, K/V that are the first Lk rows of
 * a longer cache ([B, Hkv, capacity, D] with stride_h = capacity * D: rows at
 * and past Lk are never read), and padded rows.  Requirements, checked
 * before any launch:
 *   data 16-byte aligned (FA_ERR_ALIGN) and non-NULL when non-empty;
 *   strides of dimensions with extent > 1 are >= 0 and multiples of 8
 *   elements, stride_l < 2^24 (FA_ERR_STRIDE); a stride of an extent-1
 *   dimension is ignored;
 *   inputs may overlap one another or themselves (stride 0 broadcasts);
 *   an output (o, dq, dk, dv) must not overlap itself: in order of
 *   increasing stride each dimension's stride is at least the span of the
 *   dimensions inside it, the D elements first (FA_ERR_STRIDE).
 *   Outputs must not overlap inputs or other outputs (not checked).
 * lse and delta are contiguous [B, Hq, Lq] float32 as in the plain calls.
 * All other arguments, checks and errors are those of the plain calls, of
 * which these are the general form: fa_fwd(...) is fa_fwd_ex with dense
 * [B, H, L, D] tensors, FA_BF16 and no mask.
 */
typedef enum { FA_BF16 = 0, FA_F16 = 1 } fa_dtype;

typedef struct fa_tensor {
  void* data;        /* DEVICE pointer owned by the caller (const for inputs) */
  int64_t stride_b;  /* element strides of batch, head and row            */
  int64_t stride_h;
  int64_t stride_l;
} fa_tensor;

fa_status fa_fwd_ex(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, void* stream);

fa_status fa_bwd_delta_ex(fa_tensor o, fa_tensor dO, float* delta, int B, int H, int Lq, int D,
                          fa_dtype dtype, void* stream);

/* grads: FA_GRAD_DQ (writes dq), FA_GRAD_DKV (writes dk and dv), or both
 * (fa_bwd); the tensors of a gradient not asked for may be NULL. */
#define FA_GRAD_DQ 1u
#define FA_GRAD_DKV 2u

fa_status fa_bwd_ex(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                    fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, unsigned grads, void* stream);

/*
 * fa_bwd_ex with a workspace for the dK/dV kernel's load balance.  The
 * dK/dV kernel gives each workgroup one key tile (128 keys; 64 at D = 256)
 * and loops over the query tiles that see it (page "feat(attention):
 * complete Flash Attention VJP implementation", Architecture / Two-Kernel
 * Design).  Under a causal mask the first key tile is seen by every query
 * tile and the last by almost none; with few key/value heads (fewer than two
 * workgroups per CU) the kernel then lasts as long as its first tile, and a
 * block mask can give one key tile every query tile (a sink or global
 * column, same page, "Sparse Block Masks").  With a workspace, a key tile
 * whose list of query tiles is long is shared by several workgroups, each
 * taking a run of the list and writing fp32 partial dK and dV to the
 * workspace; a second kernel adds them up (no atomics).  Without a mask, when
 * there are fewer than two key-tile workgroups per CU, every list is split
 * the same number of ways (at most 8); under a mask a planning kernel reads
 * the mask on the device and splits only the lists longer than 1.25x the
 * mean, into chunks of about half the mean.  dk and dv equal those of
 * fa_bwd_ex up to the order of fp32 additions.
 *
 * fa_bwd_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, masked) is the workspace
 * these calls use for that shape, with (masked != 0) or without a block
 * mask; 0 means no split is planned and the workspace may be NULL.  The
 * workspace is a DEVICE buffer of at least that many bytes, 16-byte aligned,
 * whose contents on entry do not matter; it must not be shared by calls that
 * may run at the same time.  It grows linearly with Lk: about
 * B * Hkv * Lk * D * 8 bytes times the number of chunks without a mask, and
 * about B * Hkv * Lk * D * 4 bytes under one.  Other arguments, checks and
 * errors are those of fa_bwd_ex; FA_ERR_NULL / FA_ERR_ALIGN /
 * FA_ERR_WORKSPACE for the workspace when dk/dv are asked for and a split is
 * planned.
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D, int masked);

fa_status fa_bwd_ws(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                    fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                    int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                    fa_dtype dtype, const unsigned char* block_mask, unsigned grads,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Short queries (Lq <= FA_SHORT_MAX_LQ; decode-style shapes).  Page
 * "feat(attention): complete Flash Attention VJP implementation" sends query
 * lengths of at most 8 to separate vector kernels with fp32 accumulators
 * (overview and file summary).  Same results as fa_fwd_ex / fa_bwd_ex, without
 * block masks, for shapes with few query rows and many keys:
 *   - the G = Hq/Hkv query heads' rows of a key/value head are computed
 *     together, so K and V are read once per group;
 *   - the keys are split into chunks processed in parallel, whose fp32
 *     partial results go to a caller-provided DEVICE workspace of at least
 *     fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D) bytes (16-byte
 *     aligned; contents on entry do not matter and are overwritten; it must
 *     not be shared by calls that may run at the same time).
 * fa_short_workspace_bytes returns 0 for sizes the short calls refuse.
 * fa_bwd_short writes dk/dv with the key-block kernel of fa_bwd_ex (no
 * workspace needed for them) and dq from key chunks reduced in a second
 * pass.  Errors: those of the *_ex calls, FA_ERR_SHAPE for Lq >
 * FA_SHORT_MAX_LQ, FA_ERR_NULL / FA_ERR_ALIGN / FA_ERR_WORKSPACE for the
 * workspace when one is needed.  lse and delta as in the plain calls.
 */
#define FA_SHORT_MAX_LQ 8

size_t fa_short_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lk, int D);

fa_status fa_fwd_short(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                       int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                       fa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

fa_status fa_bwd_short(fa_tensor q, fa_tensor k, fa_tensor v, const float* lse, const float* delta,
                       fa_tensor dO, fa_tensor dq, fa_tensor dk, fa_tensor dv,
                       int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                       fa_dtype dtype, unsigned grads, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * fa_fwd_short without a caller workspace, for callers that cannot allocate
 * device memory or pass one: code recorded under HIP graph capture, tight
 * serving and decode loops, harnesses that forbid allocation.  The split
 * partials go to a static device array of FA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on, until the process ends; the call
 * itself allocates nothing.  Arguments, results, checks and errors are those
 * of fa_fwd_short, and FA_ERR_WORKSPACE when the shape needs more scratch
 * than FA_NOALLOC_SCRATCH_BYTES (fa_short_workspace_bytes(...) tells).
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that may run at the
 * same time on one GPU (other streams, other host threads) race and must
 * be ordered by the caller.  FA_ERR_LAUNCH if the array's device address
 * cannot be obtained.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)

fa_status fa_fwd_short_noalloc(fa_tensor q, fa_tensor k, fa_tensor v, fa_tensor o, float* lse,
                               int B, int Hq, int Hkv, int Lq, int Lk, int D, float scale, int causal,
                               fa_dtype dtype, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_str(fa_status s);

/* Library version string, e.g. "0.1.0 gfx950". */
const char* fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CGQA_FA_H */
