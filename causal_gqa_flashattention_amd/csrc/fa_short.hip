// Short-query path for gfx950 (Lq <= 8, decode-style shapes).
//
// Page "feat(attention): complete Flash Attention VJP implementation"
// dispatches query lengths of at most 8 to separate vector kernels with fp32
// accumulators (Copilot overview and file summary).  The quantities are the
// same as for long queries (forward and dQ of the same page's Background, in
// the exp2 domain of its "Reference implementation"); what changes is the
// shape: a handful of query rows against many keys.  One query head's rows
// give a workgroup almost nothing to do, and the query heads of a group would
// each stream the same K and V.  So here:
//   * packed rows: the G * Lq (query head, query) pairs of one key/value head
//     are the rows of one workgroup, r = (h_q - G h_kv) * Lq + i, and read K
//     and V once for the whole group;
//   * split keys: each workgroup takes one chunk of keys and writes partial
//     results (fp32) to a caller workspace; a second kernel combines them.
//     Forward partials are (m, l, acc) with sum_j 2^s_j = 2^m l and
//     sum_j 2^s_j v_j = 2^m acc, combined as O = sum_c 2^(m_c - M) acc_c /
//     sum_c 2^(m_c - M) l_c and LSE = (M + log2 sum_c 2^(m_c - M) l_c) ln 2
//     with M = max_c m_c; dQ partials are plain sums over the chunk's keys.
// The per-tile products are those of the long-query kernels (transposed
// S^T = K Q^T with one packed row per lane pair, O^T += V^T P^T or
// dQ^T += K^T dS^T), on the same swizzled double-buffered tiles.
#include <mutex>

#include "fa_device.h"
#include "fa_kernels.h"

// Split partials of fa_fwd_short_noalloc: one array per GPU, for callers that
// cannot allocate.  In host code `scratch` names a host-side stand-in, never
// the device memory: kernels and copies take the address obtained below.
static __device__ __align__(256) unsigned char scratch[cgqa::kNoAllocScratchBytes];

namespace cgqa {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Each GPU holds its own copy of the array at its own address: look it up
// once per device, with that device current, and keep it.
hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

// Which chunk and packed rows a workgroup has, and what a lane's row is.
struct SplitWork {
  int b, hk, bh, s, rb;  // batch, key/value head, b * Hkv + hk, key chunk, row block
  int kb, ke;            // the chunk's keys [kb, ke)
  int r, hq, qi;         // this lane's packed row, its query head and query index
  bool row_ok;           // r < R
  __device__ SplitWork(const SplitArgs& a, int w, int lr) {
    const int id = blockIdx.x;
    rb = id % a.nrb;
    const int t = id / a.nrb;
    s = t % a.nsplit;
    bh = t / a.nsplit;
    b = bh / a.Hkv;
    hk = bh - b * a.Hkv;
    kb = s * a.chunk;
    ke = min(a.Lk, kb + a.chunk);
    r = rb * 128 + 32 * w + lr;
    row_ok = r < a.R;
    const int rr = min(r, a.R - 1);  // rows past R compute on a copy; never stored
    const int hi = rr / a.Lq;
    qi = rr - hi * a.Lq;
    hq = hk * a.G + hi;
  }
};

}  // namespace

// Both split kernels stream their chunk through NBUF tile buffers, loading
// NBUF - 1 tiles ahead: with one tile in flight a workgroup would wait out
// the memory latency on every tile, and these kernels are bound by HBM.
// Each wavefront issues ROUNDS loads per operand and tile, so after tile t
// it waits until at most (NBUF - 2) tiles' loads are outstanding.
template <int D, int BN, int NBUF>
struct SplitPipe {
  static constexpr int P = Tile<D>::P;
  static constexpr int BUF = 2 * BN * P;  // [K tile | V tile]
  static constexpr int ROUNDS = BN * Tile<D>::PC / 256;
  static constexpr int AHEAD = NBUF - 1;
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  static_assert(NBUF == 2 || NBUF == 4, "the readers step through 2 or 4 buffers by XOR");
  // XOR moving the readers from buffer t % NBUF to (t + 1) % NBUF
  __device__ static constexpr int step(int t) { return (NBUF == 4 && (t & 1)) ? 3 * BUF : BUF; }
  // the wait after tile t: tiles t + 2 .. t + AHEAD may still be in flight
  template <int OPS>
  __device__ static void wait(int t, int nt) {
    if constexpr (NBUF == 4) {
      const int pend = min(AHEAD - 1, nt - 2 - t);  // tiles issued beyond t + 1
      if (pend >= 2)
        wait_vmem_n<2 * OPS * ROUNDS>();
      else if (pend == 1)
        wait_vmem_n<OPS * ROUNDS>();
      else
        wait_vmem();
    } else {
      wait_vmem();
    }
  }
};

// ---------------------------------------------------------------- forward
template <class E, int D, int BN, bool CAUSAL, int NBUF>
__global__ __launch_bounds__(256, (D <= 128 && NBUF == 2 ? 2 : 1)) void fa_fwd_split_kernel(SplitArgs a) {
  using Pipe = SplitPipe<D, BN, NBUF>;
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr float kSlack = 8.f;
  constexpr int BUF = Pipe::BUF;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NBUF * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SplitWork wk(a, w, lr);
  const int Lk = a.Lk, off = a.off;

  const bf16_t* kp = a.k.head(wk.b, wk.hk);
  const bf16_t* vp = a.v.head(wk.b, wk.hk);
  const int nt = (wk.ke - wk.kb + BN - 1) / BN;
  // keys below full_end are visible to every row (query 0 sees keys <= off)
  const int full_end = CAUSAL ? min(Lk, off + 1) : Lk;
  const int n_full = max(0, min(nt, (full_end - wk.kb) / BN));

  const TileLoader<D> ldk(w, lane, a.k.sl), ldv(w, lane, a.v.sl);
  auto issue = [&](int t) {
    bf16_t* buf = smem + (t % NBUF) * BUF;
    ldk.template load<BN>(buf, kp, wk.kb + t * BN, Lk, w);
    ldv.template load<BN>(buf + BN * P, vp, wk.kb + t * BN, Lk, w);
  };
#pragma unroll
  for (int t = 0; t < Pipe::AHEAD; ++t)
    if (t < nt) issue(t);

  bf16x8 qf[NKD];
  {
    const bf16_t* qp = a.q.head(wk.b, wk.hq) + (int64_t)wk.qi * a.q.sl;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + 16 * kd + 8 * lg));
  }
  const int last = CAUSAL ? min(wk.qi + off, Lk - 1) : Lk - 1;  // this row's last visible key

  // a wavefront whose 32 rows are all past R only helps with the loads
  const bool w_rows = wk.rb * 128 + 32 * w < a.R;

  TileReader<D> rd(lane);
  const float c2 = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  Pipe::template wait<2>(-1, nt);  // tile 0 landed
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    if (t + Pipe::AHEAD < nt) issue(t + Pipe::AHEAD);
    const bf16_t* Ks = smem;
    const bf16_t* Vs = smem + BN * P;
    if (w_rows) {
    f32x16 s[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) s[nb] = E::mma(rd.row16(Ks, nb * 32, kd), qf[kd], s[nb]);
    }
    read_ahead<NNB * NKD, 1>();
    if (t >= n_full) {  // keys past this row's diagonal or past Lk
      __asm__ volatile("");
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (wk.kb + t * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = (crow(i, 0) <= thr) ? s[nb][i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_cand = mx * c2;
    if (__any(m_cand > m_run + kSlack)) {
      __asm__ volatile("");  // a real branch: the rescale is rare, not done on every tile
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (D > 128)
          scale_agpr(acc[db], alpha);
        else
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[nb][i], c2, -m_use));
        s[nb][i] = p;
        rs += p;
      }
    l_run += rs;
    bf16x8 pf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = E::pack8(s[ks / 2], ks % 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[db] = E::mma(rd.trA(Vs, 16 * ks, db), pf[ks], acc[db]);
    }

    rd.flip(Pipe::step(t));
    Pipe::template wait<2>(t, nt);
    __syncthreads();
  }

  // ---- partials of this chunk: (m, l) and the unnormalised accumulator
  const float l_tot = l_run + xor32(l_run);
  if (wk.row_ok) {
    const int64_t idx = ((int64_t)wk.bh * a.R + wk.r) * a.nsplit + wk.s;  // a row's chunks adjacent
    float* pa = a.part + idx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = acc[db];
        *reinterpret_cast<float4*>(pa + 32 * db + 8 * q4 + 4 * lg) =
            make_float4(c[4 * q4], c[4 * q4 + 1], c[4 * q4 + 2], c[4 * q4 + 3]);
      }
    if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * idx) = make_float2(m_run, l_tot);
  }
}

// ---------------------------------------------------------------- forward, R <= 32
// When all packed rows fit one wavefront (R <= 32) the kernel above computes
// on one wavefront of four, and at D = 256 a workgroup fills a CU.  Here (the
// host picks it for D = 256) the four wavefronts of a workgroup split
// the chunk's key tiles instead (wavefront w takes tiles w, w + 4, ...), each
// with the same rows, its own K and V buffers in LDS and no barrier, and each
// writes its own partial (a.nsplit = 4 x chunks; partial 4 c + w of chunk c).
// A wavefront's K tile is reloaded as soon as its score products have read
// it, and its V tile after the value products, so the next tile's loads
// overlap the rest of this one.
template <class E, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd_split4_kernel(SplitArgs a) {
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr float kSlack = 8.f;
  constexpr int BUF = 2 * BN * P;  // [K tile | V tile] per wavefront
  using WL = WaveTileLoader<D, BN>;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = a.nsplit / 4;
  const int s = blockIdx.x % nch, bh = blockIdx.x / nch;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int r = lr;  // packed row (R <= 32)
  const bool row_ok = r < a.R;
  const int rr = min(r, a.R - 1), hi = rr / a.Lq, qi = rr - hi * a.Lq, hq = hk * a.G + hi;
  const int Lk = a.Lk, off = a.off;
  const int kb = s * a.chunk, ke = min(Lk, kb + a.chunk);

  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  const int nt = (ke - kb + BN - 1) / BN;
  const int ntw = nt > w ? (nt - w + 3) / 4 : 0;  // this wavefront's tiles
  const int full_end = CAUSAL ? min(Lk, off + 1) : Lk;
  const int n_full = max(0, min(nt, (full_end - kb) / BN));

  bf16_t* const tk = smem + w * BUF;
  bf16_t* const tv = tk + BN * P;
  const WL ldk(lane, a.k.sl), ldv(lane, a.v.sl);
  if (ntw > 0) {
    ldk.load(tk, kp, kb + w * BN, Lk);
    ldv.load(tv, vp, kb + w * BN, Lk);
  }
  bf16x8 qf[NKD];
  {
    const bf16_t* qp = a.q.head(b, hq) + (int64_t)qi * a.q.sl;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + 16 * kd + 8 * lg));
  }
  const int last = CAUSAL ? min(qi + off, Lk - 1) : Lk - 1;

  TileReader<D> rd(lane);
  const float c2 = a.scale_log2;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  wait_vmem();  // first tile and the Q rows
  for (int i = 0; i < ntw; ++i) {
    const int t = w + 4 * i;
    const bool more = i + 1 < ntw;
    f32x16 sc[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      sc[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) sc[nb] = E::mma(rd.row16(tk, nb * 32, kd), qf[kd], sc[nb]);
    }
    read_ahead<NNB * NKD, 1>();
    if (more) {  // K tile read: load the next one
      wait_lds();
      ldk.load(tk, kp, kb + (t + 4) * BN, Lk);
    }
    if (t >= n_full) {  // keys past this row's diagonal or past Lk
      __asm__ volatile("");
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (kb + t * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[nb][j] = (crow(j, 0) <= thr) ? sc[nb][j] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[nb][j]);
    mx = fmaxf(mx, xor32(mx));
    const float m_cand = mx * c2;
    if (__any(m_cand > m_run + kSlack)) {
      __asm__ volatile("");  // a real branch: the rescale is rare, not done on every tile
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        if constexpr (D > 128)
          scale_agpr(acc[db], alpha);
        else
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[db][j] *= alpha;
      }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
    float rsum = 0.f;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = fast_exp2(fmaf(sc[nb][j], c2, -m_use));
        sc[nb][j] = p;
        rsum += p;
      }
    l_run += rsum;
    bf16x8 pf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = E::pack8(sc[ks / 2], ks % 2);
    // V tile of t: it was issued before the next K tile, so at most that
    // one's loads may still be in flight
    if (more)
      wait_vmem_n<WL::NBLK>();
    else
      wait_vmem();
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[db] = E::mma(rd.trA(tv, 16 * ks, db), pf[ks], acc[db]);
    read_ahead<NKS * NDB, 2>();
    if (more) {  // V tile read: load the next one, then wait for the next K tile
      wait_lds();
      ldv.load(tv, vp, kb + (t + 4) * BN, Lk);
      wait_vmem_n<WL::NBLK>();
    }
  }

  // ---- this wavefront's partial: (m, l) and the unnormalised accumulator
  // (a wavefront without tiles writes l = 0, which the merge skips)
  const float l_tot = l_run + xor32(l_run);
  if (row_ok) {
    const int64_t idx = ((int64_t)bh * a.R + r) * a.nsplit + 4 * s + w;
    float* pa = a.part + idx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = acc[db];
        *reinterpret_cast<float4*>(pa + 32 * db + 8 * q4 + 4 * lg) =
            make_float4(c[4 * q4], c[4 * q4 + 1], c[4 * q4 + 2], c[4 * q4 + 3]);
      }
    if (lg == 0) *reinterpret_cast<float2*>(a.part_ml + 2 * idx) = make_float2(m_run, l_tot);
  }
}

// Merge of one packed row's chunk partials, one workgroup per row.  A row's
// nsplit partials are adjacent in the workspace, so the workgroup streams
// one contiguous block: thread t takes float4 column t % (D/4) of chunks
// t / (D/4), + G, + 2G, ... (G = 256 / (D/4) groups), and the groups' sums
// are added through LDS.  `wts` holds the chunks' weights 2^(m_c - M).
template <int D, bool WEIGHTED>
__device__ __forceinline__ void merge_row(const float* part, const float* wts, int ns, float* out,
                                          float4* red) {
  constexpr int NF4 = D / 4;
  constexpr int G = 256 / NF4;
  const int t = threadIdx.x;
  const int d4 = t % NF4, g = t / NF4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g < G) {
    const float4* p4 = reinterpret_cast<const float4*>(part);
    int c = g;
    for (; c + 3 * G < ns; c += 4 * G) {  // four independent loads in flight per thread
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = p4[(int64_t)(c + u * G) * NF4 + d4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = WEIGHTED ? wts[c + u * G] : 1.f;
        acc.x = fmaf(x[u].x, wgt, acc.x);
        acc.y = fmaf(x[u].y, wgt, acc.y);
        acc.z = fmaf(x[u].z, wgt, acc.z);
        acc.w = fmaf(x[u].w, wgt, acc.w);
      }
    }
    for (; c < ns; c += G) {
      const float4 x = p4[(int64_t)c * NF4 + d4];
      const float wgt = WEIGHTED ? wts[c] : 1.f;
      acc.x = fmaf(x.x, wgt, acc.x);
      acc.y = fmaf(x.y, wgt, acc.y);
      acc.z = fmaf(x.z, wgt, acc.z);
      acc.w = fmaf(x.w, wgt, acc.w);
    }
    red[g * NF4 + d4] = acc;
  }
  __syncthreads();
  if (t < NF4) {
    float4 sum = red[t];
    for (int k = 1; k < G; ++k) {
      const float4 x = red[k * NF4 + t];
      sum.x += x.x;
      sum.y += x.y;
      sum.z += x.z;
      sum.w += x.w;
    }
    reinterpret_cast<float4*>(out)[t] = sum;
  }
  __syncthreads();
}

// Block-wide max or sum of one float per thread (256 threads).
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* scratch) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float y = __shfl_xor(x, m, 64);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[w] = x;
  __syncthreads();
  x = scratch[0];
#pragma unroll
  for (int k = 1; k < 4; ++k) x = MAX ? fmaxf(x, scratch[k]) : x + scratch[k];
  return x;
}

constexpr int kMaxSplit = 1024;  // chunks per row (the host plans at most this many)

// Forward merge: O = sum_c 2^(m_c - M) acc_c / L, L = sum_c 2^(m_c - M) l_c.
template <class E, int D>
__global__ __launch_bounds__(256) void fa_fwd_combine_kernel(SplitArgs a) {
  __shared__ float wts[kMaxSplit];
  __shared__ float4 red[256];
  __shared__ float scratch[4];
  __shared__ __attribute__((aligned(16))) float orow[D];
  const int64_t row = blockIdx.x;  // (b * Hkv + hk) * R + r
  const int bh = (int)(row / a.R), r = (int)(row - (int64_t)bh * a.R);
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int hi = r / a.Lq, qi = r - hi * a.Lq, hq = hk * a.G + hi;
  const int ns = a.nsplit;
  const int64_t base = row * ns;

  float m = -INFINITY;
  for (int c = threadIdx.x; c < ns; c += 256) m = fmaxf(m, a.part_ml[2 * (base + c)]);
  const float M = block_reduce<true>(m, scratch);
  float l = 0.f;
  for (int c = threadIdx.x; c < ns; c += 256) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * (base + c));
    const float wgt = ml.y > 0.f ? fast_exp2(ml.x - M) : 0.f;  // a chunk this row saw nothing of: 0
    wts[c] = wgt;
    l = fmaf(ml.y, wgt, l);
  }
  const float L = block_reduce<false>(l, scratch);  // (its barriers also publish wts)
  merge_row<D, true>(a.part + base * D, wts, ns, orow, red);

  const float inv = L > 0.f ? 1.f / L : 0.f;  // no visible key at all: O = 0, LSE = -inf
  bf16_t* op = a.o.head(b, hq) + (int64_t)qi * a.o.sl;
  for (int d = 4 * threadIdx.x; d < D; d += 1024)
    *reinterpret_cast<uint2*>(op + d) =
        E::pack4(orow[d] * inv, orow[d + 1] * inv, orow[d + 2] * inv, orow[d + 3] * inv);
  if (threadIdx.x == 0)
    a.lse[((int64_t)b * a.Hq + hq) * a.Lq + qi] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- dQ
template <class E, int D, int BN, bool CAUSAL, int NBUF>
__global__ __launch_bounds__(256, (D <= 128 && NBUF == 2 ? 2 : 1)) void fa_dq_split_kernel(SplitArgs a) {
  using Pipe = SplitPipe<D, BN, NBUF>;
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr int BUF = Pipe::BUF;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[NBUF * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const SplitWork wk(a, w, lr);
  const int Lk = a.Lk, off = a.off;

  const bf16_t* kp = a.k.head(wk.b, wk.hk);
  const bf16_t* vp = a.v.head(wk.b, wk.hk);
  const int nt = (wk.ke - wk.kb + BN - 1) / BN;
  const int full_end = CAUSAL ? min(Lk, off + 1) : Lk;
  const int n_full = max(0, min(nt, (full_end - wk.kb) / BN));

  const TileLoader<D> ldk(w, lane, a.k.sl), ldv(w, lane, a.v.sl);
  auto issue = [&](int t) {
    bf16_t* buf = smem + (t % NBUF) * BUF;
    ldk.template load<BN>(buf, kp, wk.kb + t * BN, Lk, w);
    ldv.template load<BN>(buf + BN * P, vp, wk.kb + t * BN, Lk, w);
  };
#pragma unroll
  for (int t = 0; t < Pipe::AHEAD; ++t)
    if (t < nt) issue(t);

  bf16x8 qf[NKD], dof[NKD];
  {
    const bf16_t* qp = a.q.head(wk.b, wk.hq) + (int64_t)wk.qi * a.q.sl;
    const bf16_t* dp = a.dO.head(wk.b, wk.hq) + (int64_t)wk.qi * a.dO.sl;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      qf[kd] = as_bf16x8(ldg16(qp + 16 * kd + 8 * lg));
      dof[kd] = as_bf16x8(ldg16(dp + 16 * kd + 8 * lg));
    }
  }
  const int64_t srow = ((int64_t)wk.b * a.Hq + wk.hq) * a.Lq + wk.qi;
  // rows past R: lse = +inf makes every P exactly 0
  const float lse2 = wk.row_ok ? a.lse[srow] * kLog2e : INFINITY;
  const float dl = wk.row_ok ? a.delta[srow] : 0.f;
  const int last = CAUSAL ? min(wk.qi + off, Lk - 1) : Lk - 1;

  const bool w_rows = wk.rb * 128 + 32 * w < a.R;  // else this wavefront only loads

  TileReaderX<D> rd(lane);
  const float c2 = a.scale_log2;
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();

  Pipe::template wait<2>(-1, nt);
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    if (t + Pipe::AHEAD < nt) issue(t + Pipe::AHEAD);
    const bf16_t* Ks = smem;
    const bf16_t* Vs = smem + BN * P;
    if (w_rows) {
    f32x16 s[NNB], dp[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
      dp[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        s[nb] = E::mma(rd.row16(Ks, nb * 32, kd), qf[kd], s[nb]);
        dp[nb] = E::mma(rd.row16(Vs, nb * 32, kd), dof[kd], dp[nb]);
      }
    }
    read_ahead<2 * NNB * NKD, 1>();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = fast_exp2(fmaf(s[nb][i], c2, -lse2));
    if (t >= n_full) {
      __asm__ volatile("");
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (wk.kb + t * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = (crow(i, 0) <= thr) ? s[nb][i] : 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = s[nb][i] * (dp[nb][i] - dl);  // dS^T
    bf16x8 dsf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dsf[ks] = E::pack8(s[ks / 2], ks % 2);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = E::mma(rd.trA(Ks, 16 * ks, db), dsf[ks], dq[db]);
    read_ahead<NKS * NDB, 2>();
    }

    rd.flip(Pipe::step(t));
    Pipe::template wait<2>(t, nt);
    __syncthreads();
  }

  if (wk.row_ok) {
    const int64_t idx = ((int64_t)wk.bh * a.R + wk.r) * a.nsplit + wk.s;  // a row's chunks adjacent
    float* pd = a.part + idx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = dq[db];
        *reinterpret_cast<float4*>(pd + 32 * db + 8 * q4 + 4 * lg) =
            make_float4(c[4 * q4], c[4 * q4 + 1], c[4 * q4 + 2], c[4 * q4 + 3]);
      }
  }
}

// ---------------------------------------------------------------- dQ, R <= 32
// The split of fa_fwd_split4_kernel for dQ: the four wavefronts take the
// chunk's key tiles in turn, each with its own K and V buffers, and write
// their own plain partial sums.  dP (V) comes before S (K) in each tile, so
// that V is reloaded once dP has read it and K once the dQ products have.
template <class E, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_dq_split4_kernel(SplitArgs a) {
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr int BUF = 2 * BN * P;
  using WL = WaveTileLoader<D, BN>;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[4 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nch = a.nsplit / 4;
  const int s = blockIdx.x % nch, bh = blockIdx.x / nch;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int r = lr;
  const bool row_ok = r < a.R;
  const int rr = min(r, a.R - 1), hi = rr / a.Lq, qi = rr - hi * a.Lq, hq = hk * a.G + hi;
  const int Lk = a.Lk, off = a.off;
  const int kb = s * a.chunk, ke = min(Lk, kb + a.chunk);

  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  const int nt = (ke - kb + BN - 1) / BN;
  const int ntw = nt > w ? (nt - w + 3) / 4 : 0;
  const int full_end = CAUSAL ? min(Lk, off + 1) : Lk;
  const int n_full = max(0, min(nt, (full_end - kb) / BN));

  bf16_t* const tk = smem + w * BUF;
  bf16_t* const tv = tk + BN * P;
  const WL ldk(lane, a.k.sl), ldv(lane, a.v.sl);
  if (ntw > 0) {
    ldv.load(tv, vp, kb + w * BN, Lk);
    ldk.load(tk, kp, kb + w * BN, Lk);
  }
  bf16x8 qf[NKD], dof[NKD];
  {
    const bf16_t* qp = a.q.head(b, hq) + (int64_t)qi * a.q.sl;
    const bf16_t* dp = a.dO.head(b, hq) + (int64_t)qi * a.dO.sl;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      qf[kd] = as_bf16x8(ldg16(qp + 16 * kd + 8 * lg));
      dof[kd] = as_bf16x8(ldg16(dp + 16 * kd + 8 * lg));
    }
  }
  const int64_t srow = ((int64_t)b * a.Hq + hq) * a.Lq + qi;
  // rows past R: lse = +inf makes every P exactly 0
  const float lse2 = row_ok ? a.lse[srow] * kLog2e : INFINITY;
  const float dl = row_ok ? a.delta[srow] : 0.f;
  const int last = CAUSAL ? min(qi + off, Lk - 1) : Lk - 1;

  TileReaderX<D> rd(lane);
  const float c2 = a.scale_log2;
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();

  wait_vmem();
  for (int i = 0; i < ntw; ++i) {
    const int t = w + 4 * i;
    const bool more = i + 1 < ntw;
    f32x16 sc[NNB], dp[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      dp[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) dp[nb] = E::mma(rd.row16(tv, nb * 32, kd), dof[kd], dp[nb]);
    }
    read_ahead<NNB * NKD, 1>();
    // V tile read: load the next one; the K tile of t, issued before it, has
    // to be in
    if (more) {
      wait_lds();
      ldv.load(tv, vp, kb + (t + 4) * BN, Lk);
      wait_vmem_n<WL::NBLK>();
    } else {
      wait_vmem();
    }
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      sc[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) sc[nb] = E::mma(rd.row16(tk, nb * 32, kd), qf[kd], sc[nb]);
    }
    read_ahead<NNB * NKD, 1>();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[nb][j] = fast_exp2(fmaf(sc[nb][j], c2, -lse2));
    if (t >= n_full) {
      __asm__ volatile("");
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (kb + t * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[nb][j] = (crow(j, 0) <= thr) ? sc[nb][j] : 0.f;
      }
    }
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[nb][j] = sc[nb][j] * (dp[nb][j] - dl);  // dS^T
    bf16x8 dsf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dsf[ks] = E::pack8(sc[ks / 2], ks % 2);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = E::mma(rd.trA(tk, 16 * ks, db), dsf[ks], dq[db]);
    read_ahead<NKS * NDB, 2>();
    if (more) {  // K tile read: load the next one, then wait for the next V tile
      wait_lds();
      ldk.load(tk, kp, kb + (t + 4) * BN, Lk);
      wait_vmem_n<WL::NBLK>();
    }
  }

  if (row_ok) {
    const int64_t idx = ((int64_t)bh * a.R + r) * a.nsplit + 4 * s + w;
    float* pd = a.part + idx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = dq[db];
        *reinterpret_cast<float4*>(pd + 32 * db + 8 * q4 + 4 * lg) =
            make_float4(c[4 * q4], c[4 * q4 + 1], c[4 * q4 + 2], c[4 * q4 + 3]);
      }
  }
}

// dQ = scale * sum over chunks, one workgroup per packed row.
template <class E, int D>
__global__ __launch_bounds__(256) void fa_dq_reduce_kernel(SplitArgs a) {
  __shared__ float4 red[256];
  __shared__ __attribute__((aligned(16))) float orow[D];
  const int64_t row = blockIdx.x;
  const int bh = (int)(row / a.R), r = (int)(row - (int64_t)bh * a.R);
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int hi = r / a.Lq, qi = r - hi * a.Lq, hq = hk * a.G + hi;
  merge_row<D, false>(a.part + row * a.nsplit * D, nullptr, a.nsplit, orow, red);
  bf16_t* out = a.dq.head(b, hq) + (int64_t)qi * a.dq.sl;
  const float sc = a.scale;
  for (int d = 4 * threadIdx.x; d < D; d += 1024)
    *reinterpret_cast<uint2*>(out + d) =
        E::pack4(orow[d] * sc, orow[d + 1] * sc, orow[d + 2] * sc, orow[d + 3] * sc);
}

// ---------------------------------------------------------------- dK / dV
// Streaming dK/dV for short queries (R <= 64 packed rows).  Each key's
// gradient depends only on the group's R rows, so instead of a key-block
// grid that reloads those rows per block, one workgroup keeps the rows
// resident: Q and dO in LDS (gathered once from their heads), LSE and delta
// beside them.  Its four wavefronts walk their own 32-key blocks of the
// workgroup's chunk (block j of wavefront w: keys kb + 32 (w + 4 j)),
// loading the next block's K and V operand fragments straight into
// registers while the current block is computed, and store each block's
// dV and then dK when done: no barrier inside the loop, and one set of
// accumulators serves both.  Per block and 32-row block rb of the packed
// rows (lane = key, as in the long kernel):
//   S = Q K^T, dP = dO V^T                 (A = rows from LDS, B = K, V)
//   P = exp2(S c - LSE log2 e), dS = P (dP - delta)
//   dV^T = sum_rb dO^T P, dK^T = sum_rb Q^T dS   (A by transposed LDS reads)
template <class E, int D, bool CAUSAL, int NRB>
__global__ __launch_bounds__(256, (D <= 128 && NRB == 1 ? 2 : 1)) void fa_dkv_stream_kernel(SplitArgs a) {
  constexpr int BM = 32 * NRB;  // packed rows held
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * 64 * P];  // [Q rows | dO rows]
  __shared__ __attribute__((aligned(16))) float stat[2][64];          // [lse | delta][row]
  // per-wavefront staging of a finished 32-key block, rows of D + 8
  // elements (16-byte aligned, bank-shifted), so that its rows leave in
  // 16-byte pieces that fill whole rows instead of one 8-byte piece per key
  constexpr int SP = D + 8;
  __shared__ __attribute__((aligned(16))) bf16_t stage[4][32 * SP];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x % a.nsplit, bh = blockIdx.x / a.nsplit;
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off, R = a.R;
  const int kb = s * a.chunk, ke = min(Lk, kb + a.chunk);

  // ---- resident rows: packed row r is query r % Lq of query head hk G + r / Lq
  // (rows past R repeat row R - 1 and are masked)
  {
    const TileLoader<D> ld(w, lane, 0);
    auto rowoff = [&](const Tensor& t) {
      return [&t, R, Lq](int r) {
        const int rr = min(r, R - 1), hi = rr / Lq;
        return (int)(hi * t.sh + (int64_t)(rr - hi * Lq) * t.sl);
      };
    };
    ld.template gather<64>(smem, a.q.head(b, hk * a.G), rowoff(a.q), w);
    ld.template gather<64>(smem + 64 * P, a.dO.head(b, hk * a.G), rowoff(a.dO), w);
    const int64_t srow = ((int64_t)b * a.Hq + hk * a.G) * Lq;  // the group's rows are adjacent
    if (w == 0) load_row_stat(&stat[0][0], a.lse + srow, 0, R, lane);
    if (w == 1) load_row_stat(&stat[1][0], a.delta + srow, 0, R, lane);
  }

  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  auto fetch = [&](int key0, bf16x8* kf, bf16x8* vf) {
    const int key = min(key0 + lr, Lk - 1);  // keys past Lk: a copy, never stored
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      kf[kd] = as_bf16x8(ldg16(kp + (int64_t)key * a.k.sl + 16 * kd + 8 * lg));
      vf[kd] = as_bf16x8(ldg16(vp + (int64_t)key * a.v.sl + 16 * kd + 8 * lg));
    }
  };
  int key0 = kb + 32 * w;
  bf16x8 kf[NKD], vf[NKD];
  if (key0 < ke) fetch(key0, kf, vf);
  wait_vmem();
  __syncthreads();

  TileReaderX<D> rq(lane);
  const bf16_t* Qs = smem;
  const bf16_t* Ds = smem + 64 * P;
  const float c2 = a.scale_log2, sc = a.scale;

  for (; key0 < ke; key0 += 128) {
    bf16x8 kn[NKD], vn[NKD];
    const bool more = key0 + 128 < ke;
    if (more) fetch(key0 + 128, kn, vn);
    const int krow = key0 + lr;
    bf16x8 pf[NRB][2], ds[NRB][2];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int r0 = 32 * rb;
      f32x16 sv = zero16(), dp = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        sv = E::mma(rq.row16(Qs, r0, kd), kf[kd], sv);
        dp = E::mma(rq.row16(Ds, r0, kd), vf[kd], dp);
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[0][r0 + 8 * i4 + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * i4 + e] = fast_exp2(fmaf(sv[4 * i4 + e], c2, l4[e] * -kLog2e));
      }
      // rows past R, and (causal) keys past a row's diagonal: key krow is
      // visible to packed row r iff krow <= r % Lq + off
      if (r0 + 32 > R || (CAUSAL && key0 + 31 > off)) {
        __asm__ volatile("");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = r0 + crow(i, lg);
          const bool ok = r < R && (!CAUSAL || krow <= r % Lq + off);
          sv[i] = ok ? sv[i] : 0.f;
        }
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[1][r0 + 8 * i4 + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = sv[4 * i4 + e] * (dp[4 * i4 + e] - d4[e]);
      }
      pf[rb][0] = E::pack8(sv, 0);
      pf[rb][1] = E::pack8(sv, 1);
      ds[rb][0] = E::pack8(dp, 0);
      ds[rb][1] = E::pack8(dp, 1);
    }
    // dV^T, then dK^T, through one set of accumulators
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const bf16_t* src = pass == 0 ? Ds : Qs;
      f32x16 acc[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] = zero16();
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            acc[db] = E::mma(rq.trA(src, 32 * rb + 16 * h, db), pass == 0 ? pf[rb][h] : ds[rb][h], acc[db]);
      // C layout (lane = key, registers = d) into the staging rows, then
      // whole rows out: lane l takes 16-byte chunk l % CPR of row l / CPR
      const float mul = pass == 0 ? 1.f : sc;
      bf16_t* stg = stage[w];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16& c = acc[db];
          *reinterpret_cast<uint2*>(stg + lr * SP + 32 * db + 8 * q4 + 4 * lg) =
              E::pack4(c[4 * q4] * mul, c[4 * q4 + 1] * mul, c[4 * q4 + 2] * mul, c[4 * q4 + 3] * mul);
        }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's LDS writes are in order
      constexpr int CPR = D / 8, RPI = 64 / CPR;               // 16-byte chunks per row, rows per pass
      const Tensor& out = pass == 0 ? a.dv : a.dk;
      if (lane < RPI * CPR) {
        const int c8 = 8 * (lane % CPR);
#pragma unroll
        for (int r = lane / CPR; r < 32; r += RPI) {
          const int key = key0 + r;
          if (key < Lk)
            *reinterpret_cast<uint4*>(out.head(b, hk) + (int64_t)key * out.sl + c8) =
                *reinterpret_cast<const uint4*>(stg + r * SP + c8);
        }
      }
      __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next pass writes
    }
    if (more) {
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        kf[kd] = kn[kd];
        vf[kd] = vn[kd];
      }
    }
  }
}

// ---------------------------------------------------------------- launchers
#ifndef CGQA_SPLIT_NBUF
#define CGQA_SPLIT_NBUF 2
#endif
constexpr int kSplitBufs = CGQA_SPLIT_NBUF;

template <class E, int D, int BN>
static hipError_t launch_fwd_short_d(const SplitArgs& a, bool causal, hipStream_t stream) {
  if (a.wsplit) {
    const int nwg = a.B * a.Hkv * (a.nsplit / 4);
    if (causal)
      hipLaunchKernelGGL((fa_fwd_split4_kernel<E, D, BN, true>), dim3(nwg), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fa_fwd_split4_kernel<E, D, BN, false>), dim3(nwg), dim3(256), 0, stream, a);
    const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
    hipLaunchKernelGGL((fa_fwd_combine_kernel<E, D>), dim3((unsigned)rows), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int nwg = a.B * a.Hkv * a.nsplit * a.nrb;
  if (causal)
    hipLaunchKernelGGL((fa_fwd_split_kernel<E, D, BN, true, kSplitBufs>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_split_kernel<E, D, BN, false, kSplitBufs>), dim3(nwg), dim3(256), 0, stream, a);
  const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
  hipLaunchKernelGGL((fa_fwd_combine_kernel<E, D>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class E, int D, int BN>
static hipError_t launch_dq_short_d(const SplitArgs& a, bool causal, hipStream_t stream) {
  if (a.wsplit) {
    const int nwg = a.B * a.Hkv * (a.nsplit / 4);
    if (causal)
      hipLaunchKernelGGL((fa_dq_split4_kernel<E, D, BN, true>), dim3(nwg), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fa_dq_split4_kernel<E, D, BN, false>), dim3(nwg), dim3(256), 0, stream, a);
    const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
    hipLaunchKernelGGL((fa_dq_reduce_kernel<E, D>), dim3((unsigned)rows), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const int nwg = a.B * a.Hkv * a.nsplit * a.nrb;
  if (causal)
    hipLaunchKernelGGL((fa_dq_split_kernel<E, D, BN, true, kSplitBufs>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_dq_split_kernel<E, D, BN, false, kSplitBufs>), dim3(nwg), dim3(256), 0, stream, a);
  const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
  hipLaunchKernelGGL((fa_dq_reduce_kernel<E, D>), dim3((unsigned)rows), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class E>
static hipError_t fwd_short_e(const SplitArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_fwd_short_d<E, 64, 64>(a, causal, stream);
    case 96: return launch_fwd_short_d<E, 96, 64>(a, causal, stream);
    case 128: return launch_fwd_short_d<E, 128, 64>(a, causal, stream);
    case 256: return launch_fwd_short_d<E, 256, 32>(a, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class E>
static hipError_t dq_short_e(const SplitArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_dq_short_d<E, 64, 64>(a, causal, stream);
    case 96: return launch_dq_short_d<E, 96, 64>(a, causal, stream);
    case 128: return launch_dq_short_d<E, 128, 64>(a, causal, stream);
    case 256: return launch_dq_short_d<E, 256, 32>(a, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

template <class E, int D, int NRB>
static void launch_dkv_short_r(const SplitArgs& a, bool causal, hipStream_t stream) {
  const int nwg = a.B * a.Hkv * a.nsplit;
  if (causal)
    hipLaunchKernelGGL((fa_dkv_stream_kernel<E, D, true, NRB>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_dkv_stream_kernel<E, D, false, NRB>), dim3(nwg), dim3(256), 0, stream, a);
}

template <class E, int D>
static hipError_t launch_dkv_short_d(const SplitArgs& a, bool causal, hipStream_t stream) {
  if (a.R <= 32)
    launch_dkv_short_r<E, D, 1>(a, causal, stream);
  else if constexpr (D <= 128)  // 64 rows at D = 256 would not fit the registers
    launch_dkv_short_r<E, D, 2>(a, causal, stream);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <class E>
static hipError_t dkv_short_e(const SplitArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_dkv_short_d<E, 64>(a, causal, stream);
    case 96: return launch_dkv_short_d<E, 96>(a, causal, stream);
    case 128: return launch_dkv_short_d<E, 128>(a, causal, stream);
    case 256: return launch_dkv_short_d<E, 256>(a, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dkv_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? dkv_short_e<FP16>(a, D, causal, stream) : dkv_short_e<BF16>(a, D, causal, stream);
}

hipError_t launch_fwd_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? fwd_short_e<FP16>(a, D, causal, stream) : fwd_short_e<BF16>(a, D, causal, stream);
}

hipError_t launch_dq_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? dq_short_e<FP16>(a, D, causal, stream) : dq_short_e<BF16>(a, D, causal, stream);
}

}  // namespace cgqa
