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
#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

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

// ---------------------------------------------------------------- forward
template <class E, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void fa_fwd_split_kernel(SplitArgs a) {
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr float kSlack = 8.f;
  constexpr int BUF = 2 * BN * P;  // [K tile | V tile], double buffered
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];

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
    bf16_t* buf = smem + (t & 1) * BUF;
    ldk.template load<BN>(buf, kp, wk.kb + t * BN, Lk, w);
    ldv.template load<BN>(buf + BN * P, vp, wk.kb + t * BN, Lk, w);
  };
  if (nt > 0) issue(0);

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

  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    if (t + 1 < nt) issue(t + 1);
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
      const float m_new = fmaxf(m_run, m_cand);
      const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
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

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }

  // ---- partials of this chunk: (m, l) and the unnormalised accumulator
  const float l_tot = l_run + xor32(l_run);
  if (wk.row_ok) {
    const int64_t idx = ((int64_t)wk.bh * a.nsplit + wk.s) * a.R + wk.r;
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

// One wavefront per packed row: merge the chunks' (m, l, acc) into O and LSE.
template <class E, int D>
__global__ __launch_bounds__(256) void fa_fwd_combine_kernel(SplitArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Hkv + hk) * R + r
  if (row >= (int64_t)a.B * a.Hkv * a.R) return;                     // whole wavefronts leave
  const int bh = (int)(row / a.R), r = (int)(row - (int64_t)bh * a.R);
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int hi = r / a.Lq, qi = r - hi * a.Lq, hq = hk * a.G + hi;
  const int ns = a.nsplit;
  const int64_t base = (int64_t)bh * ns * a.R + r;  // chunk c: base + c * R

  float M = -INFINITY;
  for (int c = lane; c < ns; c += 64) M = fmaxf(M, a.part_ml[2 * (base + (int64_t)c * a.R)]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
  float L = 0.f;
  for (int c = lane; c < ns; c += 64) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * (base + (int64_t)c * a.R));
    if (ml.y > 0.f) L += ml.y * fast_exp2(ml.x - M);
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) L += __shfl_xor(L, m, 64);

  const float inv = L > 0.f ? 1.f / L : 0.f;  // no visible key at all: O = 0, LSE = -inf
  bf16_t* op = a.o.head(b, hq) + (int64_t)qi * a.o.sl;
  constexpr int PER = (D + 63) / 64;
  float o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int c = 0; c < ns; ++c) {
    const int64_t idx = base + (int64_t)c * a.R;
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + 2 * idx);
    if (!(ml.y > 0.f)) continue;  // a chunk this row saw nothing of
    const float wgt = fast_exp2(ml.x - M);
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (lane + 64 * e < D) o[e] = fmaf(a.part[idx * D + lane + 64 * e], wgt, o[e]);
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (lane + 64 * e < D) {
      const uint2 u = E::pack4(o[e] * inv, 0.f, 0.f, 0.f);
      op[lane + 64 * e] = (bf16_t)(u.x & 0xFFFFu);
    }
  if (lane == 0)
    a.lse[((int64_t)b * a.Hq + hq) * a.Lq + qi] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------- dQ
template <class E, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void fa_dq_split_kernel(SplitArgs a) {
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16, NDB = D / 32, NNB = BN / 32, NKS = BN / 16;
  constexpr int BUF = 2 * BN * P;
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];

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
    bf16_t* buf = smem + (t & 1) * BUF;
    ldk.template load<BN>(buf, kp, wk.kb + t * BN, Lk, w);
    ldv.template load<BN>(buf + BN * P, vp, wk.kb + t * BN, Lk, w);
  };
  if (nt > 0) issue(0);

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

  wait_vmem();
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    if (t + 1 < nt) issue(t + 1);
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

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }

  if (wk.row_ok) {
    const int64_t idx = ((int64_t)wk.bh * a.nsplit + wk.s) * a.R + wk.r;
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

// One wavefront per packed row: dQ = scale * sum over chunks.
template <class E, int D>
__global__ __launch_bounds__(256) void fa_dq_reduce_kernel(SplitArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)a.B * a.Hkv * a.R) return;
  const int bh = (int)(row / a.R), r = (int)(row - (int64_t)bh * a.R);
  const int b = bh / a.Hkv, hk = bh - b * a.Hkv;
  const int hi = r / a.Lq, qi = r - hi * a.Lq, hq = hk * a.G + hi;
  const int64_t base = (int64_t)bh * a.nsplit * a.R + r;
  constexpr int PER = (D + 63) / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c = 0; c < a.nsplit; ++c) {
    const float* pd = a.part + (base + (int64_t)c * a.R) * D;
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (lane + 64 * e < D) acc[e] += pd[lane + 64 * e];
  }
  bf16_t* out = a.dq.head(b, hq) + (int64_t)qi * a.dq.sl;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (lane + 64 * e < D) {
      const uint2 u = E::pack4(acc[e] * a.scale, 0.f, 0.f, 0.f);
      out[lane + 64 * e] = (bf16_t)(u.x & 0xFFFFu);
    }
}

// ---------------------------------------------------------------- launchers
template <class E, int D, int BN>
static hipError_t launch_fwd_short_d(const SplitArgs& a, bool causal, hipStream_t stream) {
  const int nwg = a.B * a.Hkv * a.nsplit * a.nrb;
  if (causal)
    hipLaunchKernelGGL((fa_fwd_split_kernel<E, D, BN, true>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_split_kernel<E, D, BN, false>), dim3(nwg), dim3(256), 0, stream, a);
  const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
  hipLaunchKernelGGL((fa_fwd_combine_kernel<E, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class E, int D, int BN>
static hipError_t launch_dq_short_d(const SplitArgs& a, bool causal, hipStream_t stream) {
  const int nwg = a.B * a.Hkv * a.nsplit * a.nrb;
  if (causal)
    hipLaunchKernelGGL((fa_dq_split_kernel<E, D, BN, true>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_dq_split_kernel<E, D, BN, false>), dim3(nwg), dim3(256), 0, stream, a);
  const int64_t rows = (int64_t)a.B * a.Hkv * a.R;
  hipLaunchKernelGGL((fa_dq_reduce_kernel<E, D>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
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

hipError_t launch_fwd_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? fwd_short_e<FP16>(a, D, causal, stream) : fwd_short_e<BF16>(a, D, causal, stream);
}

hipError_t launch_dq_short(const SplitArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? dq_short_e<FP16>(a, D, causal, stream) : dq_short_e<BF16>(a, D, causal, stream);
}

}  // namespace cgqa
