// Backward attention kernels for gfx950: the delta precompute, the dQ kernel
// (gridded over query blocks, looping over key blocks) and the dK/dV kernel
// (gridded over key blocks and key/value heads, looping over the query heads
// of the group and then over query blocks).  Both gradient kernels recompute
// P = exp2(S * scale * log2 e - LSE * log2 e) from the saved log-sum-exp and
// own their outputs, so nothing is accumulated with atomics.
//
// Method: page "feat(attention): complete Flash Attention VJP
// implementation", Background (the backward's products: recomputed S,
// dP = dO V^T, dS = P * (dP - delta) scaled, dQ = dS K, dK = dS^T Q,
// dV = P^T dO), "Reference implementation" (delta = rowsum(dO * O) computed
// once outside the kernels, base-2 exponentials, two kernels without
// atomics) and Architecture / Two-Kernel Design (dQ grid over query blocks
// looping over key blocks; dK/dV grid over key blocks and key/value heads,
// looping over the group, then over query blocks).  The scale of dS is
// applied once to the finished dQ and dK.
#include <climits>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

// ---------------------------------------------------------------- delta
// delta[row] = sum_d f32(O[row, d]) * f32(dO[row, d]).  HBM-bound: each
// thread reads 16 bytes of O and of dO; TPR threads share one row.  Rows are
// numbered (b * H + h) * Lq + i; delta is contiguous in that order.
template <class E, int D>
__global__ __launch_bounds__(256) void fa_delta_kernel(DeltaArgs a) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int TPR = CPR <= 8 ? 8 : (CPR <= 16 ? 16 : 32);  // power of two >= CPR
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int sub = tid % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  float acc = 0.f;
  if (row < a.rows && sub < CPR) {
    int bh, i;  // b * H + h < 2^31 (checked on the host); i < Lq
    if (a.rows <= INT_MAX) {  // 32-bit division where it suffices
      bh = (int)row / a.Lq;
      i = (int)row - bh * a.Lq;
    } else {
      bh = (int)(row / a.Lq);
      i = (int)(row - (int64_t)bh * a.Lq);
    }
    const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
    const uint4 uo = ldg16(a.o.head(b, h) + (int64_t)i * a.o.sl + sub * 8);
    const uint4 ud = ldg16(a.dO.head(b, h) + (int64_t)i * a.dO.sl + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(E::get(uo, e), E::get(ud, e), acc);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < a.rows && sub == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------- dQ
// One workgroup = 4 wavefronts = 128 query rows of one query head; each
// wavefront owns 32 rows, one row per lane pair (transposed products, as in
// the forward).  Per key tile (K, V double buffered in LDS, direct loads one
// tile ahead):
//   S^T  = K Q^T        (A = K from LDS, B = Q^T in registers)
//   dP^T = V dO^T       (A = V from LDS, B = dO^T in registers)
//   dS^T = P^T * (dP^T - delta)
//   dQ^T += K^T dS^T    (A = K^T by transposed LDS reads, B = dS^T)
template <class E, int D, int BN, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void fa_dq_kernel(BwdArgs a) {
  constexpr int BM = 128;
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NNB = BN / 32;
  constexpr int NKS = BN / 16;

  // two buffers of [K tile | V tile], BUF elements apart (a power of two)
  constexpr int BUF = 2 * BN * P;
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.G;
  const TileHead th = tile_major(blockIdx.x, a.B * a.Hq);  // query tiles x (batch, query head)
  const int t = th.t, bg = th.h / G, hi = th.h - (th.h / G) * G;
  const int qt = CAUSAL ? (a.nqt - 1 - t) : t;
  const int b = bg / a.Hkv, hk = bg - (bg / a.Hkv) * a.Hkv;
  const int hq = hk * G + hi;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int64_t qh = (int64_t)(b * a.Hq + hq) * Lq;  // LSE and delta rows
  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  const int ks = a.k.sl, vs = a.v.sl;

  const int q0 = qt * BM;
  const int qrow = q0 + 32 * w + lr;
  const bool row_ok = qrow < Lq;

  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, min(q0 + BM, Lq) + off);
  const int nkt = (kv_end + BN - 1) / BN;
  int n_full = Lk / BN;  // tiles that need no mask (keys past Lk repeat the last key)
  if (CAUSAL) n_full = min(n_full, (q0 + off + 1) / BN);
  n_full = max(0, min(n_full, nkt));

  // ---- under a block mask: the key tiles some row of this workgroup needs
  // (dynamic LDS: up to nkt entries, then the count)
  extern __shared__ int tlist[];
  int nt = nkt;
  if constexpr (MASKED) {
    const int qb0 = q0 / kMaskBlock, qb1 = (min(q0 + BM, Lq) - 1) / kMaskBlock;
    if (w == 0) {
      const int cnt = build_list(tlist, nkt, lane, [](int i) { return i; }, [&](int jj) {
        bool any = false;
        for (int qb = qb0; qb <= qb1; ++qb) any |= a.mask[qb * a.nkb + jj * BN / kMaskBlock] != 0;
        return any;
      });
      if (lane == 0) tlist[nkt] = cnt;
    }
    __syncthreads();
    nt = __builtin_amdgcn_readfirstlane(tlist[nkt]);
  }
  auto tile = [&](int ti) { return MASKED ? __builtin_amdgcn_readfirstlane(tlist[ti]) : ti; };
  const int wqb = (q0 + 32 * w) / kMaskBlock;  // mask row of this wavefront's rows
  const bool w_rows = q0 + 32 * w < Lq;

  const TileLoader<D> ldk(w, lane, ks), ldv(w, lane, vs);
  const uint32_t smem_a = lds_addr(smem);  // (byte addresses: no pointer conversion per load)
  auto issue = [&](int ti) {
    const int j = tile(ti);
    const uint32_t buf = smem_a + (uint32_t)(ti & 1) * (BUF * 2);
    ldk.template load_at<BN>(buf, kp, j * BN, Lk, w);
    ldv.template load_at<BN>(buf + BN * P * 2, vp, j * BN, Lk, w);
  };
  if (nt > 0) issue(0);

  bf16x8 qf[NKD], dof[NKD];
  {
    const int qr = min(qrow, Lq - 1);
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      qf[kd] = as_bf16x8(ldg16(a.q.head(b, hq) + (int64_t)qr * a.q.sl + 16 * kd + 8 * lg));
      dof[kd] = as_bf16x8(ldg16(a.dO.head(b, hq) + (int64_t)qr * a.dO.sl + 16 * kd + 8 * lg));
    }
  }
  // rows past Lq: lse = +inf makes every P exactly 0.  (A row that sees no
  // key under a block mask has LSE = -inf; it meets only diagonal tiles, whose
  // mask zeroes its P.)
  const float lse2 = row_ok ? a.lse[qh + qrow] * kLog2e : INFINITY;
  const float dl = row_ok ? a.delta[qh + qrow] : 0.f;

  TileReaderX<D> rd(lane);
  const float c2 = a.scale_log2;
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();

  wait_vmem();
  __syncthreads();
  for (int ti = 0; ti < nt; ++ti) {
    const int j = tile(ti);
    if (ti + 1 < nt) issue(ti + 1);
    bool skip = false;  // this wavefront's rows do not see tile j
    if constexpr (MASKED) skip = !w_rows || a.mask[wqb * a.nkb + j * BN / kMaskBlock] == 0;
    if (!skip) {
    const bf16_t* Ks = smem;  // + (ti & 1) * BUF through the reader's offsets
    const bf16_t* Vs = smem + BN * P;

    f32x16 s[NNB], dp[NNB];
    prio_hi();
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
    prio_lo();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[nb][i] = fast_exp2(fmaf(s[nb][i], c2, -lse2));
    if (j >= n_full) {  // diagonal or ragged tile
      __asm__ volatile("");
      const int last = CAUSAL ? min(qrow + off, Lk - 1) : Lk - 1;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (j * BN + nb * 32 + 4 * lg);
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
    prio_hi();
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) dq[db] = E::mma(rd.trA(Ks, 16 * ks, db), dsf[ks], dq[db]);
    read_ahead<NKS * NDB, 2>();
    prio_lo();
    }

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }

  if (row_ok) {
    bf16_t* out = a.dq.head(b, hq) + (int64_t)qrow * a.dq.sl;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = dq[db];
        *reinterpret_cast<uint2*>(out + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(c[4 * q4] * sc, c[4 * q4 + 1] * sc, c[4 * q4 + 2] * sc, c[4 * q4 + 3] * sc);
      }
  }
}

// ---------------------------------------------------------------- dK / dV split
// Query-range split (nsplit > 1, with a workspace): the workgroups that share
// a key tile are chunks 0 .. nc - 1 of its query-tile list (`len` entries),
// chunk c taking entries c, c + nc, c + 2 nc, ... and writing fp32 partials
// that fa_dkv_reduce_kernel adds up.  Strided, not consecutive, entries: the
// workgroups of one chunk index walk the query tiles in the same order, last
// first, and those running at the same time share the tiles they load in L2
// (with runs of consecutive entries they read different tiles and the
// head-dim-256 kernel became bound by HBM).
//  * Without a mask every list is split min(nsplit, len) ways and chunk c runs
//    in slot c of the tile's nsplit consecutive workgroups: workgroups are
//    dealt round-robin to the XCDs by index, so one XCD runs one chunk index
//    of many tiles in step.  (Only chunk 0 then records nc.)
//  * Under a mask most lists may be short and a few long (a sink column).
//    fa_dkv_plan_kernel has measured every list and chosen nc per tile; the
//    grid starts with one workgroup per extra chunk (c >= 1) of the long
//    lists, then one per key tile for chunk 0.
struct DkvWork {
  int bh, kt, chunk;
};

// at most this many chunks per key tile under a mask (the extra-chunk table
// keeps kt * kMaxChunks + c)
constexpr int kMaxChunks = 32;

// Which (head, key tile, chunk) this workgroup takes; false: nothing (an
// unused extra-chunk workgroup, which exits at once).
template <bool MASKED>
__device__ __forceinline__ bool dkv_work(const BwdArgs& a, DkvWork& wk) {
  const int nh = a.B * a.Hkv;
  if (a.nsplit <= 1) {
    const TileHead th = tile_major(blockIdx.x, nh);  // key tiles x heads, tile 0 (heaviest) first
    wk = {th.h, th.t, 0};
    return true;
  }
  if constexpr (!MASKED) {
    const TileHead th = tile_major(blockIdx.x, nh);
    const int kt = th.t / a.nsplit;
    wk = {th.h, kt, th.t - kt * a.nsplit};
    return true;
  } else {
    if ((int)blockIdx.x < a.nextra) {
      const TileHead th = tile_major(blockIdx.x, nh);  // extra chunks x heads
      if (th.t >= a.plan[0]) return false;
      const int e = a.plan[3 + 2 * a.nkt + th.t];
      wk = {th.h, e / kMaxChunks, e % kMaxChunks};
      return true;
    }
    const TileHead th = tile_major(blockIdx.x - a.nextra, nh);
    wk = {th.h, th.t, 0};
    return true;
  }
}

struct SplitRange {
  int lo, step, cnt;  // list entries lo, lo + step, ... (cnt of them)
  float* part;        // this chunk's partials, or null: write dK / dV directly
};

// This workgroup's share of its key tile's list of `len` entries; false when
// it has none (the caller exits before its first barrier or after one every
// wavefront passes).
template <bool MASKED, int BN, int D>
__device__ __forceinline__ bool split_range(const BwdArgs& a, const DkvWork& wk, int len, int tid, SplitRange& r) {
  r = {0, 1, len, nullptr};
  if (a.nsplit <= 1) return true;
  int nc;
  float* slot0;
  if constexpr (!MASKED) {
    nc = min(a.nsplit, len);
    if (wk.chunk == 0 && tid == 0) a.split_cnt[wk.bh * a.nkt + wk.kt] = nc;
    slot0 = a.part + ((int64_t)(wk.bh * a.nkt + wk.kt) * a.nsplit) * (2 * BN * D);
  } else {
    nc = a.plan[3 + wk.kt];
    slot0 = a.part + ((int64_t)wk.bh * a.slots + a.plan[3 + a.nkt + wk.kt]) * (2 * BN * D);
  }
  if (nc <= 1) return wk.chunk == 0;
  if (wk.chunk >= nc) return false;
  r = {wk.chunk, nc, (len - wk.chunk + nc - 1) / nc, slot0 + (int64_t)wk.chunk * (2 * BN * D)};
  return true;
}

// The partials of every split key tile added up.  kReduceSlices workgroups
// per (batch, key/value head, split tile), each over a slice of the tile's
// dK and dV elements, with the chunks' loads issued four at a time (a tile's
// partials are a few MB: one workgroup per tile was bound by load latency).
// Without a mask every tile is a candidate (tiles written directly exit);
// under one the plan lists the split tiles.  dK takes the factor ksc (the
// sign and scale the dK/dV kernel left out), dV none.
constexpr int kReduceSlices = 8;
template <class E, int D, int BN>
__global__ __launch_bounds__(256) void fa_dkv_reduce_kernel(BwdArgs a) {
  const bool planned = a.plan != nullptr;
  const int per_head = (planned ? a.jmax : a.nkt) * kReduceSlices;
  const int bh = blockIdx.x / per_head;
  const int rest = blockIdx.x - bh * per_head;
  const int ti = rest / kReduceSlices, slice = rest - ti * kReduceSlices;
  int kt, nc;
  const float* base;
  if (planned) {
    if (ti >= a.plan[2]) return;
    kt = a.plan[3 + 2 * a.nkt + a.jmax + ti];
    nc = a.plan[3 + kt];
    base = a.part + ((int64_t)bh * a.slots + a.plan[3 + a.nkt + kt]) * (2 * BN * D);
  } else {
    kt = ti;
    nc = a.split_cnt[bh * a.nkt + kt];
    base = a.part + ((int64_t)(bh * a.nkt + kt) * a.nsplit) * (2 * BN * D);
  }
  if (nc <= 1) return;
  const int b = bh / a.Hkv, hk = bh - (bh / a.Hkv) * a.Hkv;
  const int k0 = kt * BN;
  constexpr int NV = 2 * BN * D / 4;  // float4 of dK then dV
  constexpr int PER = NV / kReduceSlices;
  static_assert(NV % kReduceSlices == 0 && PER % 256 == 0, "reduction slices");
  for (int e = slice * PER + threadIdx.x; e < (slice + 1) * PER; e += 256) {
    const int which = e >= NV / 2;
    const int el = 4 * e - which * BN * D;
    const int key = el / D, d = el - key * D;
    if (k0 + key >= a.Lk) continue;
    const float* p = base + 4 * e;
    float4 acc = *reinterpret_cast<const float4*>(p);
    int c = 1;
    for (; c + 4 <= nc; c += 4) {
      float4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(p + (int64_t)(c + u) * 2 * BN * D);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc.x += x[u].x;
        acc.y += x[u].y;
        acc.z += x[u].z;
        acc.w += x[u].w;
      }
    }
    for (; c < nc; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(p + (int64_t)c * 2 * BN * D);
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const float f = which ? 1.f : a.ksc;
    const Tensor& t = which ? a.dv : a.dk;
    *reinterpret_cast<uint2*>(t.head(b, hk) + (int64_t)(k0 + key) * t.sl + d) =
        E::pack4(acc.x * f, acc.y * f, acc.z * f, acc.w * f);
  }
}

// List length of every key tile under a block mask: one wavefront per key
// tile counts the BM-row query tiles that some key of the BN-key tile sees
// (the lists the dK/dV kernel builds), 64 candidates per step.  The mask is
// the same for every head, so are the lengths.
template <int BM, int BN, bool CAUSAL>
__global__ __launch_bounds__(64) void fa_dkv_count_kernel(BwdArgs a) {
  const int kt = blockIdx.x, lane = threadIdx.x;
  const int nqt = (a.Lq + BM - 1) / BM, nqb = (a.Lq + kMaskBlock - 1) / kMaskBlock;
  const int k0 = kt * BN;
  const int qt_first = (CAUSAL ? max(0, k0 - a.off) : 0) / BM;
  const int kb0 = k0 / kMaskBlock, kb1 = (min(k0 + BN, a.Lk) - 1) / kMaskBlock;
  int cnt = 0;
  for (int q0 = qt_first; q0 < nqt; q0 += 64) {
    const int qt = q0 + lane;
    bool any = false;
    if (qt < nqt) {
      const int rb_end = min((qt + 1) * (BM / kMaskBlock), nqb);
      for (int rb = qt * (BM / kMaskBlock); rb < rb_end; ++rb)
        for (int kbk = kb0; kbk <= kb1; ++kbk) any |= a.mask[rb * a.nkb + kbk] != 0;
    }
    cnt += __popcll(__ballot(any));
  }
  if (lane == 0) a.plan[3 + 2 * a.nkt + 2 * a.jmax + kt] = cnt;
}

// The split plan under a block mask (one workgroup, after
// fa_dkv_count_kernel): lists up to 1.25x the mean length are computed whole;
// a longer one is cut into chunks of cs = max(ceil(mean / 2),
// ceil(max / kMaxChunks)) entries, cs doubled until the extra chunks fit
// jmax; tile kt gets nc chunks, its first slot, and its chunks c >= 1 a place
// in the extra-chunk table.  (Half-mean chunks keep a long list's extra work
// in pieces small enough to fill the gaps the short lists leave: with chunks
// of 1.25 means, the 8192-token shape with a 1024-key window and one sink
// block took 0.48 ms for dK/dV, with half-mean chunks 0.43 ms.)
__global__ __launch_bounds__(1024) void fa_dkv_plan_kernel(BwdArgs a) {
  __shared__ int len_s[kMaxPlanTiles];
  __shared__ int red[2][16];
  __shared__ int cs_s, thr_s;
  const int tid = threadIdx.x, nkt = a.nkt;
  const int* lens = a.plan + 3 + 2 * nkt + 2 * a.jmax;
  int sum = 0, mx = 0;
  for (int kt = tid; kt < nkt; kt += 1024) {
    const int l = lens[kt];
    len_s[kt] = l;
    sum += l;
    mx = max(mx, l);
  }
  for (int o = 32; o >= 1; o >>= 1) {
    sum += __shfl_xor(sum, o, 64);
    mx = max(mx, __shfl_xor(mx, o, 64));
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sum;
    red[1][tid >> 6] = mx;
  }
  __syncthreads();
  if (tid == 0) {
    int s = 0, m = 0;
    for (int i = 0; i < 16; ++i) {
      s += red[0][i];
      m = max(m, red[1][i]);
    }
    thr_s = (5 * s + 4 * nkt - 1) / (4 * nkt);
    cs_s = max(1, max((s + 2 * nkt - 1) / (2 * nkt), (m + kMaxChunks - 1) / kMaxChunks));
  }
  __syncthreads();
  const int thr = thr_s;
  // double cs until the extra chunks fit (every thread counts its tiles)
  for (;;) {
    const int cs = cs_s;
    int extra = 0;
    for (int kt = tid; kt < nkt; kt += 1024)
      if (len_s[kt] > thr) extra += (len_s[kt] + cs - 1) / cs - 1;
    for (int o = 32; o >= 1; o >>= 1) extra += __shfl_xor(extra, o, 64);
    __syncthreads();
    if ((tid & 63) == 0) red[0][tid >> 6] = extra;
    __syncthreads();
    int tot = 0;
    for (int i = 0; i < 16; ++i) tot += red[0][i];
    if (tot <= a.jmax) break;  // (the same decision in every thread)
    __syncthreads();
    if (tid == 0) cs_s = 2 * cs;
    __syncthreads();
  }
  if (tid == 0) {
    const int cs = cs_s;
    int* plan = a.plan;
    int slot = 0, j = 0, ns = 0;
    for (int kt = 0; kt < nkt; ++kt) {
      const int nc = len_s[kt] > thr ? max(1, (len_s[kt] + cs - 1) / cs) : 1;
      plan[3 + kt] = nc;
      plan[3 + nkt + kt] = nc > 1 ? slot : 0;
      if (nc > 1) {
        slot += nc;
        plan[3 + 2 * nkt + a.jmax + ns++] = kt;
        for (int c = 1; c < nc; ++c) plan[3 + 2 * nkt + j++] = kt * kMaxChunks + c;
      }
    }
    plan[0] = j;
    plan[1] = cs;
    plan[2] = ns;
  }
}

// ---------------------------------------------------------------- dK / dV
// One workgroup = 2 KB wavefronts = 32 KB keys of one key/value head.  The
// keys form KB 32-key blocks; wavefront w owns block w % KB for the query rows
// 32*(w / KB) .. +31 of every query tile, so two wavefronts accumulate partial
// dK/dV for the same keys over different rows and add them once at the end.
// KB = 4 (8 wavefronts, one workgroup per CU) by default; KB = 2 at head dim
// 64 without a split, where three 4-wavefront workgroups share a CU: their
// barriers are independent, so one workgroup's vector work can overlap
// another's matrix products.
// K and V sit in LDS for the whole kernel (each wave's K operand fragments
// also in registers); query tiles of Q and dO stream through LDS (double
// buffered, direct loads one tile ahead) with their LSE and delta, for every
// query head of the group in turn.
// H1 (head dims 96 and 128 without a causal mask or a split): KB = 4
// wavefronts of 32 keys each over 32-row query tiles, one row half, so that
// two 4-wavefront workgroups share a CU with independent barriers, as at
// head dim 64.  (With a causal mask the key tiles' work is unequal and two
// heavy ones would share a CU; one workgroup per CU in heaviest-first order
// balances them.)  The K tile is read into registers through the query-tile
// buffers before the first query tile arrives: the LDS of two workgroups
// holds no more.
// Per query tile and wavefront (32 rows x 32 keys):
//   S  = Q K^T          (A = Q rows from LDS, B = K rows in registers)
//   dP = dO V^T         (A = dO rows, B = V rows, from LDS)
//   dS = P * (dP - delta), formed as -dS = P * (delta - dP) (V negated)
//   dV^T += dO^T P      (A = dO^T by transposed LDS reads, B = P)
//   dK^T += Q^T dS      (A = Q^T by transposed LDS reads, B = -dS)
template <class E, int D, bool CAUSAL, bool MASKED, int KB = 4, bool H1 = false>
__global__ __launch_bounds__(H1 ? 64 * KB : 128 * KB, KB == 4 && !H1 ? 1 : 2) void fa_dkv_kernel(BwdArgs a) {
  static_assert(KB == 4 || KB == 2, "four or two key blocks");
  static_assert(!H1 || (KB == 4 && D >= 96), "one row half: 128-key workgroups");
  constexpr int NW = H1 ? KB : 2 * KB;  // wavefronts
  constexpr int BN = 32 * KB;  // keys per workgroup
  // query rows per tile: 64 (two halves of 32), or 128 at head dim 64 with
  // eight wavefronts, where a 64-row tile is too little matrix work per
  // barrier; each wave then takes two 32-row units per tile (under a block
  // mask, one per 64-row mask block)
  constexpr int BM = H1 ? 32 : D == 64 && KB == 4 ? 128 : 64;
  static_assert(BM % kMaskBlock == 0 || kMaskBlock % BM == 0, "query tiles tile the mask blocks");
  constexpr int NU = BM < 64 ? 1 : BM / 64;  // 32-row units of this wave per tile (64 rows each apart)
  constexpr int SR = BM < 64 ? 64 : BM;      // rows of a stat buffer (64-row loads)
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;

  // two buffers of [Q tile | dO tile], BUF elements apart (a power of two),
  // then the K and V tiles of this workgroup
  constexpr int BUF = 2 * BM * P;
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  static_assert(!H1 || 2 * BUF == BN * P, "H1: the K tile fills the two query-tile buffers");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF + (H1 ? 1 : 2) * BN * P];
  bf16_t* const sK = H1 ? smem : smem + 2 * BUF;
  bf16_t* const sV = smem + 2 * BUF + (H1 ? 0 : BN * P);
  __shared__ __attribute__((aligned(16))) float stat[2][2][SR];  // [buf][lse / delta][row]

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w & (KB - 1), qhalf = H1 ? 0 : w / KB;
  const int G = a.G;
  // key tiles (x chunks) x (batch, key/value head); key tile 0 sees the most
  // queries: heaviest first
  DkvWork wk;
  if (!dkv_work<MASKED>(a, wk)) return;
  const int bh = wk.bh, kt = wk.kt;
  const int b = bh / a.Hkv, hk = bh - (bh / a.Hkv) * a.Hkv;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int k0 = kt * BN;
  const int krow = k0 + 32 * kb + lr;
  const bool key_ok = krow < Lk;

  // first query row that can see key k0: i >= k0 - off
  const int qfirst = CAUSAL ? max(0, k0 - off) : 0;
  const int qt_first = qfirst / BM;
  const int nqt = (Lq + BM - 1) / BM;
  const int nq = max(0, nqt - qt_first);
  // iteration n: query tile nqt - 1 - n / G of query head n % G.  Last tile
  // first and heads innermost, so the workgroups of one key/value head on one
  // XCD read the same Q/dO tile at about the same time and share it in L2,
  // whatever their first tile.
  // ---- under a block mask: the query tiles (last first) that some key of
  // this workgroup sees (dynamic LDS: up to nq entries, then the count)
  extern __shared__ int qlist[];
  int nql = nq;
  if constexpr (MASKED) {
    const int kb0 = k0 / kMaskBlock, kb1 = (min(k0 + BN, Lk) - 1) / kMaskBlock;
    if (w == 0) {
      const int cnt = build_list(qlist, nq, lane, [&](int i) { return nqt - 1 - i; }, [&](int qtl) {
        bool any = false;
        const int rb_end = min(((qtl + 1) * BM - 1) / kMaskBlock + 1, (Lq + kMaskBlock - 1) / kMaskBlock);
        for (int rb = qtl * BM / kMaskBlock; rb < rb_end; ++rb)
          for (int kbk = kb0; kbk <= kb1; ++kbk) any |= a.mask[rb * a.nkb + kbk] != 0;
        return any;
      });
      if (lane == 0) qlist[nq] = cnt;
    }
    __syncthreads();
    nql = __builtin_amdgcn_readfirstlane(qlist[nq]);
  }
  SplitRange sr;
  if (!split_range<MASKED, BN, D>(a, wk, nql, tid, sr)) return;  // (uniform: nql is)
  const int niter = G * sr.cnt;
  const int wkb = (k0 + 32 * kb) / kMaskBlock;  // mask column of this wavefront's keys
  const bool w_keys = k0 + 32 * kb < Lk;
  const int nqb = (Lq + kMaskBlock - 1) / kMaskBlock;  // mask rows

  // eight waves load as two groups of four: waves 0-3 fill Q, waves 4-7 fill
  // dO; four waves fill both
  const int wl = w & 3;
  const TileLoader<D> ld(wl, lane, NW == 4 || w < 4 ? a.q.sl : a.dO.sl);
  const TileLoader<D> ldo(wl, lane, a.dO.sl);  // (four waves: their dO)
  constexpr int WDELTA = NW == 8 ? 4 : 1;  // the wave that loads the rows' delta
  // Q and dO are direct global->LDS loads, and so are the rows' delta
  // (wave WDELTA), rows past Lq repeating the last row.  The rows' LSE goes
  // to LDS already multiplied by -log2 e, so that a score's probability is
  // one fma and one exp2: wave 0 loads it into a register with the tile and
  // writes it scaled before the barrier that ends the iteration
  // (publish_lse), when the buffer's previous readers are done.
  // The next tile to load is kept as running state (query head nx_hi of the
  // group, list entry nx_i, the head's Q / dO / LSE / delta bases), advanced
  // by additions: no division by the group size and no 64-bit products per
  // tile, and LDS destinations as plain byte addresses.
  float lse_next[NU];
  const uint32_t smem_a = lds_addr(smem), stat_a = lds_addr(&stat[0][0][0]);
  const int64_t srow0 = (int64_t)(b * a.Hq + hk * G) * Lq;  // LSE / delta row of the group's first head
  const bf16_t* nx_q = a.q.head(b, hk * G);
  const bf16_t* nx_o = a.dO.head(b, hk * G);
  const float* nx_l = a.lse + srow0;
  const float* nx_d = a.delta + srow0;
  int nx_hi = 0, nx_i = sr.lo, q0_nx = 0;
  auto issue = [&](int n) {  // tile n (the next in order)
    const uint32_t qt_a = smem_a + (uint32_t)(n & 1) * (BUF * 2);
    const uint32_t dt_a = qt_a + BM * P * 2;
    const int qtile = MASKED ? __builtin_amdgcn_readfirstlane(qlist[nx_i]) : nqt - 1 - nx_i;
    const int qbase = qtile * BM;
    q0_nx = qbase;
    if constexpr (NW == 8) {
      if (w < 4)
        ld.template load_at<BM>(qt_a, nx_q, qbase, Lq, wl);
      else
        ld.template load_at<BM>(dt_a, nx_o, qbase, Lq, wl);
    } else {
      ld.template load_at<BM>(qt_a, nx_q, qbase, Lq, wl);
      ldo.template load_at<BM>(dt_a, nx_o, qbase, Lq, wl);
    }
    // 64 rows per load; a half past Lq repeats row Lq - 1 (with 32-row
    // tiles the second 32 rows are loaded and not read)
#pragma unroll
    for (int hr = 0; hr < NU; ++hr) {
      if (w == 0) lse_next[hr] = nx_l[min(qbase + 64 * hr + lane, Lq - 1)];
      if (w == WDELTA)
        load_row_stat_at(stat_a + (uint32_t)(((n & 1) * 2 + 1) * SR + 64 * hr) * 4u, nx_d, min(qbase + 64 * hr, Lq - 1),
                         Lq, lane);
    }
    // advance: heads innermost, then the list
    if (++nx_hi < G) {
      nx_q += a.q.sh;
      nx_o += a.dO.sh;
      nx_l += Lq;
      nx_d += Lq;
    } else {
      nx_hi = 0;
      nx_i += sr.step;
      nx_q -= (int64_t)(G - 1) * a.q.sh;
      nx_o -= (int64_t)(G - 1) * a.dO.sh;
      nx_l -= (int64_t)(G - 1) * Lq;
      nx_d -= (int64_t)(G - 1) * Lq;
    }
  };
  auto publish_lse = [&](int n) {
    if (w == 0) {
#pragma unroll
      for (int hr = 0; hr < NU; ++hr) stat[n & 1][0][64 * hr + lane] = lse_next[hr] * -kLog2e;
    }
  };
  // K and V of this key tile, once (rows past Lk repeat the last key)
  if constexpr (NW == 8) {
    const TileLoader<D> lkv(wl, lane, w < 4 ? a.k.sl : a.v.sl);
    lkv.template load<BN>(w < 4 ? sK : sV, w < 4 ? a.k.head(b, hk) : a.v.head(b, hk), k0, Lk, wl);
  } else {
    TileLoader<D>(wl, lane, a.k.sl).template load<BN>(sK, a.k.head(b, hk), k0, Lk, wl);
    TileLoader<D>(wl, lane, a.v.sl).template load<BN>(sV, a.v.head(b, hk), k0, Lk, wl);
  }
  int q0_cur = 0;
  if (!H1 && niter > 0) {
    issue(0);
    publish_lse(0);
    q0_cur = q0_nx;
  }

  TileReaderX<D> rq(lane);  // Q and dO tiles: offsets flip with the buffer
  // ... and, at head dim >= 96 without a mask, carry this wave's row half, so
  // that every read's row offset is a constant (the instruction's immediate,
  // not a vector add per address).  (Elsewhere the extra live offsets cost
  // occupancy or a spill.)
  constexpr bool FOLD_ROWS = !MASKED && D >= 96;
  if constexpr (FOLD_ROWS) rq.shift(2 * 32 * qhalf * P);
  TileReaderX<D> rk(lane);  // K and V tiles (resident)
  const float c2 = a.scale_log2;
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  wait_vmem();
  __syncthreads();
  // V with its sign bits flipped (bf16 and half alike): the dP products,
  // started from delta, then give delta - dP, and P times that is -dS in one
  // multiply; dK takes the sign back with the scale at the end
  {
    constexpr int NCH = BN * P * 2 / 16;  // 16-byte chunks of the V tile
    uint4* vv = reinterpret_cast<uint4*>(sV);
#pragma unroll
    for (int i = tid; i < NCH; i += 64 * NW) {
      uint4 x = vv[i];
      x.x ^= 0x80008000u;
      x.y ^= 0x80008000u;
      x.z ^= 0x80008000u;
      x.w ^= 0x80008000u;
      vv[i] = x;
    }
  }
  __syncthreads();
  // this wavefront's K operand fragments stay in registers (loop-invariant)
  bf16x8 kf[NKD];
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) kf[kd] = rk.row16(sK, 32 * kb, kd);
  if constexpr (H1) {
    // the K tile's LDS is the query-tile buffers: every wave has read its
    // fragments before the first query tile goes there
    __syncthreads();
    if (niter > 0) {
      issue(0);
      publish_lse(0);
      q0_cur = q0_nx;
    }
    wait_vmem();
    __syncthreads();
  }
  for (int n = 0; n < niter; ++n) {
    const int buf = n & 1;
    const int q0 = q0_cur;
    if (n + 1 < niter) issue(n + 1);
    const bf16_t* Qs = smem;            // + buf * BUF through rq's flipped offsets
    const bf16_t* Ds = smem + BM * P;
    {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
    const int r0 = 32 * qhalf + 64 * u;  // this wave's rows within the tile
    const int rr = FOLD_ROWS ? 64 * u : r0;  // the same as the reads take it
    // under a block mask, a unit whose 64-row block this wavefront's keys do
    // not see is skipped (blocks past the mask's last row are computed, to
    // zero contributions, as without a mask)
    if constexpr (MASKED) {
      const int rb = q0 / kMaskBlock + u;
      if (!w_keys || (rb < nqb && a.mask[rb * a.nkb + wkb] == 0)) continue;
    }

    // dp starts from each row's delta (C layout: register 4 i4 + e holds
    // row 8 i4 + 4 lg + e); with V negated it ends as delta - dP
    f32x16 s = zero16(), dp;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[buf][1][r0 + 8 * i4 + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = d4[e];
    }
    prio_hi();
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      s = E::mma(rq.row16(Qs, rr, kd), kf[kd], s);
      dp = E::mma(rq.row16(Ds, rr, kd), rk.row16(sV, 32 * kb, kd), dp);
    }
    // (no read-ahead pattern here: with eight wavefronts in step it only
    // bunches the LDS reads, measured slower)
    prio_lo();
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[buf][0][r0 + 8 * i4 + 4 * lg]);  // -LSE log2 e
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * i4 + e] = fast_exp2(fmaf(s[4 * i4 + e], c2, l4[e]));
    }
    // tiles that cross the diagonal or hold rows past Lq
    if ((CAUSAL && k0 + BN - 1 > q0 + off) || q0 + BM > Lq) {
      __asm__ volatile("");
      // key krow is visible to row q0 + r0 + crow(i, lg) iff crow(i, 0) >= thr,
      // and that row exists iff crow(i, 0) < rlim
      const int thr = CAUSAL ? krow - off - q0 - r0 - 4 * lg : INT_MIN;
      const int rlim = Lq - q0 - r0 - 4 * lg;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (crow(i, 0) >= thr && crow(i, 0) < rlim) ? s[i] : 0.f;
    }
    // -dS = P (delta - dP)
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = s[i] * dp[i];
    const bf16x8 pf[2] = {E::pack8(s, 0), E::pack8(s, 1)};
    const bf16x8 ds[2] = {E::pack8(dp, 0), E::pack8(dp, 1)};
    prio_hi();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dv[db] = E::mma(rq.trA(Ds, rr + 16 * h, db), pf[h], dv[db]);
        dk[db] = E::mma(rq.trA(Qs, rr + 16 * h, db), ds[h], dk[db]);
      }
    prio_lo();
    }
    }

    rq.flip(BUF);
    if (n + 1 < niter) publish_lse(n + 1);
    q0_cur = q0_nx;
    wait_vmem();
    __syncthreads();
  }

  // ---- add the two row halves: waves KB.. hand their partials to waves
  // 0..KB-1 through LDS (the tile buffers are free now), lane-contiguous per
  // register
  float* red = reinterpret_cast<float*>(smem);
  static_assert(H1 || (2 * BUF + 2 * BN * P) * 2 >= KB * NDB * 16 * 64 * 4, "reduction buffer too small");
#pragma unroll
  for (int pass = 0; pass < (H1 ? 0 : 2); ++pass) {
    f32x16* acc = pass == 0 ? dk : dv;
    if (w >= KB) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((kb * NDB + db) * 16 + i) * 64 + lane] = acc[db][i];
    }
    __syncthreads();
    if (w < KB) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] += red[((kb * NDB + db) * 16 + i) * 64 + lane];
    }
    __syncthreads();
  }

  if (sr.part != nullptr) {
    if (w < KB) {
      float* pk = sr.part + (32 * kb + lr) * D;
      float* pv = pk + BN * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16 &ck = dk[db], &cv = dv[db];
          *reinterpret_cast<float4*>(pk + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(ck[4 * q4], ck[4 * q4 + 1], ck[4 * q4 + 2], ck[4 * q4 + 3]);
          *reinterpret_cast<float4*>(pv + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(cv[4 * q4], cv[4 * q4 + 1], cv[4 * q4 + 2], cv[4 * q4 + 3]);
        }
    }
  } else if (w < KB && key_ok) {
    bf16_t* dkp = a.dk.head(b, hk) + (int64_t)krow * a.dk.sl;
    bf16_t* dvp = a.dv.head(b, hk) + (int64_t)krow * a.dv.sl;
    const float sc = -a.scale;  // the accumulators hold -dK / scale
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16 &ck = dk[db], &cv = dv[db];
        *reinterpret_cast<uint2*>(dkp + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(ck[4 * q4] * sc, ck[4 * q4 + 1] * sc, ck[4 * q4 + 2] * sc, ck[4 * q4 + 3] * sc);
        *reinterpret_cast<uint2*>(dvp + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(cv[4 * q4], cv[4 * q4 + 1], cv[4 * q4 + 2], cv[4 * q4 + 3]);
      }
  }
}

// ---------------------------------------------------------------- dK / dV, wide heads
// Head dim 256: the dK/dV accumulators of 32 keys take 256 registers per
// wavefront, so two wavefronts cannot share a SIMD.  One workgroup = 4
// wavefronts = 64 keys, one wavefront per SIMD: wavefront w owns keys
// 32 (w & 1) .. + 31 and row half w >> 1 of every query tile, keeps its K and
// V operand fragments in registers, and query tiles of 64 rows of Q and dO
// (with LSE and delta) stream through LDS, double buffered.  Per query tile
// the products are those of fa_dkv_kernel; the two row halves' dK/dV are
// added through LDS at the end.  (64-key workgroups: at 8192 tokens and two
// key/value heads that is 256 workgroups, one per CU.)
template <class E, int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, 1) void fa_dkv_reg_kernel(BwdArgs a) {
  constexpr int BN = 64;    // keys per workgroup
  constexpr int BM = 64;    // query rows per tile (two halves of 32)
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;

  constexpr int BUF = 2 * BM * P;  // [Q tile | dO tile]
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float stat[2][2][64];  // [buf][lse / delta][row]

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w & 1, qhalf = w >> 1;
  const int r0 = 32 * qhalf;  // this wavefront's rows within a tile
  const int G = a.G;
  // key tiles (x chunks) x (batch, key/value head); key tile 0 sees the most
  // queries: heaviest first
  DkvWork wk;
  if (!dkv_work<MASKED>(a, wk)) return;
  const int bh = wk.bh, kt = wk.kt;
  const int b = bh / a.Hkv, hk = bh - (bh / a.Hkv) * a.Hkv;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int k0 = kt * BN;
  const int krow = k0 + 32 * kb + lr;
  const bool key_ok = krow < Lk;

  const int qfirst = CAUSAL ? max(0, k0 - off) : 0;
  const int qt_first = qfirst / BM;
  const int nqt = (Lq + BM - 1) / BM;
  const int nq = max(0, nqt - qt_first);
  // iteration n: query tile nqt - 1 - n / G of query head n % G.  Last tile
  // first and heads innermost, so the workgroups of one key/value head on one
  // XCD read the same Q/dO tile at about the same time and share it in L2,
  // whatever their first tile.
  // ---- under a block mask: the query tiles (last first) that some key of
  // this workgroup sees (dynamic LDS: up to nq entries, then the count)
  extern __shared__ int qlist[];
  int nql = nq;
  if constexpr (MASKED) {
    const int kb0 = k0 / kMaskBlock, kb1 = (min(k0 + BN, Lk) - 1) / kMaskBlock;
    if (w == 0) {
      const int cnt = build_list(qlist, nq, lane, [&](int i) { return nqt - 1 - i; }, [&](int qtl) {
        bool any = false;
        for (int kbk = kb0; kbk <= kb1; ++kbk) any |= a.mask[qtl * a.nkb + kbk] != 0;
        return any;
      });
      if (lane == 0) qlist[nq] = cnt;
    }
    __syncthreads();
    nql = __builtin_amdgcn_readfirstlane(qlist[nq]);
  }
  SplitRange sr;
  if (!split_range<MASKED, BN, D>(a, wk, nql, tid, sr)) return;  // (uniform: nql is)
  const int niter = G * sr.cnt;
  auto qtile_of = [&](int n) {
    const int i = sr.lo + sr.step * (n / G);
    return MASKED ? __builtin_amdgcn_readfirstlane(qlist[i]) : nqt - 1 - i;
  };

  const TileLoader<D> ldq(w, lane, a.q.sl), ldo(w, lane, a.dO.sl);
  const bf16_t* const qsrc = a.q.head(b, hk * G);
  const bf16_t* const osrc = a.dO.head(b, hk * G);
  // Q, dO and the rows' delta (wave 1) by direct loads.  The rows' LSE goes
  // to LDS already multiplied by -log2 e (one fma and one exp2 per score):
  // wave 0 loads it into a register with the tile and writes it scaled before
  // the barrier that ends the iteration (publish_lse).
  float lse_next = 0.f;
  const uint32_t smem_a = lds_addr(smem);  // (byte addresses: no pointer conversion per load)
  auto issue = [&](int n) {
    const uint32_t qt_a = smem_a + (uint32_t)(n & 1) * (BUF * 2);
    const int hi = n % G, qtile = qtile_of(n);
    const int64_t qh = (int64_t)(b * a.Hq + hk * G + hi) * Lq;
    const int qbase = qtile * BM;
    if (w == 1) load_row_stat(&stat[n & 1][1][0], a.delta + qh, qbase, Lq, lane);
    ldq.template load_at<BM>(qt_a, qsrc + hi * a.q.sh, qbase, Lq, w);
    ldo.template load_at<BM>(qt_a + BM * P * 2, osrc + hi * a.dO.sh, qbase, Lq, w);
    if (w == 0) lse_next = a.lse[qh + min(qbase + lane, Lq - 1)];
  };
  auto publish_lse = [&](int n) {
    if (w == 0) stat[n & 1][0][lane] = lse_next * -kLog2e;
  };
  if (niter > 0) {
    issue(0);
    publish_lse(0);
  }

  bf16x8 kf[NKD], vf[NKD];
  {
    const int kr = min(krow, Lk - 1);  // keys past Lk: a copy, never stored
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      kf[kd] = as_bf16x8(ldg16(a.k.head(b, hk) + (int64_t)kr * a.k.sl + 16 * kd + 8 * lg));
      // V with its sign bits flipped (bf16 and half alike): the dP products,
      // started from delta, then give delta - dP, and P times that is -dS in
      // one multiply; dK takes the sign back with the scale at the end
      uint4 x = ldg16(a.v.head(b, hk) + (int64_t)kr * a.v.sl + 16 * kd + 8 * lg);
      x.x ^= 0x80008000u;
      x.y ^= 0x80008000u;
      x.z ^= 0x80008000u;
      x.w ^= 0x80008000u;
      vf[kd] = as_bf16x8(x);
    }
  }

  TileReader<D> rd(lane);
  // the reads' offsets carry this wave's row half: row offsets are immediates
  rd.shift(2 * r0 * P);
  const float c2 = a.scale_log2;
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }

  wait_vmem();
  __syncthreads();
  for (int n = 0; n < niter; ++n) {
    const int buf = n & 1;
    const int q0 = qtile_of(n) * BM;
    if (n + 1 < niter) issue(n + 1);
    const bf16_t* Qs = smem;  // + buf * BUF through the reader's flipped offsets
    const bf16_t* Ds = smem + BM * P;

    // dp starts from each row's delta (C layout: register 4 i4 + e holds
    // row 8 i4 + 4 lg + e); with V negated it ends as delta - dP
    f32x16 s = zero16(), dp;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[buf][1][r0 + 8 * i4 + 4 * lg]);
#pragma unroll
      for (int e = 0; e < 4; ++e) dp[4 * i4 + e] = d4[e];
    }
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
      s = E::mma(rd.row16(Qs, 0, kd), kf[kd], s);
      dp = E::mma(rd.row16(Ds, 0, kd), vf[kd], dp);
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[buf][0][r0 + 8 * i4 + 4 * lg]);  // -LSE log2 e
#pragma unroll
      for (int e = 0; e < 4; ++e) s[4 * i4 + e] = fast_exp2(fmaf(s[4 * i4 + e], c2, l4[e]));
    }
    // tiles that cross the diagonal or hold rows past Lq
    if ((CAUSAL && k0 + BN - 1 > q0 + off) || q0 + BM > Lq) {
      __asm__ volatile("");
      const int thr = CAUSAL ? krow - off - q0 - r0 - 4 * lg : INT_MIN;
      const int rlim = Lq - q0 - r0 - 4 * lg;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = (crow(i, 0) >= thr && crow(i, 0) < rlim) ? s[i] : 0.f;
    }
    // -dS = P (delta - dP)
#pragma unroll
    for (int i = 0; i < 16; ++i) dp[i] = s[i] * dp[i];
    const bf16x8 pf0 = E::pack8(s, 0), pf1 = E::pack8(s, 1);
    const bf16x8 ds0 = E::pack8(dp, 0), ds1 = E::pack8(dp, 1);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[db] = E::mma(rd.trA(Ds, 0, db), pf0, dv[db]);
      dv[db] = E::mma(rd.trA(Ds, 16, db), pf1, dv[db]);
      dk[db] = E::mma(rd.trA(Qs, 0, db), ds0, dk[db]);
      dk[db] = E::mma(rd.trA(Qs, 16, db), ds1, dk[db]);
    }

    rd.flip(BUF);
    if (n + 1 < niter) publish_lse(n + 1);
    wait_vmem();
    __syncthreads();
  }

  // ---- add the two row halves: waves 2-3 hand their partials to waves 0-1
  // through LDS (the tile buffers are free now), lane-contiguous per register
  float* red = reinterpret_cast<float*>(smem);
  static_assert(2 * BUF * 2 >= 2 * NDB * 16 * 64 * 4, "reduction buffer too small");
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dk : dv;
    if (qhalf == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) red[((kb * NDB + db) * 16 + i) * 64 + lane] = acc[db][i];
    }
    __syncthreads();
    if (qhalf == 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] += red[((kb * NDB + db) * 16 + i) * 64 + lane];
    }
    __syncthreads();
  }

  if (sr.part != nullptr) {
    if (qhalf == 0) {
      float* pk = sr.part + (32 * kb + lr) * D;
      float* pv = pk + BN * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16 &ck = dk[db], &cv = dv[db];
          *reinterpret_cast<float4*>(pk + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(ck[4 * q4], ck[4 * q4 + 1], ck[4 * q4 + 2], ck[4 * q4 + 3]);
          *reinterpret_cast<float4*>(pv + 32 * db + 8 * q4 + 4 * lg) =
              make_float4(cv[4 * q4], cv[4 * q4 + 1], cv[4 * q4 + 2], cv[4 * q4 + 3]);
        }
    }
  } else if (qhalf == 0 && key_ok) {
    bf16_t* dkp = a.dk.head(b, hk) + (int64_t)krow * a.dk.sl;
    bf16_t* dvp = a.dv.head(b, hk) + (int64_t)krow * a.dv.sl;
    const float sc = -a.scale;  // the accumulators hold -dK / scale
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16 &ck = dk[db], &cv = dv[db];
        *reinterpret_cast<uint2*>(dkp + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(ck[4 * q4] * sc, ck[4 * q4 + 1] * sc, ck[4 * q4 + 2] * sc, ck[4 * q4 + 3] * sc);
        *reinterpret_cast<uint2*>(dvp + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(cv[4 * q4], cv[4 * q4 + 1], cv[4 * q4 + 2], cv[4 * q4 + 3]);
      }
  }
}

// ---------------------------------------------------------------- dK / dV, wide heads, 32 keys
// Head dim 256 with few key/value heads: with 64-key workgroups a causal
// triangle at 8192 tokens and two heads is 256 workgroups, one per CU, and
// the kernel lasts as long as the first key tile.  Here a workgroup of 4
// wavefronts takes 32 keys, which doubles the workgroups; they are numbered
// key tile major (tile_major), heaviest first, so every XCD gets a share of
// each stretch of key tiles (at two key/value heads: one head, every fourth
// tile), and the second round fills the CUs that light first-round
// workgroups free.
// Wavefront w owns rows 16 w .. 16 w + 15 of every 64-row query tile and all
// 32 keys: S and dP are 16x16x32 products over two 16-key blocks, which
// v_permlane16_swap turns into the k-major B operand of the 32x32x16 dV / dK
// products (k = this wavefront's 16 rows).  The four wavefronts' partial dK /
// dV are added through LDS at the end, each finishing a quarter of the
// columns.
template <class E, int D, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, 1) void fa_dkv_k32_kernel(BwdArgs a) {
  constexpr int BN = 32;  // keys per workgroup
  constexpr int BM = 64;  // query rows per tile, 16 per wavefront
  constexpr int P = Tile<D>::P;
  constexpr int NS = D / 32;   // 16x16x32 steps over the head dim
  constexpr int NDB = D / 32;  // 32-column blocks of dK / dV
  constexpr int OWN = NDB / 4;  // column blocks each wavefront finishes
  static_assert(NDB % 4 == 0, "column blocks must split over four wavefronts");

  constexpr int BUF = 2 * BM * P;  // [Q tile | dO tile]
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];
  __shared__ __attribute__((aligned(16))) float stat[2][2][64];  // [buf][lse / delta][row]

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r0 = 16 * w;  // this wavefront's rows within a tile
  const int G = a.G;
  const TileHead th = tile_major(blockIdx.x, a.B * a.Hkv);  // key tiles x (batch, key/value head)
  const int bh = th.h;
  const int kt = th.t;  // key tile 0 sees the most queries: heaviest first
  const int b = bh / a.Hkv, hk = bh - (bh / a.Hkv) * a.Hkv;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int k0 = kt * BN;
  const int krow = k0 + lr;  // key of this lane's dK / dV column
  const bool key_ok = krow < Lk;

  const int qfirst = CAUSAL ? max(0, k0 - off) : 0;
  const int qt_first = qfirst / BM;
  const int nqt = (Lq + BM - 1) / BM;
  const int nq = max(0, nqt - qt_first);
  // iteration n: query tile nqt - 1 - n / G of query head n % G (last tile
  // first, heads innermost: the workgroups on one XCD share each tile in L2)
  extern __shared__ int qlist[];
  int nql = nq;
  if constexpr (MASKED) {
    const int kb0 = k0 / kMaskBlock, kb1 = (min(k0 + BN, Lk) - 1) / kMaskBlock;
    if (w == 0) {
      const int cnt = build_list(qlist, nq, lane, [&](int i) { return nqt - 1 - i; }, [&](int qtl) {
        bool any = false;
        for (int kbk = kb0; kbk <= kb1; ++kbk) any |= a.mask[qtl * a.nkb + kbk] != 0;
        return any;
      });
      if (lane == 0) qlist[nq] = cnt;
    }
    __syncthreads();
    nql = __builtin_amdgcn_readfirstlane(qlist[nq]);
  }
  const int niter = G * nql;
  auto qtile_of = [&](int n) { return MASKED ? __builtin_amdgcn_readfirstlane(qlist[n / G]) : nqt - 1 - n / G; };

  const TileLoader<D> ldq(w, lane, a.q.sl), ldo(w, lane, a.dO.sl);
  const bf16_t* const qsrc = a.q.head(b, hk * G);
  const bf16_t* const osrc = a.dO.head(b, hk * G);
  const uint32_t smem_a = lds_addr(smem);  // (byte addresses: no pointer conversion per load)
  auto issue = [&](int n) {
    const uint32_t qt_a = smem_a + (uint32_t)(n & 1) * (BUF * 2);
    const int hi = n % G, qtile = qtile_of(n);
    const int64_t qh = (int64_t)(b * a.Hq + hk * G + hi) * Lq;
    const int qbase = qtile * BM;
    if (w == 0) load_row_stat(&stat[n & 1][0][0], a.lse + qh, qbase, Lq, lane);
    if (w == 1) load_row_stat(&stat[n & 1][1][0], a.delta + qh, qbase, Lq, lane);
    ldq.template load_at<BM>(qt_a, qsrc + hi * a.q.sh, qbase, Lq, w);
    ldo.template load_at<BM>(qt_a + BM * P * 2, osrc + hi * a.dO.sh, qbase, Lq, w);
  };
  if (niter > 0) issue(0);

  // K and V as 16x16x32 B fragments: key 16 kb + lane % 16, head-dim slots
  // 32 s + 8 (lane / 16) + e
  bf16x8 kf[NS][2], vf[NS][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kr = min(k0 + 16 * kb + l16, Lk - 1);  // keys past Lk: a copy, never stored
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      kf[st][kb] = as_bf16x8(ldg16(a.k.head(b, hk) + (int64_t)kr * a.k.sl + 32 * st + 8 * g16));
      vf[st][kb] = as_bf16x8(ldg16(a.v.head(b, hk) + (int64_t)kr * a.v.sl + 32 * st + 8 * g16));
    }
  }

  TileReader16<D> rd(lane);
  const float c2 = a.scale_log2;
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  const int rq = r0 + 4 * g16;  // first of this lane's four S rows within a tile

  wait_vmem();
  __syncthreads();
  for (int n = 0; n < niter; ++n) {
    const int buf = n & 1;
    const int q0 = qtile_of(n) * BM;
    if (n + 1 < niter) issue(n + 1);
    const bf16_t* Qs = smem;  // + buf * BUF through the reader's flipped offsets
    const bf16_t* Ds = smem + BM * P;

    f32x4 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kb][i] = dp[kb][i] = 0.f;
    }
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const bf16x8 qa = rd.a16(Qs, r0, st), da = rd.a16(Ds, r0, st);
      s[0] = E::mma16(qa, kf[st][0], s[0]);
      s[1] = E::mma16(qa, kf[st][1], s[1]);
      dp[0] = E::mma16(da, vf[st][0], dp[0]);
      dp[1] = E::mma16(da, vf[st][1], dp[1]);
    }
    const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[buf][0][rq]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], c2, l4[i] * -kLog2e));
    // tiles that cross the diagonal or hold rows past Lq
    if ((CAUSAL && k0 + BN - 1 > q0 + off) || q0 + BM > Lq) {
      __asm__ volatile("");
      const int rlim = Lq - q0 - rq;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int thr = CAUSAL ? k0 + 16 * kb + l16 - off - q0 - rq : INT_MIN;
#pragma unroll
        for (int i = 0; i < 4; ++i) s[kb][i] = (i >= thr && i < rlim) ? s[kb][i] : 0.f;
      }
    }
    // dP is read from its accumulators only after this point.  The products
    // that write it may end right before the branch above, and on the path
    // that skips the masking the compiler has left too few wait states before
    // those reads (stale dP, seen on gfx950): 12 wait states here, on both paths.
    asm volatile("s_nop 7\n\ts_nop 3" : "+a"(dp[0]), "+a"(dp[1]));
    const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[buf][1][rq]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dp[kb][i] = s[kb][i] * (dp[kb][i] - d4[i]);
    // C layout (rows 4 (lane / 16) + i of key block kb) -> B operand (key
    // lane % 32, rows 8 (lane / 32) + e): even 16-lane rows keep block 0 and
    // take the odd row's block 0, odd rows give their block 0 for the even
    // row's block 1
    uint2 p0 = E::pack4(s[0][0], s[0][1], s[0][2], s[0][3]);
    uint2 p1 = E::pack4(s[1][0], s[1][1], s[1][2], s[1][3]);
    uint2 t0 = E::pack4(dp[0][0], dp[0][1], dp[0][2], dp[0][3]);
    uint2 t1 = E::pack4(dp[1][0], dp[1][1], dp[1][2], dp[1][3]);
    swap16(p0.x, p1.x);
    swap16(p0.y, p1.y);
    swap16(t0.x, t1.x);
    swap16(t0.y, t1.y);
    const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(p0.x, p0.y, p1.x, p1.y));
    const bf16x8 dsf = __builtin_bit_cast(bf16x8, make_uint4(t0.x, t0.y, t1.x, t1.y));
    // dV / dK: the transposed reads run two column blocks ahead of their
    // products (one wavefront per SIMD: nothing else covers their latency)
    bf16x8 fo[2], fq[2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
      fo[db] = rd.trA(Ds, r0, db);
      fq[db] = rd.trA(Qs, r0, db);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dv[db] = E::mma(fo[db & 1], pf, dv[db]);
      dk[db] = E::mma(fq[db & 1], dsf, dk[db]);
      if (db + 2 < NDB) {
        fo[db & 1] = rd.trA(Ds, r0, db + 2);
        fq[db & 1] = rd.trA(Qs, r0, db + 2);
      }
    }
    // keep that order: LDS reads (delta, then blocks 0 and 1), then per block
    // its two products and the reads of the block two ahead
    __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (db + 2 < NDB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    }

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }

  // ---- add the four wavefronts' partials: each hands the column blocks it
  // does not finish to their owner through LDS (the tile buffers are free)
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [wave][db][i4][lane]
  static_assert(4 * NDB * 4 * 64 * 16 <= 2 * BUF * 2, "reduction buffer too small");
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dk : dv;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      if (db / OWN != w) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          red[((w * NDB + db) * 4 + i4) * 64 + lane] =
              f32x4{acc[db][4 * i4], acc[db][4 * i4 + 1], acc[db][4 * i4 + 2], acc[db][4 * i4 + 3]};
      }
    __syncthreads();
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      if (db / OWN == w) {
#pragma unroll
        for (int src = 0; src < 4; ++src)
          if (src != w) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const f32x4 v = red[((src * NDB + db) * 4 + i4) * 64 + lane];
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[db][4 * i4 + e] += v[e];
            }
          }
      }
    __syncthreads();
  }

  if (key_ok) {
    bf16_t* dkp = a.dk.head(b, hk) + (int64_t)krow * a.dk.sl;
    bf16_t* dvp = a.dv.head(b, hk) + (int64_t)krow * a.dv.sl;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      if (db / OWN == w) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x16 &ck = dk[db], &cv = dv[db];
          *reinterpret_cast<uint2*>(dkp + 32 * db + 8 * q4 + 4 * lg) =
              E::pack4(ck[4 * q4] * sc, ck[4 * q4 + 1] * sc, ck[4 * q4 + 2] * sc, ck[4 * q4 + 3] * sc);
          *reinterpret_cast<uint2*>(dvp + 32 * db + 8 * q4 + 4 * lg) =
              E::pack4(cv[4 * q4], cv[4 * q4 + 1], cv[4 * q4 + 2], cv[4 * q4 + 3]);
        }
      }
  }
}

// ---------------------------------------------------------------- launchers

template <class E>
static hipError_t launch_delta_e(const DeltaArgs& a, int D, hipStream_t stream) {
  auto go = [&](auto kern, int tpr) {
    const int rpb = 256 / tpr;
    const int64_t nblocks = (a.rows + rpb - 1) / rpb;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  };
  switch (D) {
    case 64: go(fa_delta_kernel<E, 64>, 8); break;
    case 96: go(fa_delta_kernel<E, 96>, 16); break;
    case 128: go(fa_delta_kernel<E, 128>, 16); break;
    case 256: go(fa_delta_kernel<E, 256>, 32); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_delta(const DeltaArgs& a, int D, bool f16, hipStream_t stream) {
  return f16 ? launch_delta_e<FP16>(a, D, stream) : launch_delta_e<BF16>(a, D, stream);
}

template <class E, int D, int BN_Q>
static hipError_t launch_bwd_d(const BwdArgs& a0, bool causal, int which, hipStream_t stream) {
  BwdArgs a = a0;
  // keys per dK/dV workgroup: 128 up to D = 128; at D = 256, 64, or 32 when
  // 64-key workgroups would make fewer than two per CU (measured: 32-key
  // workgroups are faster at 128-258 64-key ones, slower from 512).  With a
  // query-range split (a.part, from a workspace) the 64-key kernel runs: the
  // split balances the causal triangle instead.
  const bool split = a.part != nullptr && a.nsplit > 1;
  if (!split) {
    a.nsplit = 1;
    a.part = nullptr;
    a.split_cnt = nullptr;
    a.plan = nullptr;
  }
  const bool k32 = D > 128 && !split && (int64_t)a.B * a.Hkv * ((a.Lk + 63) / 64) < 512;
  // head dim 64 without a split: 64-key workgroups of four wavefronts, two per CU
  const bool kb2 = D == 64 && !split;
  // head dims 96 and 128 without a causal mask or a split: four wavefronts of
  // the same 128 keys over 32-row query tiles, two workgroups per CU
  const bool h1 = (D == 96 || D == 128) && !split && !causal;
  const int bnk = D > 128 ? (k32 ? 32 : 64) : kb2 ? 64 : 128;
  a.nkt = (a.Lk + bnk - 1) / bnk;
  // the dK accumulators of the kernels that write partials hold -dK / scale
  // (V negated)
  a.ksc = -a.scale;
  const bool masked = a.mask != nullptr;
  // dynamic LDS under a block mask: each workgroup's tile list and its count
  const size_t dq_list = masked ? ((size_t)(a.Lk + BN_Q - 1) / BN_Q + 1) * sizeof(int) : 0;
  const size_t dkv_list = masked ? ((size_t)(a.Lq + (h1 ? 31 : 63)) / (h1 ? 32 : 64) + 1) * sizeof(int) : 0;
  const int nh = a.B * a.Hkv;
  const int ndq = (which & 1) ? a.B * a.Hq * a.nqt : 0;
  // dK/dV workgroups: key tiles (x chunks without a mask; extra chunks first
  // under one)
  const int ndkv = !(which & 2) ? 0 : !split ? nh * a.nkt : masked ? a.nextra + nh * a.nkt : nh * a.nkt * a.nsplit;
  auto dq = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(ndq), dim3(256), dq_list, stream, a); };
  auto dkv = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(ndkv), dim3(D > 128 || kb2 || h1 ? 256 : 512), dkv_list, stream, a);
  };
  if (split && masked && ndkv > 0) {
    constexpr int BMK = D == 64 ? 128 : 64;  // the dK/dV kernel's query tile
    if (causal)
      hipLaunchKernelGGL((fa_dkv_count_kernel<BMK, dkv_split_keys(D), true>), dim3(a.nkt), dim3(64), 0, stream, a);
    else
      hipLaunchKernelGGL((fa_dkv_count_kernel<BMK, dkv_split_keys(D), false>), dim3(a.nkt), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(fa_dkv_plan_kernel, dim3(1), dim3(1024), 0, stream, a);
  }
  if (ndq > 0) {
    if (causal)
      masked ? dq(fa_dq_kernel<E, D, BN_Q, true, true>) : dq(fa_dq_kernel<E, D, BN_Q, true, false>);
    else
      masked ? dq(fa_dq_kernel<E, D, BN_Q, false, true>) : dq(fa_dq_kernel<E, D, BN_Q, false, false>);
  }
  if (ndkv > 0) {
    if constexpr (D > 128) {
      if (k32) {
        if (causal)
          masked ? dkv(fa_dkv_k32_kernel<E, D, true, true>) : dkv(fa_dkv_k32_kernel<E, D, true, false>);
        else
          masked ? dkv(fa_dkv_k32_kernel<E, D, false, true>) : dkv(fa_dkv_k32_kernel<E, D, false, false>);
      } else if (causal)
        masked ? dkv(fa_dkv_reg_kernel<E, D, true, true>) : dkv(fa_dkv_reg_kernel<E, D, true, false>);
      else
        masked ? dkv(fa_dkv_reg_kernel<E, D, false, true>) : dkv(fa_dkv_reg_kernel<E, D, false, false>);
    } else {
      auto go = [&](auto kb) {
        constexpr int KB = decltype(kb)::value;
        if (causal)
          masked ? dkv(fa_dkv_kernel<E, D, true, true, KB>) : dkv(fa_dkv_kernel<E, D, true, false, KB>);
        else
          masked ? dkv(fa_dkv_kernel<E, D, false, true, KB>) : dkv(fa_dkv_kernel<E, D, false, false, KB>);
      };
      if constexpr (D == 64) {
        if (kb2) go(std::integral_constant<int, 2>{});
        else go(std::integral_constant<int, 4>{});
      } else {
        if (h1)
          masked ? dkv(fa_dkv_kernel<E, D, false, true, 4, true>) : dkv(fa_dkv_kernel<E, D, false, false, 4, true>);
        else
          go(std::integral_constant<int, 4>{});
      }
    }
    if (split)
      hipLaunchKernelGGL((fa_dkv_reduce_kernel<E, D, dkv_split_keys(D)>),
                         dim3(nh * (masked ? a.jmax : a.nkt) * kReduceSlices), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_bwd_e(const BwdArgs& a, int D, bool causal, int which, hipStream_t stream) {
  switch (D) {
    case 64: return launch_bwd_d<E, 64, 64>(a, causal, which, stream);
    case 96: return launch_bwd_d<E, 96, 64>(a, causal, which, stream);
    case 128: return launch_bwd_d<E, 128, 64>(a, causal, which, stream);
    case 256: return launch_bwd_d<E, 256, 64>(a, causal, which, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int which, bool f16, hipStream_t stream) {
  return f16 ? launch_bwd_e<FP16>(a, D, causal, which, stream) : launch_bwd_e<BF16>(a, D, causal, which, stream);
}

}  // namespace cgqa
