// Forward attention kernel for gfx950: tiled online softmax that writes O and
// one log-sum-exp per query row.
//
// Method: page "When the Bottleneck Moved: From Fused Cross-Entropy to
// FlashAttention on MLX", section 3 (running max m, denominator l and
// unnormalised accumulator per key block; O = acc / l, L = m + log l), in the
// base-2 domain of page "feat(attention): complete Flash Attention VJP
// implementation", "Reference implementation" section (exp2 with the scale
// pre-multiplied by log2 e); key blocks entirely above the causal diagonal
// are skipped (same page, "When fused wins: causal masking").
//
// Work decomposition (one workgroup = 4 wavefronts = 128 query rows of one
// query head; each wavefront owns 32 rows):
//   S^T = K Q^T on MFMA: K (the A operand) comes from LDS, Q^T (B operand)
//   stays in registers for the whole key loop.  Computing the transpose puts
//   one query row per lane pair, so row max / row sum are per-lane plus one
//   exchange with the lane 32 away.
//   O^T += V^T P^T on MFMA: P^T goes from the fp32 C layout to bf16 operand
//   registers directly; V^T is read from the row-major V tile with the
//   transposed LDS read.
// K and V tiles are double buffered in LDS and filled by direct global->LDS
// loads issued one tile ahead.  Tiles that need no mask (fully below the
// diagonal and inside Lk) run a mask-free body.  At head dim 256 (one
// wavefront per SIMD, nothing to hide one wavefront's softmax behind) and
// without a block mask, K runs a tile ahead of V instead: the scores of the
// next tile go to the matrix cores between the current tile's exponentials.
//
// Running max with slack: the accumulator is rescaled only when some row's
// max grows by more than 2^8 (in exp2 units) over the max it was last scaled
// with.  O = acc / l and L = m + log2 l do not depend on which m is used, and
// with the slack every p = exp2(s - m) stays <= 256, far from overflow.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

// LDS reads kept this many fragments ahead of the MFMAs that use them
constexpr int kLookahead = 6;

template <class E, int D, int BN, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void fa_fwd_kernel(FwdArgs a) {
  constexpr int BM = 128;
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16;      // 16-wide k steps over the head dim
  constexpr int NDB = D / 32;      // 32-row blocks of O^T
  constexpr int NNB = BN / 32;     // 32-key blocks per key tile
  constexpr int NKS = BN / 16;     // 16-key k steps per key tile
  constexpr float kSlack = 8.f;

  // two buffers of [K tile | V tile], BUF elements apart (a power of two)
  constexpr int BUF = 2 * BN * P;
  static_assert((BUF & (BUF - 1)) == 0, "buffer size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[2 * BUF];

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- which (batch, head, query tile) this workgroup computes
  const int G = a.G;
  const TileHead th = tile_major(blockIdx.x, a.B * a.Hq);  // query tiles x (batch, query head)
  const int t = th.t, bg = th.h / G, hi = th.h - (th.h / G) * G;
  const int qt = CAUSAL ? (a.nqt - 1 - t) : t;  // heaviest tiles first
  const int b = bg / a.Hkv, hk = bg - (bg / a.Hkv) * a.Hkv;
  const int hq = hk * G + hi;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const bf16_t* qp = a.q.head(b, hq);
  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  const int qs = a.q.sl, ks = a.k.sl, vs = a.v.sl;

  const int q0 = qt * BM;
  const int qrow = q0 + 32 * w + lr;

  // ---- key range: causal rows see keys j <= i + off
  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, min(q0 + BM, Lq) + off);
  const int nkt = (kv_end + BN - 1) / BN;
  int n_full = Lk / BN;  // tiles that need no mask
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
  // mask row of this wavefront's 32 rows (rows past Lq: none, the wave idles)
  const int wqb = (q0 + 32 * w) / kMaskBlock;
  const bool w_rows = q0 + 32 * w < Lq;

  const TileLoader<D> ldk(w, lane, ks), ldv(w, lane, vs);
  const uint32_t smem_a = lds_addr(smem);  // (byte addresses: no pointer conversion per load)
  // K (and V) of tile ti into buffer ti & 1
  auto issue_k = [&](int ti) {
    ldk.template load_at<BN>(smem_a + (uint32_t)(ti & 1) * (BUF * 2), kp, tile(ti) * BN, Lk, w);
  };
  auto issue_v = [&](int ti) {
    ldv.template load_at<BN>(smem_a + (uint32_t)(ti & 1) * (BUF * 2) + BN * P * 2, vp, tile(ti) * BN, Lk, w);
  };
  // One wavefront per SIMD (head dim 256) without a block mask: K runs one
  // tile ahead of V, so that the scores of tile ti + 1 go to the matrix cores
  // while tile ti is exponentiated (the second loop below).
  constexpr bool LEAD = D > 128 && !MASKED;
  if (nt > 0) {
    issue_k(0);
    issue_v(0);
  }
  if (LEAD && nt > 1) issue_k(1);

  // ---- Q^T operand (B): lane holds query qrow, head-dim slots 16*kd + 8*lg + s
  bf16x8 qf[NKD];
  {
    const int qr = min(qrow, Lq - 1);  // rows past Lq compute on a copy; never stored
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + (int64_t)qr * qs + 16 * kd + 8 * lg));
  }

  TileReader<D> rd(lane);  // offsets point into buffer (ti & 1); flipped every tile
  const float c2 = a.scale_log2;
  float m_run = -INFINITY;  // max (exp2 units) the accumulator is scaled with
  float l_run = 0.f;        // this lane's share of the running denominator
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  if constexpr (!LEAD) {
  wait_vmem();
  __syncthreads();
  for (int ti = 0; ti < nt; ++ti) {
    const int j = tile(ti);
    if (ti + 1 < nt) {
      issue_k(ti + 1);
      issue_v(ti + 1);
    }
    const bf16_t* Ks = smem;           // + (ti & 1) * BUF through the reader's offsets
    const bf16_t* Vs = smem + BN * P;
    bool skip = false;  // this wavefront's rows do not see tile j
    if constexpr (MASKED) skip = !w_rows || a.mask[wqb * a.nkb + j * BN / kMaskBlock] == 0;
    if (!skip) {
    f32x16 s[NNB];
    prio_hi();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) s[nb] = E::mma(rd.row16(Ks, nb * 32, kd), qf[kd], s[nb]);
    }
    // keep LDS reads kLookahead fragments ahead of the products that use them
    __builtin_amdgcn_sched_group_barrier(0x100, kLookahead, 0);
#pragma unroll
    for (int t = 0; t < NNB * NKD - kLookahead; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kLookahead, 0);
    prio_lo();
    if (j >= n_full) {  // diagonal or ragged tile: hide keys past the diagonal or past Lk
      __asm__ volatile("");  // keep this a real branch (not speculated into every tile)
      // key = base + crow(i, 0) is visible iff crow(i, 0) <= last - base
      const int last = CAUSAL ? min(qrow + off, Lk - 1) : Lk - 1;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (j * BN + nb * 32 + 4 * lg);
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
    prio_hi();
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[db] = E::mma(rd.trA(Vs, 16 * ks, db), pf[ks], acc[db]);
    prio_lo();
    }

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }
  } else {
    // Iteration ti holds S(ti) (computed in the iteration before) and issues
    // K(ti + 2) and V(ti + 1); it forms S(ti + 1) = K(ti + 1) Q^T with the
    // softmax of S(ti) laid between those products (they do not depend on
    // each other), then O += P(ti) V(ti).  K(ti + 1) and V(ti) are resident:
    // the key-read offsets run one buffer ahead of the transposed ones.
    const bf16_t* Ks = smem;
    const bf16_t* Vs = smem + BN * P;
    auto scores = [&](f32x16 (&t)[NNB]) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        t[nb] = zero16();
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) t[nb] = E::mma(rd.row16(Ks, nb * 32, kd), qf[kd], t[nb]);
      }
    };
    // hide keys past the diagonal or past Lk (tile j; every tile from
    // n_full on), without a branch
    auto mask_tile = [&](f32x16 (&t)[NNB], int j) {
      const int last = CAUSAL ? min(qrow + off, Lk - 1) : Lk - 1;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (j * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int i = 0; i < 16; ++i) t[nb][i] = (crow(i, 0) <= thr) ? t[nb][i] : -INFINITY;
      }
    };
    // running max of S (exp2 units): a candidate for m_run
    auto tile_max = [&](const f32x16 (&t)[NNB]) {
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, t[nb][i]);
      return max_xor32(mx) * c2;
    };
    f32x16 sc[NNB];
    wait_vmem();
    __syncthreads();
    if (nt > 0) {
      scores(sc);
      if (n_full == 0) mask_tile(sc, 0);
      m_run = tile_max(sc);  // (the accumulator is still zero)
    }
    rd.flip_ra(BUF);
    __syncthreads();  // K(0) read by every wavefront before K(2) goes to its buffer
    // Iteration ti, one basic block up to the rare rescale: S(ti + 1) on the
    // matrix cores with the exponentials of S(ti) between the products, then
    // O += P(ti) V(ti) with the mask and running max of S(ti + 1) between
    // those.  If that max grew past the slack, the accumulator is rescaled
    // after the products (it then holds tiles up to ti, all at the old max).
    // The exponentials need only m_run from the iteration before; the loop is
    // split where the next tile starts to need the mask, so that no branch
    // sits between them and the products they hide under.
    auto step = [&](int ti, auto has_next, auto mask_next) {
      constexpr bool NXT = decltype(has_next)::value;
      constexpr bool MSK = decltype(mask_next)::value;
      if constexpr (NXT) {
        if (ti + 2 < nt) issue_k(ti + 2);
        issue_v(ti + 1);
      }
      f32x16 sn[NNB];
      if constexpr (NXT) scores(sn);
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float rs = 0.f;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(sc[nb][i], c2, -m_use));
          sc[nb][i] = p;
          rs += p;
        }
      bf16x8 pf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) pf[ks] = E::pack8(sc[ks / 2], ks % 2);
      l_run += rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) acc[db] = E::mma(rd.trA(Vs, 16 * ks, db), pf[ks], acc[db]);
      if constexpr (NXT) {
        if constexpr (MSK) mask_tile(sn, ti + 1);
        const float m_cand = tile_max(sn);
        // score products: K reads kLookahead ahead, exponentials between
        __builtin_amdgcn_sched_group_barrier(0x100, kLookahead, 0);
#pragma unroll
        for (int t = 0; t < NNB * NKD - kLookahead; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 5, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kLookahead, 0);
        // P V products: V reads four products ahead, mask and max between
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int t = 0; t < NDB * NKS - 4; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        const bool resc = __any(m_cand > m_run + kSlack);
        if (resc) {
          __asm__ volatile("");  // a real branch: the rescale is rare
          const float m_new = fmaxf(m_run, m_cand);
          const float alpha = (m_new == m_run) ? 1.f : fast_exp2(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) scale_agpr(acc[db], alpha);
          m_run = m_new;
        }
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) sc[nb] = sn[nb];
        rd.flip(BUF);
        wait_vmem();
        __syncthreads();
      }
    };
    // (without a block mask tile(ti) = ti: tile ti + 1 needs the mask from n_full on)
    int ti = 0;
    for (; ti + 1 < min(nt, n_full); ++ti) step(ti, std::true_type{}, std::false_type{});
    for (; ti + 1 < nt; ++ti) step(ti, std::true_type{}, std::true_type{});
    if (nt > 0) step(nt - 1, std::false_type{}, std::false_type{});
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2; a row that saw no
  // key (possible only under a block mask) gets O = 0, LSE = -inf
  const float l_tot = l_run + xor32(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    bf16_t* op = a.o.head(b, hq) + (int64_t)qrow * a.o.sl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = acc[db];
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(c[4 * q4] * inv, c[4 * q4 + 1] * inv, c[4 * q4 + 2] * inv, c[4 * q4 + 3] * inv);
      }
    if (lg == 0)
      a.lse[(int64_t)(b * a.Hq + hq) * Lq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------- ping-pong
// Head dims 96 and 128.  One workgroup = 8 wavefronts = 256 query rows of one
// query head, 32 rows per wavefront, the same per-tile products as above.
// Wavefronts w and w + 4 share a SIMD.  On gfx950 a tile's softmax costs a
// wavefront about as much vector time (32 exponentials at a quarter of the
// FMA rate, plus max, sum and conversion) as its products cost matrix time,
// and within one wavefront the two depend on each other.  So the two groups
// (waves 0-3 and 4-7) run half a key tile apart, in phases separated by
// workgroup barriers:
//   phase 2j     group A: S(j) = K_j Q^T and O += P(j-1) V(j-1)   (matrix)
//                group B: softmax of S(j-1) -> P(j-1)             (vector)
//   phase 2j + 1 group A: softmax of S(j) -> P(j)                 (vector)
//                group B: S(j) and O += P(j-1) V(j-1)             (matrix)
// K and V tiles each rotate through four LDS buffers.  Only matrix steps
// issue loads (a load issue can stall its wavefront): group A's matrix step j
// loads K_{j+2}, group B's loads V_{j+1}, and each ends by waiting for its
// previous batch, so a tile is resident at least one phase before it is read.
// A vector step also reads the next matrix step's K fragments into registers,
// so that step's S products start on register operands.
template <class E, int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fa_fwd_pp_kernel(FwdArgs a) {
  constexpr int BM = 256;
  constexpr int P = Tile<D>::P;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NNB = BN / 32;
  constexpr int NKS = BN / 16;
  constexpr int ROUNDS = BN * Tile<D>::PC / 256;  // direct loads per wavefront per tile
  constexpr float kSlack = 8.f;

  // K tiles at [0, 4*TILE), V tiles at [4*TILE, 8*TILE); tile j in buffer j & 3
  constexpr int TILE = BN * P;
  static_assert((TILE & (TILE - 1)) == 0, "tile size must be a power of two");
  __shared__ __attribute__((aligned(1024))) bf16_t smem[8 * TILE];
  bf16_t* const sK = smem;
  bf16_t* const sV = smem + 4 * TILE;

  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool grp_b = w >= 4;

  const int G = a.G;
  const TileHead th = tile_major(blockIdx.x, a.B * a.Hq);  // query tiles x (batch, query head)
  const int t = th.t, bg = th.h / G, hi = th.h - (th.h / G) * G;
  const int qt = CAUSAL ? (a.nqt - 1 - t) : t;  // heaviest tiles first
  const int b = bg / a.Hkv, hk = bg - (bg / a.Hkv) * a.Hkv;
  const int hq = hk * G + hi;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const bf16_t* qp = a.q.head(b, hq);
  const bf16_t* kp = a.k.head(b, hk);
  const bf16_t* vp = a.v.head(b, hk);
  const int qs = a.q.sl, ks = a.k.sl, vs = a.v.sl;

  const int q0 = qt * BM;
  const int r0 = q0 + 32 * w;  // this wavefront's first row
  const int qrow = r0 + lr;

  // key tiles of the workgroup, and of this wavefront (a prefix of them)
  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, min(q0 + BM, Lq) + off);
  const int nkt = (kv_end + BN - 1) / BN;
  int wv_end = Lk;
  if (CAUSAL) wv_end = min(Lk, min(r0 + 32, Lq) + off);
  const int wnkt = r0 < Lq ? (wv_end + BN - 1) / BN : 0;
  int n_full = Lk / BN;  // tiles this wavefront reads without a mask
  if (CAUSAL) n_full = min(n_full, (r0 + off + 1) / BN);
  n_full = max(0, min(n_full, wnkt));

  const int nt = nkt;
  // does this wavefront's work include key tile x?
  auto need = [&](int x) { return x >= 0 && x < wnkt; };

  const TileLoader<D> ld(w & 3, lane, w < 4 ? ks : vs);  // waves 0-3 load K, 4-7 load V
  if (w < 4) {
    if (nt > 0) ld.template load<BN>(sK, kp, 0, Lk, w);
    if (nt > 1) ld.template load<BN>(sK + TILE, kp, BN, Lk, w);
  } else {
    if (nt > 0) ld.template load<BN>(sV, vp, 0, Lk, w & 3);
  }

  bf16x8 qf[NKD];
  {
    const int qr = min(qrow, Lq - 1);  // rows past Lq compute on a copy; never stored
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + (int64_t)qr * qs + 16 * kd + 8 * lg));
  }

  // row reads (K) follow key tile x of the matrix step, transposed reads
  // (V) tile x - 1; buffer b sits b * TILE elements in, so moving from
  // buffer x & 3 to (x + 1) & 3 is an XOR of the offsets with
  // (x odd ? 3 : 1) * TILE
  TileReaderX<D> rd(lane);
  rd.shift_tr(4 * TILE * 2);  // the transposed reads (V) are given smem, not sV
  const float c2 = a.scale_log2;
  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();
  f32x16 s[NNB];
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) s[nb] = zero16();
  bf16x8 pf[NKS];

  // loads issued by matrix step x: K of tile x + 2 (waves 0-3) or V of
  // tile x + 1 (waves 4-7); returns whether this wavefront issued any
  // (LDS destinations as byte addresses: no generic-pointer conversion per load)
  const uint32_t sK_a = lds_addr(sK), sV_a = lds_addr(sV);
  auto loads = [&](int x) -> bool {
    if (w < 4) {
      if (x + 2 >= nt) return false;
      ld.template load_at<BN>(sK_a + (uint32_t)((x + 2) & 3) * (TILE * 2), kp, (x + 2) * BN, Lk, w);
    } else {
      if (x + 1 >= nt) return false;
      ld.template load_at<BN>(sV_a + (uint32_t)((x + 1) & 3) * (TILE * 2), vp, (x + 1) * BN, Lk, w & 3);
    }
    return true;
  };
  // end of a matrix step: this wavefront's previous batch of loads must have
  // landed, the one just issued may still be in flight
  auto wait_loads = [&](bool issued) {
    if (issued)
      wait_vmem_n<ROUNDS>();
    else
      wait_vmem();
  };
  // K fragments of the next matrix step, read into registers during the
  // vector step before it (the tile is resident by then)
  bf16x8 kf[NNB * NKD];
  auto prefetch_k = [&]() {
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) kf[nb * NKD + kd] = rd.row16(sK, nb * 32, kd);
  };
  // matrix step j: S(j), then O += P(j-1) V(j-1); independent accumulators
  // interleaved so that consecutive MFMAs do not wait on each other.  The
  // step also issues this wavefront's tile loads, so that the wavefronts in
  // their vector step never wait on a load issue, and ends with the wait for
  // its previous batch.
  auto mstep = [&](int x) {
    const bool issued = loads(x);
    if (need(x)) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) s[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb) s[nb] = E::mma(kf[nb * NKD + kd], qf[kd], s[nb]);
    }
    if (need(x - 1)) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] = E::mma(rd.trA(smem, 16 * ks, db), pf[ks], acc[db]);
      // the transposed reads run kLookahead ahead of the products (the K
      // fragments' registers are free by now)
      constexpr int NM = NKS * NDB, NR = 2 * NM, LA = kLookahead < NR ? kLookahead : NR;
      static_assert(LA % 2 == 0 && LA <= NR, "read pattern");
      __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
      for (int t = 0; t < (NR - LA) / 2; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - LA) / 2, 0);
    }
    rd.flip_ra(((x & 1) ? 3 : 1) * TILE);
    if (x >= 1) rd.flip_tr((((x - 1) & 1) ? 3 : 1) * TILE);
    wait_loads(issued);
  };
  // vector step x: softmax of S(x) into P
  auto vstep = [&](int x) {
    if (!need(x)) return;
    const int j = x;
    if (j >= n_full) {  // diagonal or ragged tile
      __asm__ volatile("");
      const int last = CAUSAL ? min(qrow + off, Lk - 1) : Lk - 1;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        const int thr = last - (j * BN + nb * 32 + 4 * lg);
#pragma unroll
        for (int i = 0; i < 16; ++i) s[nb][i] = (crow(i, 0) <= thr) ? s[nb][i] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = max_xor32(mx);
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
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = E::pack8(s[ks / 2], ks % 2);
  };

  wait_vmem();
  __syncthreads();
  // 2 * (nkt + 1) phases; every wavefront passes the same barriers
  if (!grp_b) {
    if (need(0)) prefetch_k();
    for (int x = 0; x <= nt; ++x) {
      mstep(x);
      __syncthreads();
      if (need(x + 1)) prefetch_k();
      vstep(x);
      __syncthreads();
    }
  } else {
    for (int x = 0; x <= nt; ++x) {
      if (need(x)) prefetch_k();
      vstep(x - 1);
      __syncthreads();
      mstep(x);
      __syncthreads();
    }
  }

  const float l_tot = l_run + xor32(l_run);
  if (qrow < Lq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;  // no key seen (block mask): O = 0
    bf16_t* op = a.o.head(b, hq) + (int64_t)qrow * a.o.sl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& c = acc[db];
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * q4 + 4 * lg) =
            E::pack4(c[4 * q4] * inv, c[4 * q4 + 1] * inv, c[4 * q4 + 2] * inv, c[4 * q4 + 3] * inv);
      }
    if (lg == 0)
      a.lse[(int64_t)(b * a.Hq + hq) * Lq + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <class E, int D, int BN>
static hipError_t launch_fwd_d(const FwdArgs& a0, bool causal, hipStream_t stream) {
  FwdArgs a = a0;
  const bool masked = a.mask != nullptr;
  // dynamic LDS under a block mask: the workgroup's key-tile list and its count
  const size_t list_bytes = masked ? ((size_t)(a.Lk + BN - 1) / BN + 1) * sizeof(int) : 0;
  auto go = [&](auto kern, int threads) {
    hipLaunchKernelGGL(kern, dim3(a.B * a.Hq * a.nqt), dim3(threads), list_bytes, stream, a);
  };
  // ping-pong for D = 96 and 128 without a mask.  At D = 64 the 4-wavefront
  // kernel runs four wavefronts per SIMD, which hides latency better; under a
  // block mask its 128-row workgroups visit fewer key tiles than 256-row ones
  // (measured faster with a 1024-key sliding window at 8192 tokens)
  if constexpr (D == 96 || D == 128) {
    if (!masked) {
      a.nqt = (a.Lq + 255) / 256;
      causal ? go(fa_fwd_pp_kernel<E, D, BN, true>, 512) : go(fa_fwd_pp_kernel<E, D, BN, false>, 512);
      return hipGetLastError();
    }
  }
  {
    a.nqt = (a.Lq + 127) / 128;
    if (causal)
      masked ? go(fa_fwd_kernel<E, D, BN, true, true>, 256) : go(fa_fwd_kernel<E, D, BN, true, false>, 256);
    else
      masked ? go(fa_fwd_kernel<E, D, BN, false, true>, 256) : go(fa_fwd_kernel<E, D, BN, false, false>, 256);
  }
  return hipGetLastError();
}

template <class E>
static hipError_t launch_fwd_e(const FwdArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_fwd_d<E, 64, 64>(a, causal, stream);
    case 96: return launch_fwd_d<E, 96, 64>(a, causal, stream);
    case 128: return launch_fwd_d<E, 128, 64>(a, causal, stream);
    case 256: return launch_fwd_d<E, 256, 64>(a, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, bool f16, hipStream_t stream) {
  return f16 ? launch_fwd_e<FP16>(a, D, causal, stream) : launch_fwd_e<BF16>(a, D, causal, stream);
}

}  // namespace cgqa
