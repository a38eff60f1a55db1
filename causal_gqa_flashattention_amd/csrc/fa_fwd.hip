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
// diagonal and inside Lk) run a mask-free body.
//
// Running max with slack: the accumulator is rescaled only when some row's
// max grows by more than 2^8 (in exp2 units) over the max it was last scaled
// with.  O = acc / l and L = m + log2 l do not depend on which m is used, and
// with the slack every p = exp2(s - m) stays <= 256, far from overflow.
#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

template <int D, int BN, bool CAUSAL>
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
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = a.nqt * G;
  const int bg = logical / per_group;
  const int rr = logical - bg * per_group;
  const int t = rr / G, hi = rr - (rr / G) * G;
  const int qt = CAUSAL ? (a.nqt - 1 - t) : t;  // heaviest tiles first
  const int b = bg / a.Hkv, hk = bg - (bg / a.Hkv) * a.Hkv;
  const int hq = hk * G + hi;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const bf16_t* qp = a.q + ((int64_t)(b * a.Hq + hq) * Lq) * D;
  const bf16_t* kp = a.k + ((int64_t)(b * a.Hkv + hk) * Lk) * D;
  const bf16_t* vp = a.v + ((int64_t)(b * a.Hkv + hk) * Lk) * D;

  const int q0 = qt * BM;
  const int qrow = q0 + 32 * w + lr;

  // ---- key range: causal rows see keys j <= i + off
  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, min(q0 + BM, Lq) + off);
  const int nkt = (kv_end + BN - 1) / BN;
  int n_full = Lk / BN;  // tiles that need no mask
  if (CAUSAL) n_full = min(n_full, (q0 + off + 1) / BN);
  n_full = max(0, min(n_full, nkt));

  const TileLoader<D> ld(w, lane);
  auto issue = [&](int j) {
    bf16_t* buf = smem + (j & 1) * BUF;
    ld.template load<BN>(buf, kp, j * BN, Lk, w);
    ld.template load<BN>(buf + BN * P, vp, j * BN, Lk, w);
  };
  if (nkt > 0) issue(0);

  // ---- Q^T operand (B): lane holds query qrow, head-dim slots 16*kd + 8*lg + s
  bf16x8 qf[NKD];
  {
    const int qr = min(qrow, Lq - 1);  // rows past Lq compute on a copy; never stored
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + (int64_t)qr * D + 16 * kd + 8 * lg));
  }

  TileReader<D> rd(lane);  // offsets point into buffer (j & 1); flipped every tile
  const float c2 = a.scale_log2;
  float m_run = -INFINITY;  // max (exp2 units) the accumulator is scaled with
  float l_run = 0.f;        // this lane's share of the running denominator
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  wait_vmem();
  __syncthreads();
  for (int j = 0; j < nkt; ++j) {
    if (j + 1 < nkt) issue(j + 1);
    const bf16_t* Ks = smem;           // + (j & 1) * BUF through the reader's offsets
    const bf16_t* Vs = smem + BN * P;

    f32x16 s[NNB];
    prio_hi();
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) s[nb] = mfma32(rd.row16(Ks, nb * 32, kd), qf[kd], s[nb]);
    }
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
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = pack8(s[ks / 2], ks % 2);
    prio_hi();
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) acc[db] = mfma32(rd.trA(Vs, 16 * ks, db), pf[ks], acc[db]);
    prio_lo();

    rd.flip(BUF);
    wait_vmem();
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
  const float l_tot = l_run + xor32(l_run);
  if (qrow < Lq) {
    const float inv = 1.f / l_tot;
    bf16_t* op = a.o + ((int64_t)(b * a.Hq + hq) * Lq + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][4 * q4 + e] * inv);
        *reinterpret_cast<bf16x4*>(op + 32 * db + 8 * q4 + 4 * lg) = v4;
      }
    if (lg == 0) a.lse[(int64_t)(b * a.Hq + hq) * Lq + qrow] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, int BN>
static hipError_t launch_fwd_d(const FwdArgs& a, bool causal, hipStream_t stream) {
  const int nblocks = a.B * a.Hq * a.nqt;
  if (causal)
    hipLaunchKernelGGL((fa_fwd_kernel<D, BN, true>), dim3(nblocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((fa_fwd_kernel<D, BN, false>), dim3(nblocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_fwd_d<64, 64>(a, causal, stream);
    case 96: return launch_fwd_d<96, 64>(a, causal, stream);
    case 128: return launch_fwd_d<128, 64>(a, causal, stream);
    case 256: return launch_fwd_d<256, 32>(a, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cgqa
