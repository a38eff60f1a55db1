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
//   one query row per lane (two lanes per row), so row max / row sum are
//   per-lane plus one exchange with the lane 32 away.
//   O^T += V^T P^T on MFMA: P^T goes from the fp32 C layout to bf16 operand
//   registers directly; V^T is read from the row-major V tile with the
//   transposed LDS read.
// K and V tiles are double buffered in LDS; the next tile's global loads are
// in flight while the current tile is computed.
#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void fa_fwd_kernel(FwdArgs a) {
  constexpr int BM = 128;
  constexpr int KP = D + 8;        // LDS row pitch in elements (pads banks)
  constexpr int NKD = D / 16;      // 16-wide k steps over the head dim
  constexpr int NDB = D / 32;      // 32-row blocks of O^T
  constexpr int NNB = BN / 32;     // 32-key blocks per key tile
  constexpr int NKS = BN / 16;     // 16-key k steps per key tile
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int CPT = BN * CPR / 256;
  static_assert(BN * CPR % 256 == 0, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][BN * KP];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;

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

  // ---- Q^T operand (B): lane holds query qrow, head-dim slots 16*kd + 8*lg + s
  bf16x8 qf[NKD];
  if (qrow < Lq) {
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(ldg16(qp + (int64_t)qrow * D + 16 * kd + 8 * lg));
  } else {
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) qf[kd] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  // ---- key range: causal rows see keys j <= i + off
  int kv_end = Lk;
  if (CAUSAL) kv_end = min(Lk, min(q0 + BM, Lq) + off);
  const int nkt = (kv_end + BN - 1) / BN;

  uint4 rk[CPT], rv[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      const int key = j * BN + row;
      if (key < Lk) {
        rk[c] = ldg16(kp + (int64_t)key * D + col);
        rv[c] = ldg16(vp + (int64_t)key * D + col);
      } else {
        rk[c] = make_uint4(0, 0, 0, 0);  // zero rows past Lk: no NaN can leak
        rv[c] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      *reinterpret_cast<uint4*>(&lds[buf][0][row * KP + col]) = rk[c];
      *reinterpret_cast<uint4*>(&lds[buf][1][row * KP + col]) = rv[c];
    }
  };

  const float c2 = a.scale_log2;
  float m_run = -INFINITY;  // running max of scaled scores (base-2 units)
  float l_run = 0.f;        // this lane's share of the running denominator
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = zero16();

  const int troff = tr_lane_offset(lane, KP);

  if (nkt > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < nkt; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkt) load_tile(j + 1);
    const bf16_t* Ks = lds[buf][0];
    const bf16_t* Vs = lds[buf][1];

    // S^T block: rows = keys, lane column = query
    f32x16 s[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd)
        s[nb] = mfma32(lds_read16(Ks + (nb * 32 + lr) * KP + 16 * kd + 8 * lg), qf[kd], s[nb]);
    }

    const int kbase = j * BN;
    const bool need_mask = (kbase + BN > Lk) || (CAUSAL && kbase + BN - 1 > q0 + off);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + nb * 32 + crow(i, lg);
          const bool vis = key < Lk && (!CAUSAL || key <= qrow + off);
          if (!vis) s[nb][i] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[nb][i]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[nb][i], c2, -m_use));
        s[nb][i] = p;
        rs += p;
      }
    l_run = fmaf(l_run, alpha, rs);
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

    bf16x8 pf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) pf[ks] = pack8(s[ks / 2], ks % 2);

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        acc[db] = mfma32(lds_read_trA(Vs, troff, 16 * ks, 32 * db, KP), pf[ks], acc[db]);

    if (j + 1 < nkt) store_tile(buf ^ 1);
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
