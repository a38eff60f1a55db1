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
#include "fa_device.h"
#include "fa_kernels.h"

namespace cgqa {

// ---------------------------------------------------------------- delta
// delta[row] = sum_d f32(O[row, d]) * f32(dO[row, d]).  HBM-bound: each
// thread reads 16 bytes of O and of dO; TPR threads share one row.
template <int D>
__global__ __launch_bounds__(256) void fa_delta_kernel(DeltaArgs a) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int TPR = CPR <= 8 ? 8 : (CPR <= 16 ? 16 : 32);  // power of two >= CPR
  constexpr int RPB = 256 / TPR;
  const int tid = threadIdx.x;
  const int sub = tid % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / TPR;
  float acc = 0.f;
  if (row < a.rows && sub < CPR) {
    const uint4 uo = ldg16(a.o + row * D + sub * 8);
    const uint4 ud = ldg16(a.dO + row * D + sub * 8);
    const bf16x8 vo = as_bf16x8(uo), vd = as_bf16x8(ud);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)vo[e], (float)vd[e], acc);
  }
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < a.rows && sub == 0) a.delta[row] = acc;
}

// ---------------------------------------------------------------- dQ
// One workgroup = 4 wavefronts = 128 query rows of one query head; each
// wavefront owns 32 rows, one row per lane pair (transposed products, as in
// the forward).  Per key tile:
//   S^T  = K Q^T        (A = K from LDS, B = Q^T in registers)
//   dP^T = V dO^T       (A = V from LDS, B = dO^T in registers)
//   dS^T = P^T * (dP^T - delta)
//   dQ^T += K^T dS^T    (A = K^T by transposed LDS reads, B = dS^T)
template <int D, int BN, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_dq_kernel(BwdArgs a) {
  constexpr int BM = 128;
  constexpr int KP = D + 8;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NNB = BN / 32;
  constexpr int NKS = BN / 16;
  constexpr int CPR = D / 8;
  constexpr int CPT = BN * CPR / 256;
  static_assert(BN * CPR % 256 == 0, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][BN * KP];

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int G = a.G;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_group = a.nqt * G;
  const int bg = logical / per_group;
  const int rr = logical - bg * per_group;
  const int t = rr / G, hi = rr - (rr / G) * G;
  const int qt = CAUSAL ? (a.nqt - 1 - t) : t;
  const int b = bg / a.Hkv, hk = bg - (bg / a.Hkv) * a.Hkv;
  const int hq = hk * G + hi;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int64_t qh = (int64_t)(b * a.Hq + hq) * Lq;
  const bf16_t* qp = a.q + qh * D;
  const bf16_t* dop = a.dO + qh * D;
  const bf16_t* kp = a.k + ((int64_t)(b * a.Hkv + hk) * Lk) * D;
  const bf16_t* vp = a.v + ((int64_t)(b * a.Hkv + hk) * Lk) * D;

  const int q0 = qt * BM;
  const int qrow = q0 + 32 * w + lr;
  const bool row_ok = qrow < Lq;

  bf16x8 qf[NKD], dof[NKD];
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {
    if (row_ok) {
      qf[kd] = as_bf16x8(ldg16(qp + (int64_t)qrow * D + 16 * kd + 8 * lg));
      dof[kd] = as_bf16x8(ldg16(dop + (int64_t)qrow * D + 16 * kd + 8 * lg));
    } else {
      qf[kd] = as_bf16x8(make_uint4(0, 0, 0, 0));
      dof[kd] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }
  // rows past Lq: lse = +inf makes every P exactly 0
  const float lse2 = row_ok ? a.lse[qh + qrow] * kLog2e : INFINITY;
  const float dl = row_ok ? a.delta[qh + qrow] : 0.f;

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
        rk[c] = make_uint4(0, 0, 0, 0);
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
  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = zero16();
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

    f32x16 s[NNB], dp[NNB];
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      s[nb] = zero16();
      dp[nb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        s[nb] = mfma32(lds_read16(Ks + (nb * 32 + lr) * KP + 16 * kd + 8 * lg), qf[kd], s[nb]);
        dp[nb] = mfma32(lds_read16(Vs + (nb * 32 + lr) * KP + 16 * kd + 8 * lg), dof[kd], dp[nb]);
      }
    }

    const int kbase = j * BN;
    const bool need_mask = (kbase + BN > Lk) || (CAUSAL && kbase + BN - 1 > q0 + off);
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(fmaf(s[nb][i], c2, -lse2));
        if (need_mask) {
          const int key = kbase + nb * 32 + crow(i, lg);
          const bool vis = key < Lk && (!CAUSAL || key <= qrow + off);
          p = vis ? p : 0.f;
        }
        s[nb][i] = p * (dp[nb][i] - dl);  // dS^T (scale applied at the end)
      }

    bf16x8 dsf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dsf[ks] = pack8(s[ks / 2], ks % 2);

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        dq[db] = mfma32(lds_read_trA(Ks, troff, 16 * ks, 32 * db, KP), dsf[ks], dq[db]);

    if (j + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (row_ok) {
    bf16_t* out = a.dq + (qh + qrow) * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(dq[db][4 * q4 + e] * sc);
        *reinterpret_cast<bf16x4*>(out + 32 * db + 8 * q4 + 4 * lg) = v4;
      }
  }
}

// ---------------------------------------------------------------- dK / dV
// One workgroup = 4 wavefronts = 128 keys of one key/value head; each
// wavefront owns 32 keys, one key per lane pair.  K and V stay in registers;
// query tiles of BM rows of Q and dO (plus their LSE and delta) stream
// through LDS, for every query head of the group in turn.  Per query tile:
//   S  = Q K^T          (A = Q from LDS, B = K^T in registers)
//   dP = dO V^T         (A = dO from LDS, B = V^T in registers)
//   dS = P * (dP - delta)
//   dV^T += dO^T P      (A = dO^T by transposed LDS reads, B = P)
//   dK^T += Q^T dS      (A = Q^T by transposed LDS reads, B = dS)
template <int D, int BM, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_dkv_kernel(BwdArgs a) {
  constexpr int BN = 128;
  constexpr int QP = D + 8;
  constexpr int NKD = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NMB = BM / 32;
  constexpr int NKS = BM / 16;
  constexpr int CPR = D / 8;
  constexpr int CPT = BM * CPR / 256;
  static_assert(BM * CPR % 256 == 0, "tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][BM * QP];  // [buf][Q / dO]
  __shared__ __attribute__((aligned(16))) float stat[2][2][BM];       // [buf][lse*log2e / delta]

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lr = lane & 31, lg = lane >> 5;
  const int G = a.G;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.nkt;
  const int kt = logical - bh * a.nkt;  // key tile 0 sees the most queries: heaviest first
  const int b = bh / a.Hkv, hk = bh - (bh / a.Hkv) * a.Hkv;
  const int Lq = a.Lq, Lk = a.Lk, off = a.off;

  const int64_t kvh = (int64_t)(b * a.Hkv + hk) * Lk;
  const int k0 = kt * BN;
  const int krow = k0 + 32 * w + lr;
  const bool key_ok = krow < Lk;

  bf16x8 kf[NKD], vf[NKD];
#pragma unroll
  for (int kd = 0; kd < NKD; ++kd) {
    if (key_ok) {
      kf[kd] = as_bf16x8(ldg16(a.k + (kvh + krow) * D + 16 * kd + 8 * lg));
      vf[kd] = as_bf16x8(ldg16(a.v + (kvh + krow) * D + 16 * kd + 8 * lg));
    } else {
      kf[kd] = as_bf16x8(make_uint4(0, 0, 0, 0));
      vf[kd] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
  }

  // first query row that can see key k0: i >= k0 - off
  const int qfirst = CAUSAL ? max(0, k0 - off) : 0;
  const int qt_first = qfirst / BM;
  const int nqt = (Lq + BM - 1) / BM;
  const int nq = max(0, nqt - qt_first);
  const int niter = G * nq;

  uint4 rq[CPT], rd[CPT];
  float rstat = 0.f;
  auto load_tile = [&](int n) {
    const int hi = n / nq, qt = qt_first + (n - (n / nq) * nq);
    const int64_t qh = (int64_t)(b * a.Hq + hk * G + hi) * Lq;
    const int qbase = qt * BM;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      const int qr = qbase + row;
      if (qr < Lq) {
        rq[c] = ldg16(a.q + (qh + qr) * D + col);
        rd[c] = ldg16(a.dO + (qh + qr) * D + col);
      } else {
        rq[c] = make_uint4(0, 0, 0, 0);
        rd[c] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 2 * BM) {
      const int r = tid % BM;
      const int qr = qbase + r;
      if (tid < BM)
        rstat = qr < Lq ? a.lse[qh + qr] * kLog2e : INFINITY;  // +inf: P = 0 on padded rows
      else
        rstat = qr < Lq ? a.delta[qh + qr] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int chunk = tid + 256 * c;
      const int row = chunk / CPR, col = (chunk % CPR) * 8;
      *reinterpret_cast<uint4*>(&lds[buf][0][row * QP + col]) = rq[c];
      *reinterpret_cast<uint4*>(&lds[buf][1][row * QP + col]) = rd[c];
    }
    if (tid < 2 * BM) stat[buf][tid / BM][tid % BM] = rstat;
  };

  const float c2 = a.scale_log2;
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = zero16();
    dv[db] = zero16();
  }
  const int troff = tr_lane_offset(lane, QP);

  if (niter > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int n = 0; n < niter; ++n) {
    const int buf = n & 1;
    const int q0 = (qt_first + (n - (n / nq) * nq)) * BM;
    if (n + 1 < niter) load_tile(n + 1);
    const bf16_t* Qs = lds[buf][0];
    const bf16_t* dOs = lds[buf][1];

    f32x16 s[NMB], dp[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      s[mb] = zero16();
      dp[mb] = zero16();
#pragma unroll
      for (int kd = 0; kd < NKD; ++kd) {
        s[mb] = mfma32(lds_read16(Qs + (mb * 32 + lr) * QP + 16 * kd + 8 * lg), kf[kd], s[mb]);
        dp[mb] = mfma32(lds_read16(dOs + (mb * 32 + lr) * QP + 16 * kd + 8 * lg), vf[kd], dp[mb]);
      }
    }

    const bool need_mask = CAUSAL && (k0 + BN - 1 > q0 + off);
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int r0 = mb * 32 + 8 * i4 + 4 * lg;  // 4 consecutive query rows
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&stat[buf][0][r0]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&stat[buf][1][r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * i4 + e;
          float p = fast_exp2(fmaf(s[mb][i], c2, -l4[e]));
          if (need_mask) p = (krow <= q0 + r0 + e + off) ? p : 0.f;
          s[mb][i] = p;
          dp[mb][i] = p * (dp[mb][i] - d4[e]);
        }
      }

    bf16x8 pf[NKS], dsf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      pf[ks] = pack8(s[ks / 2], ks % 2);
      dsf[ks] = pack8(dp[ks / 2], ks % 2);
    }

#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        dv[db] = mfma32(lds_read_trA(dOs, troff, 16 * ks, 32 * db, QP), pf[ks], dv[db]);
        dk[db] = mfma32(lds_read_trA(Qs, troff, 16 * ks, 32 * db, QP), dsf[ks], dk[db]);
      }

    if (n + 1 < niter) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (key_ok) {
    bf16_t* dkp = a.dk + (kvh + krow) * D;
    bf16_t* dvp = a.dv + (kvh + krow) * D;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 k4, v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          k4[e] = (__bf16)(dk[db][4 * q4 + e] * sc);
          v4[e] = (__bf16)(dv[db][4 * q4 + e]);
        }
        *reinterpret_cast<bf16x4*>(dkp + 32 * db + 8 * q4 + 4 * lg) = k4;
        *reinterpret_cast<bf16x4*>(dvp + 32 * db + 8 * q4 + 4 * lg) = v4;
      }
  }
}

// ---------------------------------------------------------------- launchers

hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t stream) {
  auto go = [&](auto kern, int tpr) {
    const int rpb = 256 / tpr;
    const int64_t nblocks = (a.rows + rpb - 1) / rpb;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(256), 0, stream, a);
  };
  switch (D) {
    case 64: go(fa_delta_kernel<64>, 8); break;
    case 96: go(fa_delta_kernel<96>, 16); break;
    case 128: go(fa_delta_kernel<128>, 16); break;
    case 256: go(fa_delta_kernel<256>, 32); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, int BN_Q, int BM_KV>
static hipError_t launch_bwd_d(const BwdArgs& a, bool causal, int which, hipStream_t stream) {
  const int ndq = (which & 1) ? a.B * a.Hq * a.nqt : 0;
  const int ndkv = (which & 2) ? a.B * a.Hkv * a.nkt : 0;
  if (causal) {
    if (ndq > 0) hipLaunchKernelGGL((fa_dq_kernel<D, BN_Q, true>), dim3(ndq), dim3(256), 0, stream, a);
    if (ndkv > 0) hipLaunchKernelGGL((fa_dkv_kernel<D, BM_KV, true>), dim3(ndkv), dim3(256), 0, stream, a);
  } else {
    if (ndq > 0) hipLaunchKernelGGL((fa_dq_kernel<D, BN_Q, false>), dim3(ndq), dim3(256), 0, stream, a);
    if (ndkv > 0) hipLaunchKernelGGL((fa_dkv_kernel<D, BM_KV, false>), dim3(ndkv), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int which, hipStream_t stream) {
  switch (D) {
    case 64: return launch_bwd_d<64, 64, 64>(a, causal, which, stream);
    case 96: return launch_bwd_d<96, 64, 64>(a, causal, which, stream);
    case 128: return launch_bwd_d<128, 64, 64>(a, causal, which, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cgqa
