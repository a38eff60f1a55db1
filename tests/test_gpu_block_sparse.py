"""GPU parity of the block-sparse calls (fa_fwd_block_sparse,
fa_bwd_block_sparse, fa_bwd_dq_block_sparse, fa_bwd_dkv_block_sparse)
against the fp64 oracle under the same uint8 64 x 64 block mask:

* an all-ones mask gives bitwise the results of the plain calls;
* random masks over every head dimension, causal and not, ragged lengths,
  bottom-right rectangles and GQA groups;
* rows that see no key (a zero query-block row, or a causal diagonal cut
  away) give O = 0, LSE = -inf and dQ = 0 exactly; keys no row sees get
  dK = dV = 0 exactly; an all-zero mask zeroes everything;
* local-attention bands with a sink block;
* the split dQ and dK/dV calls equal the fused backward bitwise;
* the 8192-token training shape under a 1024-key sliding window, on
  whole GQA groups of sampled rows and keys.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_synth import (WORKLOADS, block_mask_of, make_inputs, normal_bf16_bits, ramp_bits, random_block_mask,
                      window_block_mask)
from parity_util import check_masked, oracle_full, run_library, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def make_bits(B, Hq, Hkv, Lq, Lk, D, seed):
    return {
        "q": normal_bf16_bits((B, Hq, Lq, D), seed + 0),
        "k": normal_bf16_bits((B, Hkv, Lk, D), seed + 1),
        "v": normal_bf16_bits((B, Hkv, Lk, D), seed + 2),
        "do": normal_bf16_bits((B, Hq, Lq, D), seed + 3),
    }


def mask_gpu(m):
    return torch.from_numpy(np.ascontiguousarray(m, dtype=np.uint8)).cuda()


def run_masked_case(B, Hq, Hkv, Lq, Lk, D, causal, mask, seed, label="", ramp=None,
                    names=("o", "lse", "dq", "dk", "dv")):
    label = f"{label} B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal} seed={seed}"
    print(f"[case] {label} kept={int(mask.sum())}/{mask.size}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    # ramp: scores rising by that much along each row (ramp_bits)
    bits = (make_bits(B, Hq, Hkv, Lq, Lk, D, seed) if ramp is None
            else ramp_bits(B, Hq, Hkv, Lq, Lk, D, seed, rise=ramp, scale=scale))
    g = {n: to_gpu(b) for n, b in bits.items()}
    out = run_library(g["q"], g["k"], g["v"], g["do"], scale, causal, block_mask=mask_gpu(mask))
    ref = oracle_full(bits, scale, causal, block_mask=mask)
    vis = oracle.visible_mask(Lq, Lk, causal, block_mask=mask)
    rows_empty, keys_empty = ~vis.any(axis=1), ~vis.any(axis=0)
    for n in names:
        check_masked(n, to_f64(out[n]), ref[n], label, keys_empty if n in ("dk", "dv") else rows_empty)
    return out, ref


# ------------------------------------------------------- all ones == dense

@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal,Lq,Lk", [(True, 300, 300), (True, 200, 333), (False, 257, 190)])
def test_all_ones_mask_is_bitwise_dense(D, causal, Lq, Lk):
    import causal_gqa_flashattention_amd as fa
    print(f"[case] all-ones D{D} causal={causal} Lq{Lq} Lk{Lk}", flush=True)
    bits = make_bits(1, 4, 2, Lq, Lk, D, 8100 + D)
    g = {n: to_gpu(b) for n, b in bits.items()}
    scale = float(np.float32(1.0 / math.sqrt(D)))
    ones = mask_gpu(np.ones((-(-Lq // 64), -(-Lk // 64)), np.uint8))
    a = run_library(g["q"], g["k"], g["v"], g["do"], scale, causal)
    b = run_library(g["q"], g["k"], g["v"], g["do"], scale, causal, block_mask=ones)
    for n in ("o", "lse", "dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), f"{n} differs from the plain call"
    # a bool mask is the same bytes
    o2, _ = fa.fa_fwd_block_sparse(g["q"], g["k"], g["v"], ones.bool(), scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o2, a["o"])


# ------------------------------------------------------------ random masks

@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal,Lq,Lk", [(True, 320, 320), (True, 250, 390), (False, 333, 200)])
def test_random_mask(D, causal, Lq, Lk):
    mask = random_block_mask(Lq, Lk, 0.5, seed=8200 + D + Lq)
    run_masked_case(1, 4, 2, Lq, Lk, D, causal, mask, seed=8300 + D + Lk, label="random")


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_random_mask_rising_scores(D, causal):
    # the masked kernels' accumulator rescale, run several times per row
    # (scores rising by 48 along each row; see test_gpu_parity)
    mask = random_block_mask(600, 600, 0.7, seed=8400 + D)
    # (dQ is not compared on these inputs: test_gpu_parity.RAMP_CHECKED)
    run_masked_case(1, 4, 2, 600, 600, D, causal, mask, seed=8500 + D + int(causal), label="ramp",
                    ramp=48.0, names=("o", "lse", "dk", "dv"))


@pytest.mark.parametrize("density", [0.2, 0.8])
def test_random_mask_gqa_batches(density):
    mask = random_block_mask(700, 700, density, seed=8400 + int(10 * density))
    run_masked_case(2, 8, 2, 700, 700, 128, True, mask, seed=8500, label=f"random{density}")


# --------------------------------------------- empty rows, keys and masks

@pytest.mark.parametrize("D", [64, 128, 256])
def test_empty_rows_and_keys(D):
    Lq = Lk = 400
    mask = random_block_mask(Lq, Lk, 0.7, seed=8600 + D)
    mask[2, :] = 0           # query rows 128..191 see nothing
    mask[:, 4] = 0           # keys 256..319 are seen by nobody
    mask[5, 5] = 0           # causal: rows 320..383 only meet diagonal blocks
    mask[5, :5] = 0          # beyond it, so they see nothing either
    out, ref = run_masked_case(1, 4, 1, Lq, Lk, D, True, mask, seed=8700 + D, label="empty")
    lse = to_f64(out["lse"])
    assert np.all(np.isneginf(lse[:, :, 128:192])) and np.all(np.isneginf(lse[:, :, 320:384]))
    for n in ("o", "dq"):
        assert not to_f64(out[n])[:, :, 128:192].any() and not to_f64(out[n])[:, :, 320:384].any()
    for n in ("dk", "dv"):
        assert not to_f64(out[n])[:, :, 256:320].any()


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_all_zero_mask(D, causal):
    Lq, Lk = 190, 260
    bits = make_bits(1, 2, 1, Lq, Lk, D, 8800 + D)
    g = {n: to_gpu(b) for n, b in bits.items()}
    zeros = mask_gpu(np.zeros((3, 5), np.uint8))
    out = run_library(g["q"], g["k"], g["v"], g["do"], 0.1, causal, block_mask=zeros)
    assert torch.isneginf(out["lse"]).all()
    for n in ("o", "delta", "dq", "dk", "dv"):
        assert not out[n].float().any(), n


# ----------------------------------------------------- local-attention bands

@pytest.mark.parametrize("D,window,sink", [(128, 192, 1), (64, 128, 0), (96, 256, 2), (256, 130, 1)])
def test_window_band(D, window, sink):
    L = 1000
    mask = window_block_mask(L, L, window, sink)
    run_masked_case(1, 4, 1, L, L, D, True, mask, seed=8900 + D, label=f"window{window}+{sink}")


def test_window_band_rectangle():
    mask = window_block_mask(300, 1000, 256, 1)
    run_masked_case(1, 4, 2, 300, 1000, 128, True, mask, seed=9000, label="window-rect")


# ------------------------------------------------- split backward calls

@pytest.mark.parametrize("D", [64, 96, 128, 256])
def test_split_calls_equal_fused(D):
    import causal_gqa_flashattention_amd as fa
    Lq = Lk = 333
    mask = mask_gpu(random_block_mask(Lq, Lk, 0.6, seed=9100 + D))
    bits = make_bits(1, 4, 2, Lq, Lk, D, 9200 + D)
    g = {n: to_gpu(b) for n, b in bits.items()}
    sc = float(np.float32(1.0 / math.sqrt(D)))
    out = run_library(g["q"], g["k"], g["v"], g["do"], sc, True, block_mask=mask)
    dq = fa.fa_bwd_dq_block_sparse(g["q"], g["k"], g["v"], out["lse"], out["delta"], g["do"], mask,
                                   scale=sc, causal=True)
    dk, dv = fa.fa_bwd_dkv_block_sparse(g["q"], g["k"], g["v"], out["lse"], out["delta"], g["do"], mask,
                                        scale=sc, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, out["dq"]) and torch.equal(dk, out["dk"]) and torch.equal(dv, out["dv"])


def test_mask_shape_is_checked():
    import causal_gqa_flashattention_amd as fa
    q = torch.zeros((1, 2, 128, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fa.fa_fwd_block_sparse(q, k, k, mask_gpu(np.ones((2, 3), np.uint8)), scale=0.1, causal=True)
    with pytest.raises(TypeError):
        fa.fa_fwd_block_sparse(q, k, k, torch.ones((2, 2), dtype=torch.int32, device="cuda"),
                               scale=0.1, causal=True)


# ------------------------------------------- full-size training shape

@pytest.mark.slow
def test_train8k_window_sampled():
    """8192 tokens, 32/8 heads, D=128, causal, 1024-key sliding window: O,
    LSE, dQ of sampled rows of one whole GQA group, and the dK, dV of two key
    ranges (mid-sequence and the last 256 keys) from exactly the rows that
    see them."""
    w = WORKLOADS["train8k_window"]
    mask = block_mask_of(w)
    print(f"[workload] {w.name} kept blocks {int(mask.sum())}/{mask.size}", flush=True)
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    out = run_library(g["q"], g["k"], g["v"], g["do"], w.softmax_scale, True, block_mask=mask_gpu(mask))
    G = w.Hq // w.Hkv
    kvh = 6
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    rng = np.random.default_rng(w.seed)
    rows = np.union1d(rng.choice(w.Lq, 192, replace=False),
                      [0, 63, 64, 1023, 1024, 1087, 1088, 4095, 4096, w.Lq - 1])
    key_sets = [np.arange(4000, 4160), np.arange(w.Lk - 256, w.Lk)]
    for keys in key_sets:
        seen_by = np.nonzero(oracle.visible_mask(w.Lq, w.Lk, True, block_mask=mask)[:, keys].any(axis=1))[0]
        dk = np.zeros((keys.size, w.D))
        dv = np.zeros((keys.size, w.D))
        for h in range(kvh * G, (kvh + 1) * G):
            q = oracle.bf16_bits_to_f64(bits["q"][0, h])
            do = oracle.bf16_bits_to_f64(bits["do"][0, h])
            r = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=seen_by, key_rows=keys,
                                     block_mask=mask)
            dk += r["dk"]
            dv += r["dv"]
        check_masked("dk", to_f64(out["dk"][0, kvh, keys]), dk, f"{w.name} keys {keys[0]}..{keys[-1]}")
        check_masked("dv", to_f64(out["dv"][0, kvh, keys]), dv, f"{w.name} keys {keys[0]}..{keys[-1]}")
    vis = oracle.visible_mask(w.Lq, w.Lk, True, rows=rows, block_mask=mask)
    for h in range(kvh * G, (kvh + 1) * G):
        q = oracle.bf16_bits_to_f64(bits["q"][0, h])
        do = oracle.bf16_bits_to_f64(bits["do"][0, h])
        r = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=rows, block_mask=mask)
        for n in ("o", "lse", "dq"):
            check_masked(n, to_f64(out[n][0, h, rows]), r[n], f"{w.name} head {h}", ~vis.any(axis=1))
