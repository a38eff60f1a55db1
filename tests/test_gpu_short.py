"""GPU parity of the short-query calls (fa_fwd_short, fa_bwd_short; Lq <= 8)
against the fp64 oracle: every head dimension, causal and not, one to eight
query rows against 1 to 4100 keys (one chunk or many, ragged last chunks),
GQA groups of 1, 4 and 8; fp16 and strided K/V cache slices whose rows past
Lk hold NaN; agreement with the long-query calls; the workspace contract;
and decode at 32768 keys, checked on every output.
"""
import math

import numpy as np
import pytest
import torch

from fa_synth import normal_bits, ramp_bits
from parity_util import check, oracle_full, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def make_bits(B, Hq, Hkv, Lq, Lk, D, seed, dtype="bf16"):
    return {
        "q": normal_bits((B, Hq, Lq, D), seed + 0, 1.0, dtype),
        "k": normal_bits((B, Hkv, Lk, D), seed + 1, 1.0, dtype),
        "v": normal_bits((B, Hkv, Lk, D), seed + 2, 1.0, dtype),
        "do": normal_bits((B, Hq, Lq, D), seed + 3, 1.0, dtype),
    }


def run_short(g, scale, causal, workspace=None):
    import causal_gqa_flashattention_amd as fa
    o, lse = fa.fa_fwd_short(g["q"], g["k"], g["v"], scale=scale, causal=causal, workspace=workspace)
    delta = fa.fa_bwd_delta_ex(o, g["do"])
    dq, dk, dv = fa.fa_bwd_short(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=scale, causal=causal,
                                 workspace=workspace)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


def short_case(B, Hq, Hkv, Lq, Lk, D, causal, seed, dtype="bf16", ramp=None,
               names=("o", "lse", "dq", "dk", "dv")):
    label = f"short {dtype} B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal}"
    if ramp is not None:
        label += f" ramp={ramp}"
    print(f"[case] {label}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    # ramp: scores rising by that much along each row (ramp_bits)
    bits = (make_bits(B, Hq, Hkv, Lq, Lk, D, seed, dtype) if ramp is None
            else ramp_bits(B, Hq, Hkv, Lq, Lk, D, seed, rise=ramp, scale=scale, dtype=dtype))
    g = {n: to_gpu(b, dtype) for n, b in bits.items()}
    out = run_short(g, scale, causal)
    ref = oracle_full(bits, scale, causal, dtype=dtype)
    # Lk = 1: every row sees one key, P = 1 and dS = dP - delta is exactly 0;
    # the GPU's two fp32 dot products dO.V and dO.O differ by rounding only
    atol = {"dq": 1e-4, "dk": 1e-4} if Lk == 1 else {}
    for n in names:
        check(n, to_f64(out[n]), ref[n], label, atol=atol.get(n, 0.0))
    return g, out


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("Lq,Lk", [(1, 1), (1, 777), (3, 64), (8, 1000), (5, 4100)])
@pytest.mark.parametrize("causal", [True, False])
def test_short_parity(D, Lq, Lk, causal):
    short_case(1, 8, 2, Lq, Lk, D, causal, seed=10000 + D + 10 * Lq + Lk)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_short_rising_scores(D, causal):
    # scores rising by 120 along 4100 keys: a row's running max passes the
    # slack every few key tiles, in the chunk kernels and in the merge
    # (chunks far apart along the row differ by many orders of magnitude)
    # (dQ is not compared on these inputs: test_gpu_parity.RAMP_CHECKED)
    short_case(1, 8, 2, 5, 4100, D, causal, seed=10300 + D + int(causal), ramp=120.0,
               names=("o", "lse", "dk", "dv"))


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 1), (32, 4)])
def test_short_groups_and_batches(Hq, Hkv):
    short_case(2, Hq, Hkv, 2, 1500, 128, True, seed=10100 + Hq)


def test_short_f16_and_cache_slices():
    """fp16 K/V as the first Lk rows of a longer cache with NaN behind them."""
    import causal_gqa_flashattention_amd as fa
    B, Hq, Hkv, Lq, Lk, D, cap = 1, 8, 2, 4, 3000, 128, 4096
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, 10200, "f16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = {n: to_gpu(bits[n], "f16") for n in ("q", "do")}
    for n in ("k", "v"):
        cache = torch.full((B, Hkv, cap, D), float("nan"), dtype=torch.float16, device="cuda")
        cache[:, :, :Lk] = to_gpu(bits[n], "f16")
        g[n] = cache[:, :, :Lk]
    out = run_short(g, scale, True)
    ref = oracle_full(bits, scale, True, dtype="f16")
    for n in ("o", "lse", "dq", "dk", "dv"):
        check(n, to_f64(out[n]), ref[n], "short f16 cache slice")
    assert out["o"].dtype == torch.float16


@pytest.mark.parametrize("D", [64, 128, 256])
def test_short_agrees_with_long_path(D):
    import causal_gqa_flashattention_amd as fa
    bits = make_bits(1, 16, 4, 8, 2500, D, 10300 + D)
    g = {n: to_gpu(b) for n, b in bits.items()}
    sc = float(np.float32(1.0 / math.sqrt(D)))
    s = run_short(g, sc, True)
    o, lse = fa.fa_fwd_ex(g["q"], g["k"], g["v"], scale=sc, causal=True)
    delta = fa.fa_bwd_delta_ex(o, g["do"])
    dq, dk, dv = fa.fa_bwd_ex(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=sc, causal=True)
    torch.cuda.synchronize()
    assert (s["lse"] - lse).abs().max().item() < 1e-4
    for n, t in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        err = (s[n].float() - t.float()).abs().max().item()
        assert err <= 1e-2 * t.float().abs().max().item(), (n, err)
    # from the same lse and delta, the short dK/dV (rows resident, keys
    # streamed) differs from the key-block kernel only in summation order
    _, dk2, dv2 = fa.fa_bwd_short(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=sc, causal=True,
                                  grads="dkv")
    torch.cuda.synchronize()
    for a_, b_ in ((dk2, dk), (dv2, dv)):
        assert (a_.float() - b_.float()).abs().max().item() <= 4e-3 * b_.float().abs().max().item()


def test_short_workspace_contract():
    import causal_gqa_flashattention_amd as fa
    B, Hq, Hkv, Lq, Lk, D = 1, 8, 2, 3, 2000, 128
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, 10400)
    g = {n: to_gpu(b) for n, b in bits.items()}
    n = fa.fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage on entry is fine
    a = run_short(g, 0.1, True, workspace=ws)
    b = run_short(g, 0.1, True, workspace=ws)  # reused: same bits
    for k in a:
        assert torch.equal(a[k], b[k]), k
    with pytest.raises(fa.FAError):
        fa.fa_fwd_short(g["q"], g["k"], g["v"], scale=0.1, causal=True, workspace=ws[: n - 16])
    with pytest.raises(fa.FAError):  # Lq above the limit
        q9 = torch.zeros((1, 8, 9, D), dtype=torch.bfloat16, device="cuda")
        fa.fa_fwd_short(q9, g["k"], g["v"], scale=0.1, causal=True)


@pytest.mark.slow
@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (32, 8, 256)])
def test_decode_32k_every_output(Hq, Hkv, D):
    """One query row per head against 32768 keys (the decode shape of the
    head-dim-256 page's measurements), every output against the oracle."""
    short_case(1, Hq, Hkv, 1, 32768, D, True, seed=10500 + D)


@pytest.mark.parametrize("Lq,causal", [(1, True), (4, False), (4, True)])
def test_short_sequence_major_queries(Lq, causal):
    """q, dO (and the outputs) in [B, L, H, D] buffers: with one query row the
    dK/dV pass takes a group's heads as rows at the head stride; with more
    rows that stride pattern is not a single stride and the per-head pass
    runs.  Both against the oracle."""
    B, Hq, Hkv, Lk, D = 2, 8, 2, 1200, 128
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, 10600 + Lq)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = {n: to_gpu(b) for n, b in bits.items()}
    for n in ("q", "do"):
        g[n] = g[n].transpose(1, 2).contiguous().transpose(1, 2)
    out = run_short(g, scale, causal)
    ref = oracle_full(bits, scale, causal)
    for n in ("o", "lse", "dq", "dk", "dv"):
        check(n, to_f64(out[n]), ref[n], f"short bshd Lq{Lq} causal={causal}")


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("Hq,Lq,causal", [(16, 3, True), (8, 8, False), (8, 8, True)])
def test_short_two_row_blocks(D, Hq, Lq, causal):
    """More than 32 packed rows per group (48 and 64): two 32-row blocks in
    the streaming dK/dV (at D = 256 the key-block kernel takes them)."""
    short_case(1, Hq, 1, Lq, 700, D, causal, seed=10700 + D + Hq + Lq)
