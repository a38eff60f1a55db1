"""GPU parity of the general calls (fa_fwd_ex, fa_bwd_delta_ex, fa_bwd_ex):

* IEEE half inputs against the fp64 oracle on the same binary16 bits, at
  every head dimension, causal and not, ragged, GQA, with and without a
  block mask;
* strided views give bitwise the results of the same values stored
  contiguously: [B, L, H, D] buffers (inputs and outputs), K/V as the first
  Lk rows of a longer cache whose stale rows hold NaN (never read), padded
  rows whose pads stay untouched, and a key/value head broadcast by a
  zero head stride;
* the plain bf16 calls and fa_*_ex on the same contiguous tensors agree
  bitwise; the Python layer refuses a non-contiguous head dimension.
"""
import math

import numpy as np
import pytest
import torch

from fa_synth import normal_bits, random_block_mask
from parity_util import check, check_masked, oracle_full, to_f64, to_gpu

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "f16": torch.float16}


def make_bits(B, Hq, Hkv, Lq, Lk, D, seed, dtype):
    return {
        "q": normal_bits((B, Hq, Lq, D), seed + 0, 1.0, dtype),
        "k": normal_bits((B, Hkv, Lk, D), seed + 1, 1.0, dtype),
        "v": normal_bits((B, Hkv, Lk, D), seed + 2, 1.0, dtype),
        "do": normal_bits((B, Hq, Lq, D), seed + 3, 1.0, dtype),
    }


def run_ex(q, k, v, do, scale, causal, block_mask=None, outs=None):
    """fa_fwd_ex, fa_bwd_delta_ex, fa_bwd_ex; `outs` may give the o, dq, dk, dv views."""
    import causal_gqa_flashattention_amd as fa
    outs = outs or {}
    o, lse = fa.fa_fwd_ex(q, k, v, outs.get("o"), scale=scale, causal=causal, block_mask=block_mask)
    delta = fa.fa_bwd_delta_ex(o, do)
    dq, dk, dv = fa.fa_bwd_ex(q, k, v, lse, delta, do, outs.get("dq"), outs.get("dk"), outs.get("dv"),
                              scale=scale, causal=causal, block_mask=block_mask)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


# ------------------------------------------------------------ IEEE half

@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal,Lq,Lk", [(True, 300, 300), (True, 200, 333), (False, 257, 190)])
def test_f16_parity(D, causal, Lq, Lk):
    label = f"f16 D{D} causal={causal} Lq{Lq} Lk{Lk}"
    print(f"[case] {label}", flush=True)
    bits = make_bits(1, 4, 2, Lq, Lk, D, 9300 + D + Lq, "f16")
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = {n: to_gpu(b, "f16") for n, b in bits.items()}
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, causal)
    assert out["o"].dtype == torch.float16 and out["dq"].dtype == torch.float16
    ref = oracle_full(bits, scale, causal, dtype="f16")
    for n in ("o", "lse", "dq", "dk", "dv"):
        check(n, to_f64(out[n]), ref[n], label)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_f16_rising_scores(D):
    # the accumulator rescale in half precision: scores rising by 48 along
    # each row (fa_synth.ramp_bits; dQ is not compared on these inputs, see
    # test_gpu_parity.RAMP_CHECKED)
    from fa_synth import ramp_bits
    L = 600
    label = f"f16 ramp D{D} L{L} causal"
    print(f"[case] {label}", flush=True)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    bits = ramp_bits(1, 4, 2, L, L, D, 9500 + D, rise=48.0, scale=scale, dtype="f16")
    g = {n: to_gpu(b, "f16") for n, b in bits.items()}
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, True)
    ref = oracle_full(bits, scale, True, dtype="f16")
    for n in ("o", "lse", "dk", "dv"):
        check(n, to_f64(out[n]), ref[n], label)


def test_f16_gqa_batches_and_mask():
    import oracle
    B, Hq, Hkv, L, D = 2, 8, 2, 520, 128
    label = "f16 masked B2 Hq8 Hkv2 L520 D128"
    print(f"[case] {label}", flush=True)
    bits = make_bits(B, Hq, Hkv, L, L, D, 9400, "f16")
    mask = random_block_mask(L, L, 0.6, seed=9401)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = {n: to_gpu(b, "f16") for n, b in bits.items()}
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, True,
                 block_mask=torch.from_numpy(mask).cuda())
    ref = oracle_full(bits, scale, True, block_mask=mask, dtype="f16")
    vis = oracle.visible_mask(L, L, True, block_mask=mask)
    for n in ("o", "lse", "dq", "dk", "dv"):
        check_masked(n, to_f64(out[n]), ref[n], label, ~vis.any(axis=0) if n in ("dk", "dv") else ~vis.any(axis=1))


def test_f16_smaller_error_than_bf16():
    """The same real inputs in binary16 and bfloat16: half keeps 3 more
    fraction bits, so every output is at least as close to its oracle."""
    D, L = 128, 384
    x = {n: np.random.default_rng(9500 + i).standard_normal(s, dtype=np.float32)
         for i, (n, s) in enumerate((("q", (1, 4, L, D)), ("k", (1, 2, L, D)), ("v", (1, 2, L, D)),
                                     ("do", (1, 4, L, D))))}
    from fa_synth import bf16_bits_from_f32, f16_bits_from_f32
    errs = {}
    for dt, rnd in (("bf16", bf16_bits_from_f32), ("f16", f16_bits_from_f32)):
        bits = {n: rnd(a) for n, a in x.items()}
        g = {n: to_gpu(b, dt) for n, b in bits.items()}
        out = run_ex(g["q"], g["k"], g["v"], g["do"], 1 / math.sqrt(D), True)
        ref = oracle_full(bits, 1 / math.sqrt(D), True, dtype=dt)
        errs[dt] = {n: float(np.abs(to_f64(out[n]) - ref[n]).max() / np.abs(ref[n]).max())
                    for n in ("o", "dq", "dk", "dv")}
    print(f"[f16 vs bf16] {errs}", flush=True)
    for n in ("o", "dq", "dk", "dv"):
        assert errs["f16"][n] < errs["bf16"][n], n


# ---------------------------------------------------------- strided views

def contiguous_reference(bits, dtype, scale, causal, block_mask=None):
    g = {n: to_gpu(b, dtype) for n, b in bits.items()}
    return run_ex(g["q"], g["k"], g["v"], g["do"], scale, causal, block_mask)


def assert_same(a, b, names=("o", "lse", "delta", "dq", "dk", "dv")):
    for n in names:
        assert torch.equal(a[n].contiguous(), b[n].contiguous()), f"{n} differs"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 96, 128, 256])
def test_sequence_major_buffers(dtype, D):
    """Every tensor a [B, L, H, D] buffer seen as [B, H, L, D]; outputs too."""
    B, Hq, Hkv, Lq, Lk = 2, 4, 2, 200, 260
    print(f"[case] bshd {dtype} D{D}", flush=True)
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, 9600 + D, dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    ref = contiguous_reference(bits, dtype, scale, True)
    g = {n: to_gpu(b, dtype).transpose(1, 2).contiguous().transpose(1, 2) for n, b in bits.items()}
    assert g["q"].stride(2) == Hq * D and g["q"].stride(1) == D
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, True)
    assert out["o"].stride() == g["q"].stride() and out["dk"].stride() == g["k"].stride()
    assert_same(out, ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_kv_cache_slice_never_reads_stale_rows(dtype, D):
    """K and V are the first Lk rows of a [B, Hkv, capacity, D] cache whose
    rows past Lk hold NaN: a single one read would poison the outputs."""
    B, Hq, Hkv, Lq, Lk, cap = 1, 4, 2, 77, 333, 512
    print(f"[case] cache slice {dtype} D{D}", flush=True)
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, 9700 + D, dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    for causal in (True, False):
        ref = contiguous_reference(bits, dtype, scale, causal)
        g = {n: to_gpu(bits[n], dtype) for n in ("q", "do")}
        for n in ("k", "v"):
            cache = torch.full((B, Hkv, cap, D), float("nan"), dtype=TDT[dtype], device="cuda")
            cache[:, :, :Lk] = to_gpu(bits[n], dtype)
            g[n] = cache[:, :, :Lk]
        dk_buf = torch.full((B, Hkv, cap, D), 7.0, dtype=TDT[dtype], device="cuda")
        outs = {"dk": dk_buf[:, :, :Lk], "dv": torch.empty_like(g["v"])}
        out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, causal, outs=outs)
        assert_same(out, ref)
        assert torch.all(dk_buf[:, :, Lk:] == 7.0), "rows past Lk of a strided output were written"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_padded_rows_and_guarded_outputs(dtype):
    """Rows padded to D + 24 elements (inputs and outputs); the pads of the
    outputs keep their sentinel."""
    B, Hq, Hkv, L, D, pad = 1, 4, 1, 300, 128, 24
    bits = make_bits(B, Hq, Hkv, L, L, D, 9800, dtype)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    ref = contiguous_reference(bits, dtype, scale, True)

    def padded(t, fill=0.0):
        buf = torch.full(t.shape[:3] + (t.shape[3] + pad,), fill, dtype=t.dtype, device="cuda")
        buf[..., :t.shape[3]] = t
        return buf

    g = {n: padded(to_gpu(b, dtype))[..., :D] for n, b in bits.items()}
    obufs = {n: torch.full((B, Hq if n in ("o", "dq") else Hkv, L, D + pad), -3.0, dtype=TDT[dtype],
                           device="cuda") for n in ("o", "dq", "dk", "dv")}
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, True,
                 outs={n: b[..., :D] for n, b in obufs.items()})
    assert_same(out, ref)
    for n, b in obufs.items():
        assert torch.all(b[..., D:] == -3.0), f"{n}: pad written"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_broadcast_kv_head(dtype):
    """Hkv = 4 key/value heads that are one head broadcast with head stride
    0 give the results of the four copies stored out."""
    B, Hq, Hkv, L, D = 1, 8, 4, 260, 64
    one = make_bits(B, 1, 1, L, L, D, 9900, dtype)
    bits = make_bits(B, Hq, Hkv, L, L, D, 9910, dtype)
    for n in ("k", "v"):
        bits[n] = np.repeat(one[n], Hkv, axis=1)
    scale = 0.125
    ref = contiguous_reference(bits, dtype, scale, True)
    g = {n: to_gpu(bits[n], dtype) for n in ("q", "do")}
    for n in ("k", "v"):
        g[n] = to_gpu(one[n], dtype).expand(B, Hkv, L, D)
        assert g[n].stride(1) == 0
    out = run_ex(g["q"], g["k"], g["v"], g["do"], scale, True)
    assert_same(out, ref)


def test_plain_and_general_calls_agree():
    import causal_gqa_flashattention_amd as fa
    B, Hq, Hkv, L, D = 1, 4, 2, 300, 96
    bits = make_bits(B, Hq, Hkv, L, L, D, 9950, "bf16")
    g = {n: to_gpu(b) for n, b in bits.items()}
    sc = float(np.float32(1.0 / math.sqrt(D)))
    a = run_ex(g["q"], g["k"], g["v"], g["do"], sc, True)
    o, lse = fa.fa_fwd(g["q"], g["k"], g["v"], scale=sc, causal=True)
    delta = fa.fa_bwd_delta(o, g["do"])
    dq, dk, dv = fa.fa_bwd(g["q"], g["k"], g["v"], o, lse, delta, g["do"], scale=sc, causal=True)
    torch.cuda.synchronize()
    assert_same(a, {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv})
    # one gradient at a time
    dq2, dk2, dv2 = fa.fa_bwd_ex(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=sc, causal=True, grads="dq")
    torch.cuda.synchronize()
    assert dk2 is None and dv2 is None and torch.equal(dq2, dq)


def test_python_layer_checks():
    import causal_gqa_flashattention_amd as fa
    q = torch.zeros((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):   # head dimension not contiguous
        fa.fa_fwd_ex(q.transpose(2, 3), k, k, scale=0.1, causal=True)
    with pytest.raises(TypeError):    # mixed element types
        fa.fa_fwd_ex(q, k.half(), k, scale=0.1, causal=True)
    with pytest.raises(fa.FAError):   # an output that overlaps itself
        o = torch.empty((1, 2, 64, 64), dtype=torch.bfloat16, device="cuda").as_strided((1, 2, 64, 64),
                                                                                         (8192, 0, 64, 1))
        fa.fa_fwd_ex(q, k, k, o, scale=0.1, causal=True)
