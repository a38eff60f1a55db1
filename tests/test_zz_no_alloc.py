"""fa_fwd_short_noalloc (the short-query forward on the library's static
per-device scratch, for callers that cannot allocate) against fa_fwd_short
with a caller workspace: two calls in a row on one GPU, the second smaller and
on another kernel variant, each bitwise equal to the workspace call (the same
kernels on the same inputs), and the second also checked against the fp64
oracle."""
import math

import numpy as np
import pytest
import torch

from fa_synth import normal_bits
from parity_util import check, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, Lq, Lk, D, causal, seed):
    import causal_gqa_flashattention_amd as fa
    label = f"noalloc B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal}"
    need = fa.fa_short_workspace_bytes(B, Hq, Hkv, Lq, Lk, D)
    print(f"[case] {label}: {need} scratch bytes", flush=True)
    assert 0 < need <= fa.NOALLOC_SCRATCH_BYTES
    bits = {
        "q": normal_bits((B, Hq, Lq, D), seed + 0, 1.0, "bf16"),
        "k": normal_bits((B, Hkv, Lk, D), seed + 1, 1.0, "bf16"),
        "v": normal_bits((B, Hkv, Lk, D), seed + 2, 1.0, "bf16"),
    }
    g = {n: to_gpu(b) for n, b in bits.items()}
    scale = float(np.float32(1.0 / math.sqrt(D)))
    o_ws, lse_ws = fa.fa_fwd_short(g["q"], g["k"], g["v"], scale=scale, causal=causal)
    o = torch.full_like(g["q"], float("nan"))
    lse = torch.full((B, Hq, Lq), float("nan"), dtype=torch.float32, device="cuda")
    fa.fa_fwd_short_noalloc(g["q"], g["k"], g["v"], o, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ws.view(torch.int16)), label
    assert torch.equal(lse.view(torch.int32), lse_ws.view(torch.int32)), label
    return bits, scale, o, lse, label


def test_noalloc_matches_workspace_call_twice():
    import oracle
    # first call: 4 query rows x 4 heads per group, 20000 keys, D = 128
    _case(1, 32, 8, 4, 20000, 128, True, seed=31000)
    # second call, smaller, right after (the scratch keeps the first call's
    # partials): one query row, D = 256 (the four-way split kernels)
    bits, scale, o, lse, label = _case(1, 8, 2, 1, 3000, 256, False, seed=32000)
    G = 4
    for h in range(8):
        r_o, r_lse = oracle.head_forward(oracle.bf16_bits_to_f64(bits["q"][0, h]),
                                         oracle.bf16_bits_to_f64(bits["k"][0, h // G]),
                                         oracle.bf16_bits_to_f64(bits["v"][0, h // G]), scale, False)
        check("o", to_f64(o[0, h]), r_o, f"{label} head {h}")
        check("lse", to_f64(lse[0, h]), r_lse, f"{label} head {h}")
