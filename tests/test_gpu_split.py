"""GPU parity of fa_bwd_ws: the dK/dV kernel with a workspace, which shares a
key tile's long query list between several workgroups and adds their fp32
partials in a second kernel (load balance under a causal mask with few
key/value heads, and under block masks with a sink column).  Checked against
the fp64 oracle and against fa_bwd_ex (the same products in one workgroup per
key tile: equal up to the order of fp32 additions), at every head dimension,
causal and not, ragged, with random and sink-column masks, at the full
8192-token head-dim-256 shape, and the workspace contract."""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_synth import normal_bf16_bits, random_block_mask, window_block_mask
from parity_util import check, check_masked, oracle_full, to_f64, to_gpu

pytestmark = pytest.mark.gpu


def make_bits(B, Hq, Hkv, Lq, Lk, D, seed):
    return {
        "q": normal_bf16_bits((B, Hq, Lq, D), seed + 0),
        "k": normal_bf16_bits((B, Hkv, Lk, D), seed + 1),
        "v": normal_bf16_bits((B, Hkv, Lk, D), seed + 2),
        "do": normal_bf16_bits((B, Hq, Lq, D), seed + 3),
    }


def both(g, scale, causal, mask=None, workspace=True):
    """Forward, delta, then the backward without and with the workspace."""
    import causal_gqa_flashattention_amd as fa
    o, lse = fa.fa_fwd_ex(g["q"], g["k"], g["v"], scale=scale, causal=causal, block_mask=mask)
    delta = fa.fa_bwd_delta_ex(o, g["do"])
    plain = fa.fa_bwd_ex(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=scale, causal=causal,
                         block_mask=mask)
    split = fa.fa_bwd_ex(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=scale, causal=causal,
                         block_mask=mask, workspace=workspace)
    torch.cuda.synchronize()
    return o, lse, plain, split


def agree(a, b, label):
    """dK / dV of the split and the one-workgroup kernels: the same products,
    partial sums added in another order."""
    err = (a.float() - b.float()).abs().max().item()
    ref = b.float().abs().max().item()
    print(f"[split] {label}: max|split - plain| = {err:.3e} ({err / max(ref, 1e-30):.2e} of max)", flush=True)
    assert err <= 4e-3 * ref, (label, err, ref)


def split_case(B, Hq, Hkv, Lq, Lk, D, causal, seed, mask=None):
    import causal_gqa_flashattention_amd as fa
    label = f"split B{B} Hq{Hq} Hkv{Hkv} Lq{Lq} Lk{Lk} D{D} causal={causal} mask={mask is not None}"
    need = fa.fa_bwd_workspace_bytes(B, Hq, Hkv, Lq, Lk, D, mask is not None)
    print(f"[case] {label}: workspace {need} bytes", flush=True)
    assert need > 0, "these shapes are chosen to split"
    bits = make_bits(B, Hq, Hkv, Lq, Lk, D, seed)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    g = {n: to_gpu(b) for n, b in bits.items()}
    mg = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    o, lse, plain, split = both(g, scale, causal, mg)
    assert torch.equal(split[0], plain[0]), "dq does not depend on the split"
    agree(split[1], plain[1], label + " dk")
    agree(split[2], plain[2], label + " dv")
    ref = oracle_full(bits, scale, causal, block_mask=mask)
    if mask is None:
        for n, t in (("dk", split[1]), ("dv", split[2])):
            check(n, to_f64(t), ref[n], label)
    else:
        keys_empty = ~oracle.visible_mask(Lq, Lk, causal, block_mask=mask).any(axis=0)
        for n, t in (("dk", split[1]), ("dv", split[2])):
            check_masked(n, to_f64(t), ref[n], label, keys_empty)


@pytest.mark.parametrize("D", [64, 96, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_split_parity(D, causal):
    # one key/value head: few key tiles, every list split up to 8 ways
    split_case(1, 4, 1, 1000, 1000, D, causal, seed=40000 + D + causal)


@pytest.mark.parametrize("D", [128, 256])
def test_split_ragged_rectangular(D):
    split_case(1, 8, 2, 777, 1300, D, True, seed=40500 + D)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_split_sink_column_mask(D):
    # a 256-key window plus the first key block seen by every query block
    mask = window_block_mask(1500, 1500, 256, sink_blocks=1)
    split_case(1, 4, 2, 1500, 1500, D, True, seed=41000 + D, mask=mask)


@pytest.mark.parametrize("D", [96, 256])
def test_split_random_mask(D):
    mask = random_block_mask(1100, 1100, 0.4, seed=41500 + D)
    split_case(1, 4, 1, 1100, 1100, D, False, seed=41600 + D, mask=mask)


def test_split_workspace_contract():
    import causal_gqa_flashattention_amd as fa
    B, Hq, Hkv, L, D = 1, 4, 1, 900, 128
    bits = make_bits(B, Hq, Hkv, L, L, D, 42000)
    g = {n: to_gpu(b) for n, b in bits.items()}
    n = fa.fa_bwd_workspace_bytes(B, Hq, Hkv, L, L, D)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")  # garbage on entry is fine
    o, lse, plain, a = both(g, 0.1, True, workspace=ws)
    _, _, _, b = both(g, 0.1, True, workspace=ws)  # reused: the same bits
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    delta = fa.fa_bwd_delta_ex(o, g["do"])
    with pytest.raises(fa.FAError):
        fa.fa_bwd_ex(g["q"], g["k"], g["v"], lse, delta, g["do"], scale=0.1, causal=True, workspace=ws[: n - 256])
    torch.cuda.synchronize()


@pytest.mark.slow
def test_split_d256_full_size():
    """The 8192-token head-dim-256 shape (16/2 heads, causal): every key of
    both key/value heads against the one-workgroup kernel, the first and last
    keys of one head against the oracle, and the key-sum identities."""
    import causal_gqa_flashattention_amd as fa
    from fa_synth import WORKLOADS, make_inputs
    w = WORKLOADS["d256_train8k"]
    print(f"[case] split d256_train8k workspace {fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D)}",
          flush=True)
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    o, lse, plain, split = both(g, w.softmax_scale, True)
    agree(split[1], plain[1], "d256_train8k dk")
    agree(split[2], plain[2], "d256_train8k dv")
    G, kvh = w.Hq // w.Hkv, 0
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    keys = np.concatenate([np.arange(128), np.arange(w.Lk - 128, w.Lk)])
    dk = np.zeros((keys.size, w.D))
    dv = np.zeros((keys.size, w.D))
    for h in range(kvh * G, (kvh + 1) * G):
        r = oracle.head_backward(oracle.bf16_bits_to_f64(bits["q"][0, h]), k, v,
                                 oracle.bf16_bits_to_f64(bits["do"][0, h]), w.softmax_scale, True, key_rows=keys)
        dk += r["dk"]
        dv += r["dv"]
    check("dk", to_f64(split[1][0, kvh, keys]), dk, "split d256_train8k first/last 128 keys")
    check("dv", to_f64(split[2][0, kvh, keys]), dv, "split d256_train8k first/last 128 keys")
    dkf = split[1].float()
    assert dkf.sum(dim=2).abs().max().item() <= 1e-2 * dkf.abs().sum(dim=2).max().item()
    dvs = split[2].float().sum(dim=2)
    dos = g["do"].float().reshape(w.B, w.Hkv, G, w.Lq, w.D).sum(dim=(2, 3))
    assert (dvs - dos).abs().max().item() <= 1e-2 * split[2].float().abs().sum(dim=2).max().item()


@pytest.mark.slow
def test_split_train8k_sink_window():
    """The 8192-token training shape under a 1024-key window plus one sink
    block: against the one-workgroup kernel on every key, and the sink
    block's keys (seen by every row) against the oracle on one group."""
    import causal_gqa_flashattention_amd as fa
    from fa_synth import WORKLOADS, make_inputs
    w = WORKLOADS["train8k"]
    mask = window_block_mask(w.Lq, w.Lk, 1024, sink_blocks=1)
    print(f"[case] split train8k window+sink, workspace {fa.fa_bwd_workspace_bytes(1, 32, 8, 8192, 8192, 128, 1)}",
          flush=True)
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    mg = torch.from_numpy(mask).cuda()
    o, lse, plain, split = both(g, w.softmax_scale, True, mg)
    agree(split[1], plain[1], "train8k window+sink dk")
    agree(split[2], plain[2], "train8k window+sink dv")
    G, kvh = w.Hq // w.Hkv, 2
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    keys = np.arange(64)
    dk = np.zeros((64, w.D))
    dv = np.zeros((64, w.D))
    for h in range(kvh * G, (kvh + 1) * G):
        r = oracle.head_backward(oracle.bf16_bits_to_f64(bits["q"][0, h]), k, v,
                                 oracle.bf16_bits_to_f64(bits["do"][0, h]), w.softmax_scale, True, key_rows=keys,
                                 block_mask=mask)
        dk += r["dk"]
        dv += r["dv"]
    check("dk", to_f64(split[1][0, kvh, keys]), dk, "split train8k sink block")
    check("dv", to_f64(split[2][0, kvh, keys]), dv, "split train8k sink block")
