"""GPU parity at the full sizes of the measured workloads, in the launch
configuration bench.py times (the same three calls on whole tensors),
checked against the fp64 oracle on what it can compute in seconds:

* 8192-token training shape (B=1, 32/8 heads, D=128, causal): one whole
  GQA group, i.e. its 4 query heads over all 8192 rows (O, LSE, dQ) and the
  dK/dV of its key/value head over all 8192 keys;
* dense 4096 (B=2, 16/16 heads, non-causal, inputs x0.5) at D=64 and D=96:
  one whole (batch, head) pair each;
* head dim 256 forward (B=1, 16/2 heads, causal, scale 1/16) at 8192^2,
  4064x4096 and 8200^2: 512 sampled rows (first, last, tile edges, ragged
  tail, seeded rest) of all 8 query heads of one key/value head;
* 23040-token long context (B=1, 32/8, D=128, causal): 256 sampled rows of
  one group (O, LSE, dQ), dK/dV of its first 256 keys (seen by every row:
  the longest accumulations) and of its last 512 keys, the identities
  sum_j dK_j = 0 and sum_j dV_j = sum over the group of dO over the whole
  tensors, and peak device memory equal to the resident tensors (the
  library allocates nothing; a materialised fp32 score matrix would need
  63 GiB).
"""
import gc

import numpy as np
import pytest
import torch

import oracle
from fa_synth import WORKLOADS, make_inputs
from parity_util import check, run_library, to_f64, to_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_rows(L, n, seed, tile=128):
    rng = np.random.default_rng(seed)
    fixed = {0, 1, L - 1, L - 2}
    for t in range(tile, L, tile):
        fixed.update({t - 1, t, t + 1})
    fixed = sorted(r for r in fixed if 0 <= r < L)
    rng.shuffle(fixed)
    fixed = fixed[: n // 2]
    rest = rng.choice(L, size=n, replace=False)
    rows = list(dict.fromkeys(list(fixed) + list(rest)))[:n]
    return np.array(sorted(rows))


def run_workload(name):
    w = WORKLOADS[name]
    print(f"[workload] {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lq={w.Lq} Lk={w.Lk} D={w.D} causal={w.causal}",
          flush=True)
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    out = run_library(g["q"], g["k"], g["v"], g.get("do"), w.softmax_scale, w.causal, backward=w.backward)
    return w, bits, g, out


def test_train8k_whole_group():
    w, bits, g, out = run_workload("train8k")
    G = w.Hq // w.Hkv
    kvh = 5
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(kvh * G, (kvh + 1) * G):
        r = oracle.head_backward(oracle.bf16_bits_to_f64(bits["q"][0, h]), k, v,
                                 oracle.bf16_bits_to_f64(bits["do"][0, h]), w.softmax_scale, True)
        for n in ("o", "lse", "dq"):
            check(n, to_f64(out[n][0, h]), r[n], f"train8k head {h}")
        dk += r["dk"]
        dv += r["dv"]
    check("dk", to_f64(out["dk"][0, kvh]), dk, f"train8k kv head {kvh}")
    check("dv", to_f64(out["dv"][0, kvh]), dv, f"train8k kv head {kvh}")


@pytest.mark.parametrize("name,b,h", [("dense4k_d64", 1, 11), ("dense4k_d96", 0, 3)])
def test_dense4k_one_head(name, b, h):
    w, bits, g, out = run_workload(name)
    r = oracle.head_backward(*(oracle.bf16_bits_to_f64(bits[n][b, h]) for n in ("q", "k", "v", "do")),
                             w.softmax_scale, False)
    for n in ("o", "lse", "dq", "dk", "dv"):
        check(n, to_f64(out[n][b, h]), r[n], f"{name} b{b} h{h}")


@pytest.mark.parametrize("name", ["d256_8192", "d256_4064x4096", "d256_8200"])
def test_d256_forward_sampled_rows(name):
    w, bits, g, out = run_workload(name)
    G = w.Hq // w.Hkv
    kvh = 1
    rows = sample_rows(w.Lq, 512, seed=w.seed, tile=128)
    rows = np.union1d(rows, np.arange(max(0, w.Lq - 8), w.Lq))  # the ragged tail rows
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    for h in range(kvh * G, (kvh + 1) * G):
        o, lse = oracle.head_forward(oracle.bf16_bits_to_f64(bits["q"][0, h]), k, v, w.softmax_scale, True,
                                     rows=rows)
        check("o", to_f64(out["o"][0, h, rows]), o, f"{name} head {h}")
        check("lse", to_f64(out["lse"][0, h, rows]), lse, f"{name} head {h}")


def test_long23k_sampled_and_identities():
    w = WORKLOADS["long23k"]
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    torch.cuda.synchronize()
    import causal_gqa_flashattention_amd as fa
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    torch.cuda.synchronize()
    gc.collect()  # garbage of earlier tests must not be freed inside the window
    torch.cuda.reset_peak_memory_stats()
    resident = torch.cuda.memory_allocated()
    fa.fa_fwd(g["q"], g["k"], g["v"], o, lse, scale=w.softmax_scale, causal=True)
    fa.fa_bwd_delta(o, g["do"], delta)
    fa.fa_bwd(g["q"], g["k"], g["v"], o, lse, delta, g["do"], dq, dk, dv, scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    print(f"[memory] resident={resident} peak={peak} (fp32 score matrix would be "
          f"{w.Hq * w.Lq * w.Lk * 4} bytes)", flush=True)
    assert peak == resident, "the library must not allocate device memory"

    G = w.Hq // w.Hkv
    kvh = 3
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    rows = sample_rows(w.Lq, 256, seed=w.seed, tile=128)
    tail = np.arange(w.Lq - 512, w.Lq)
    head = np.arange(256)
    dk_tail, dv_tail = np.zeros((512, w.D)), np.zeros((512, w.D))
    dk_head, dv_head = np.zeros((256, w.D)), np.zeros((256, w.D))
    for h in range(kvh * G, (kvh + 1) * G):
        q = oracle.bf16_bits_to_f64(bits["q"][0, h])
        do = oracle.bf16_bits_to_f64(bits["do"][0, h])
        r = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=rows)
        for n, t in (("o", o), ("lse", lse), ("dq", dq)):
            check(n, to_f64(t[0, h, rows]), r[n], f"long23k head {h}")
        # keys j >= Lk-512 are seen only by rows i >= j (Lq == Lk)
        rt = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=tail, key_rows=tail)
        dk_tail += rt["dk"]
        dv_tail += rt["dv"]
        # keys 0..255 are seen by every row: all 23040 rows of the head
        rh = oracle.head_backward(q, k, v, do, w.softmax_scale, True, key_rows=head)
        dk_head += rh["dk"]
        dv_head += rh["dv"]
        print(f"[oracle] long23k head {h} done", flush=True)
    check("dk", to_f64(dk[0, kvh, tail]), dk_tail, f"long23k kv head {kvh} last 512 keys")
    check("dv", to_f64(dv[0, kvh, tail]), dv_tail, f"long23k kv head {kvh} last 512 keys")
    check("dk", to_f64(dk[0, kvh, head]), dk_head, f"long23k kv head {kvh} first 256 keys")
    check("dv", to_f64(dv[0, kvh, head]), dv_head, f"long23k kv head {kvh} first 256 keys")

    check_key_sums(w, dk, dv, g["do"])


def check_key_sums(w, dk, dv, do):
    """Identities over the whole tensors, every key of every head: rows of dS
    sum to zero, so sum_j dK[j] = scale * sum_i q_i * sum_j dS_ij = 0; rows of
    P sum to one, so sum_j dV[j] = sum over the group's rows of dO.  Causal
    with Lq == Lk: every row sees at least one key.  bf16 outputs: compared
    against the size of the summed terms."""
    G = w.Hq // w.Hkv
    dkf = dk.float()
    ksum = dkf.sum(dim=2).abs().max().item()
    kscale = dkf.abs().sum(dim=2).max().item()
    assert ksum <= 1e-2 * kscale, (ksum, kscale)
    dvs = dv.float().sum(dim=2)
    dos = do.float().reshape(w.B, w.Hkv, G, w.Lq, w.D).sum(dim=(2, 3))
    err = (dvs - dos).abs().max().item()
    assert err <= 1e-2 * dv.float().abs().sum(dim=2).max().item(), err


def test_d256_fwd_bwd_sampled():
    """Head dim 256 forward + backward at 8192 tokens (16/2 heads, causal):
    sampled rows of one group for O, LSE, dQ; dK/dV of the group's first 256
    keys (seen by every row) and last 512 keys; the key-sum identities over
    every head."""
    w, bits, g, out = run_workload("d256_train8k")
    G = w.Hq // w.Hkv
    kvh = 1
    k = oracle.bf16_bits_to_f64(bits["k"][0, kvh])
    v = oracle.bf16_bits_to_f64(bits["v"][0, kvh])
    rows = sample_rows(w.Lq, 128, seed=w.seed, tile=128)
    tail = np.arange(w.Lq - 512, w.Lq)
    head = np.arange(256)
    dk_tail, dv_tail = np.zeros((512, w.D)), np.zeros((512, w.D))
    dk_head, dv_head = np.zeros((256, w.D)), np.zeros((256, w.D))
    for h in range(kvh * G, (kvh + 1) * G):
        q = oracle.bf16_bits_to_f64(bits["q"][0, h])
        do = oracle.bf16_bits_to_f64(bits["do"][0, h])
        r = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=rows)
        for n in ("o", "lse", "dq"):
            check(n, to_f64(out[n][0, h, rows]), r[n], f"d256_train8k head {h}")
        rt = oracle.head_backward(q, k, v, do, w.softmax_scale, True, rows=tail, key_rows=tail)
        dk_tail += rt["dk"]
        dv_tail += rt["dv"]
        # the first 256 keys are seen by every row: the longest accumulations
        rh = oracle.head_backward(q, k, v, do, w.softmax_scale, True, key_rows=head)
        dk_head += rh["dk"]
        dv_head += rh["dv"]
    check("dk", to_f64(out["dk"][0, kvh, tail]), dk_tail, f"d256_train8k kv head {kvh} last 512 keys")
    check("dv", to_f64(out["dv"][0, kvh, tail]), dv_tail, f"d256_train8k kv head {kvh} last 512 keys")
    check("dk", to_f64(out["dk"][0, kvh, head]), dk_head, f"d256_train8k kv head {kvh} first 256 keys")
    check("dv", to_f64(out["dv"][0, kvh, head]), dv_head, f"d256_train8k kv head {kvh} first 256 keys")
    check_key_sums(w, out["dk"], out["dv"], g["do"])


@pytest.mark.parametrize("L", [4096, 8192, 16384])
def test_memory_linear_in_length(L):
    """Peak device memory of a forward + backward equals the resident tensors
    (inputs, outputs, LSE, delta), which grow linearly in L; the library
    allocates nothing, where an fp32 score matrix would grow as L^2."""
    import causal_gqa_flashattention_amd as fa
    from fa_synth import AttnShape
    w = AttnShape(name=f"mem{L}", B=1, Hq=32, Hkv=8, Lq=L, Lk=L, D=128, causal=True, seed=7000 + L // 4096)
    bits = make_inputs(w)
    g = {n: to_gpu(b) for n, b in bits.items()}
    o = torch.empty_like(g["q"])
    lse = torch.empty((w.B, w.Hq, L), dtype=torch.float32, device="cuda")
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    torch.cuda.synchronize()
    gc.collect()  # garbage of earlier tests must not be freed inside the window
    torch.cuda.reset_peak_memory_stats()
    resident = torch.cuda.memory_allocated()
    fa.fa_fwd(g["q"], g["k"], g["v"], o, lse, scale=w.softmax_scale, causal=True)
    fa.fa_bwd_delta(o, g["do"], delta)
    fa.fa_bwd(g["q"], g["k"], g["v"], o, lse, delta, g["do"], dq, dk, dv, scale=w.softmax_scale, causal=True)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated()
    tensors = sum(t.numel() * t.element_size() for t in (*g.values(), o, lse, delta, dq, dk, dv))
    print(f"[memory] L={L} resident={resident} peak={peak} tensors={tensors} "
          f"fp32 scores would be {w.Hq * L * L * 4}", flush=True)
    assert peak == resident
    assert resident >= tensors
    assert torch.isfinite(o.float()).all() and torch.isfinite(dk.float()).all()
