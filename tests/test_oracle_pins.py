"""Pins for the fp64 oracle: closed forms, invariants, finite differences and
an independent library routine (torch's CPU attention in float64 with
autograd).  None of these re-types the oracle's formulas: each checks it
against a fact that the pages or the mathematics fix.

Pages: "When the Bottleneck Moved" section 3 (definition and online
recurrence); "feat(attention): complete Flash Attention VJP implementation"
Background (the backward's five products, delta = rowsum(dO*O));
"Add a fused full-attention path for head_dim 256 on NAX devices", Design,
ragged causal inputs (bottom-right causal alignment).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from fa_synth import bf16_bits_from_f32, normal_bf16_bits

RNG = np.random.default_rng(1234)


def rnd(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


def visible_count(Lq, Lk, causal):
    if not causal:
        return np.full(Lq, Lk)
    return np.minimum(Lk, np.arange(Lq) + (Lk - Lq) + 1)


# ---------------------------------------------------------------- softmax rows


@pytest.mark.parametrize("Lq,Lk,causal", [(7, 7, True), (5, 9, True), (6, 4, False), (1, 1, True)])
def test_probabilities_sum_to_one_and_masked_are_zero(Lq, Lk, causal):
    # With V = identity (D = Lk) the output row is exactly the probability row.
    D = Lk
    q, k = rnd(Lq, D), rnd(Lk, D)
    v = np.eye(Lk)
    p, lse = oracle.head_forward(q, k, v, 0.7, causal)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-12)
    vis = np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq) if causal else np.ones((Lq, Lk), bool)
    assert np.all(p[~vis] == 0.0), "masked keys must get exactly zero probability"
    assert np.all(p[vis] > 0.0)
    # LSE lies between the largest visible score and that plus log(#visible)
    s = 0.7 * q @ k.T
    smax = np.where(vis, s, -np.inf).max(axis=1)
    n = visible_count(Lq, Lk, causal)
    assert np.all(lse >= smax - 1e-12) and np.all(lse <= smax + np.log(n) + 1e-12)


# ------------------------------------------------------------- closed forms


@pytest.mark.parametrize("Lq,Lk", [(8, 8), (5, 12), (1, 3)])
def test_zero_query_gives_running_mean_of_v(Lq, Lk):
    D = 4
    v = rnd(Lk, D)
    o, lse = oracle.head_forward(np.zeros((Lq, D)), rnd(Lk, D), v, 0.3, True)
    n = visible_count(Lq, Lk, True)
    for i in range(Lq):
        np.testing.assert_allclose(o[i], v[: n[i]].mean(axis=0), atol=1e-13)
        assert abs(lse[i] - math.log(n[i])) < 1e-13
    # K = 0 gives the same (every visible score is 0)
    o2, lse2 = oracle.head_forward(rnd(Lq, D), np.zeros((Lk, D)), v, 0.3, True)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)


def test_single_visible_key_row():
    # causal, Lq == Lk: row 0 sees only key 0, so O_0 = V_0, LSE_0 = S_00, dQ_0 = 0
    L, D, sc = 6, 5, 0.4
    q, k, v, do = rnd(L, D), rnd(L, D), rnd(L, D), rnd(L, D)
    r = oracle.head_backward(q, k, v, do, sc, True)
    np.testing.assert_allclose(r["o"][0], v[0], atol=1e-14)
    assert abs(r["lse"][0] - sc * q[0] @ k[0]) < 1e-13
    np.testing.assert_allclose(r["dq"][0], 0.0, atol=1e-14)


def test_uniform_scores_backward_closed_form():
    # Q = 0, non-causal: P = 1/Lk everywhere, O = mean(V) for every row,
    # dV_j = (1/Lk) * sum_i dO_i, dK_j = scale/Lk * sum_i (dO_i.(V_j - Vbar)) Q_i = 0,
    # dQ_i = scale/Lk * sum_j (dO_i.(V_j - Vbar)) K_j.
    Lq, Lk, D, sc = 5, 7, 3, 0.9
    k, v, do = rnd(Lk, D), rnd(Lk, D), rnd(Lq, D)
    r = oracle.head_backward(np.zeros((Lq, D)), k, v, do, sc, False)
    vbar = v.mean(axis=0)
    np.testing.assert_allclose(r["o"], np.tile(vbar, (Lq, 1)), atol=1e-14)
    np.testing.assert_allclose(r["dv"], np.tile(do.sum(axis=0) / Lk, (Lk, 1)), atol=1e-13)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-14)
    for i in range(Lq):
        want = sc / Lk * sum((do[i] @ (v[j] - vbar)) * k[j] for j in range(Lk))
        np.testing.assert_allclose(r["dq"][i], want, atol=1e-13)


# ---------------------------------------------------------------- invariances


def test_key_shift_and_value_shift():
    Lq, Lk, D, sc = 6, 9, 4, 0.5
    q, k, v = rnd(Lq, D), rnd(Lk, D), rnd(Lk, D)
    u, c = rnd(D), rnd(D)
    o, lse = oracle.head_forward(q, k, v, sc, True)
    o2, lse2 = oracle.head_forward(q, k + u, v, sc, True)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + sc * q @ u, atol=1e-12)
    o3, _ = oracle.head_forward(q, k, v + c, sc, True)
    np.testing.assert_allclose(o3, o + c, atol=1e-12)


def test_noncausal_key_permutation():
    Lq, Lk, D = 5, 8, 3
    q, k, v = rnd(Lq, D), rnd(Lk, D), rnd(Lk, D)
    perm = RNG.permutation(Lk)
    o, lse = oracle.head_forward(q, k, v, 0.8, False)
    o2, lse2 = oracle.head_forward(q, k[perm], v[perm], 0.8, False)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


@pytest.mark.parametrize("Lq,Lk,causal,bn", [(37, 37, True, 8), (20, 45, True, 16), (33, 17, False, 5)])
def test_online_recurrence_equals_direct(Lq, Lk, causal, bn):
    D = 6
    q, k, v = rnd(Lq, D, scale=2.0), rnd(Lk, D), rnd(Lk, D)
    o, lse = oracle.head_forward(q, k, v, 0.6, causal)
    o2, lse2 = oracle.head_forward_online(q, k, v, 0.6, causal, block_n=bn)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


# ---------------------------------------------------------------- gradients


def _loss(q, k, v, do, sc, causal):
    o, _ = oracle.forward(q, k, v, sc, causal)
    return float((o * do).sum())


@pytest.mark.parametrize("L,causal", [(5, True), (8, True), (13, True), (6, False)])
def test_finite_differences(L, causal):
    B, Hq, Hkv, D, sc = 1, 2, 1, 8, 0.35
    q, k, v = rnd(B, Hq, L, D), rnd(B, Hkv, L, D), rnd(B, Hkv, L, D)
    do = rnd(B, Hq, L, D)
    g = oracle.backward(q, k, v, do, sc, causal)
    eps = 1e-5
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name[1]] = xp
            args_m[name[1]] = xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, sc, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, sc, causal)) / (2 * eps)
        err = np.abs(num - g[name]).max() / max(1e-12, np.abs(num).max())
        assert err < 1e-6, (name, err)


def test_gradient_sum_identities():
    # Rows of dS sum to zero, so sum_j dK_j = 0; rows of P sum to one, so
    # sum_j dV_j = sum over the group's heads and rows of dO.
    B, Hq, Hkv, L, D = 2, 4, 2, 11, 5
    q, k, v, do = rnd(B, Hq, L, D), rnd(B, Hkv, L, D), rnd(B, Hkv, L, D), rnd(B, Hq, L, D)
    g = oracle.backward(q, k, v, do, 0.45, True)
    np.testing.assert_allclose(g["dk"].sum(axis=2), 0.0, atol=1e-12)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hkv):
            want = do[b, h * G:(h + 1) * G].sum(axis=(0, 1))
            np.testing.assert_allclose(g["dv"][b, h].sum(axis=0), want, atol=1e-12)
    # delta equals rowsum(P * dP) as well as rowsum(dO * O): check against dO.O
    np.testing.assert_allclose(g["delta"], oracle.delta(g["o"], do), atol=1e-12)


def test_delta_closed_form():
    o = np.ones((2, 3, 4, 16))
    do = np.broadcast_to(np.arange(16.0), (2, 3, 4, 16))
    np.testing.assert_array_equal(oracle.delta(o, do), np.full((2, 3, 4), 120.0))


def test_gqa_equals_repeated_mha():
    B, Hq, Hkv, L, D = 1, 6, 2, 9, 4
    G = Hq // Hkv
    q, k, v, do = rnd(B, Hq, L, D), rnd(B, Hkv, L, D), rnd(B, Hkv, L, D), rnd(B, Hq, L, D)
    g = oracle.backward(q, k, v, do, 0.5, True)
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    m = oracle.backward(q, kr, vr, do, 0.5, True)
    for n in ("o", "lse", "dq"):
        np.testing.assert_allclose(g[n], m[n], atol=1e-13)
    np.testing.assert_allclose(g["dk"], m["dk"].reshape(B, Hkv, G, L, D).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(g["dv"], m["dv"].reshape(B, Hkv, G, L, D).sum(axis=2), atol=1e-13)


# ------------------------------------------------- independent library routine


def _torch_reference(q, k, v, do, sc, causal):
    """torch float64 CPU attention with autograd; bottom-right causal mask."""
    Lq, Lk = q.shape[2], k.shape[2]
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = None
    if causal:
        mask = torch.arange(Lk)[None, :] <= torch.arange(Lq)[:, None] + (Lk - Lq)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=mask, scale=sc, enable_gqa=True)
    o.backward(torch.tensor(do))
    G = q.shape[1] // k.shape[1]
    s = torch.matmul(tq.detach(), tk.detach().repeat_interleave(G, dim=1).transpose(-1, -2)) * sc
    if causal:
        s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return {"o": o.detach().numpy(), "lse": lse.numpy(), "dq": tq.grad.numpy(),
            "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,D,causal", [
    (1, 2, 1, 61, 61, 64, True),
    (2, 4, 1, 64, 64, 16, True),
    (1, 32, 8, 64, 64, 8, True),     # the 32/8 grouping at length 64
    (1, 4, 2, 40, 97, 8, True),      # bottom-right causal, Lq < Lk
    (2, 2, 2, 33, 20, 8, False),     # dense, Lq > Lk
])
def test_matches_torch_float64_autograd(B, Hq, Hkv, Lq, Lk, D, causal):
    q, k, v, do = rnd(B, Hq, Lq, D), rnd(B, Hkv, Lk, D), rnd(B, Hkv, Lk, D), rnd(B, Hq, Lq, D)
    sc = 1.0 / math.sqrt(D)
    g = oracle.backward(q, k, v, do, sc, causal, block=16)
    t = _torch_reference(q, k, v, do, sc, causal)
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(g[n], t[n], atol=1e-10, rtol=1e-10, err_msg=n)


def test_flash_cpu_kernel_lse():
    # torch's CPU fused attention returns the log-sum-exp directly (top-left
    # causal, which equals bottom-right when Lq == Lk).
    B, H, L, D = 1, 3, 29, 16
    q, k, v = rnd(B, H, L, D), rnd(B, H, L, D), rnd(B, H, L, D)
    o_t, lse_t = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        torch.tensor(q), torch.tensor(k), torch.tensor(v), 0.0, True, scale=0.25)[:2]
    o, lse = oracle.forward(q, k, v, 0.25, True)
    np.testing.assert_allclose(o, o_t.numpy(), atol=1e-10)
    np.testing.assert_allclose(lse, lse_t.numpy(), atol=1e-10)


# ------------------------------------------------ subsets used by spot checks


def test_row_and_key_subsets_agree_with_full():
    Lq, Lk, D = 50, 70, 8
    q, k, v, do = rnd(Lq, D), rnd(Lk, D), rnd(Lk, D), rnd(Lq, D)
    full = oracle.head_backward(q, k, v, do, 0.3, True, block=16)
    rows = np.array([0, 3, 17, 49])
    part = oracle.head_backward(q, k, v, do, 0.3, True, rows=rows, block=3)
    for n in ("o", "lse", "delta", "dq"):
        np.testing.assert_allclose(part[n], full[n][rows], atol=1e-13)
    keys = np.array([0, 19, 20, 69])
    kp = oracle.head_backward(q, k, v, do, 0.3, True, key_rows=keys, block=7)
    np.testing.assert_allclose(kp["dk"], full["dk"][keys], atol=1e-13)
    np.testing.assert_allclose(kp["dv"], full["dv"][keys], atol=1e-13)
    o, lse = oracle.head_forward(q, k, v, 0.3, True, rows=rows, block=2)
    np.testing.assert_allclose(o, full["o"][rows], atol=1e-13)


def test_rows_without_visible_key_are_rejected():
    # causal with Lq > Lk leaves the first rows with no key: undefined softmax
    with pytest.raises(ValueError):
        oracle.head_forward(rnd(5, 4), rnd(3, 4), rnd(3, 4), 1.0, True)


# ----------------------------------------------------- input bits round trip


def test_bf16_widening_is_exact():
    x = np.array([1.0, -2.5, 3.140625, 0.0, 65280.0, 1e-30], dtype=np.float32)
    bits = bf16_bits_from_f32(x)
    back = oracle.bf16_bits_to_f64(bits)
    torch_bits = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, torch_bits)   # RNE agrees with torch's cast
    np.testing.assert_array_equal(back, torch.tensor(x).to(torch.bfloat16).double().numpy())
    b = normal_bf16_bits((3, 5), seed=7)
    np.testing.assert_array_equal(b, normal_bf16_bits((3, 5), seed=7))


def test_f16_widening_is_exact():
    # IEEE binary16 values by their definition: sign, 5-bit exponent (bias
    # 15), 10-bit fraction; subnormals scale the fraction by 2^-24
    bits = np.array([0x3C00, 0xC000, 0x7BFF, 0x0001, 0x03FF, 0x0400, 0x3555, 0x8000], dtype=np.uint16)
    want = np.array([1.0, -2.0, 65504.0, 2.0 ** -24, 1023 * 2.0 ** -24, 2.0 ** -14,
                     (1 + 0x155 / 1024) * 2.0 ** -2, -0.0])
    got = oracle.f16_bits_to_f64(bits)
    np.testing.assert_array_equal(got, want)
    assert np.signbit(got[-1])
    # the input rounding agrees with torch's cast (round to nearest even)
    from fa_synth import f16_bits_from_f32, normal_f16_bits
    x = np.array([1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -3.14159, 65519.0], dtype=np.float32)
    tb = torch.tensor(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f16_bits_from_f32(x), tb)
    np.testing.assert_array_equal(normal_f16_bits((3, 5), seed=7), normal_f16_bits((3, 5), seed=7))
    np.testing.assert_array_equal(oracle.bits_to_f64(bits, "f16"), want)


# ---------------------------------------------------------------- block-sparse mask
# Page "feat(attention): complete Flash Attention VJP implementation", "Sparse
# Block Masks": one uint8 entry per (query tile, key tile); here 64 x 64.


def _expand(bm, Lq, Lk, causal):
    """Element mask from a block mask, written independently of the oracle."""
    m = np.repeat(np.repeat(np.asarray(bm) != 0, 64, axis=0), 64, axis=1)[:Lq, :Lk]
    if causal:
        m &= np.arange(Lk)[None, :] <= np.arange(Lq)[:, None] + (Lk - Lq)
    return m


def _torch_masked(q, k, v, do, sc, elem):
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    m = torch.tensor(elem)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=sc, enable_gqa=True)
    o.backward(torch.tensor(do))
    G = q.shape[1] // k.shape[1]
    s = torch.matmul(tq.detach(), tk.detach().repeat_interleave(G, dim=1).transpose(-1, -2)) * sc
    lse = torch.logsumexp(s.masked_fill(~m, float("-inf")), dim=-1)
    return {"o": o.detach().numpy(), "lse": lse.numpy(), "dq": tq.grad.numpy(),
            "dk": tk.grad.numpy(), "dv": tv.grad.numpy()}


def _random_block_mask(Lq, Lk, causal, seed, density=0.5):
    """Seeded block mask in which every query row keeps at least one key:
    the block holding each row's last visible key is always kept."""
    r = np.random.default_rng(seed)
    nq, nk = -(-Lq // 64), -(-Lk // 64)
    bm = (r.random((nq, nk)) < density).astype(np.uint8)
    for qb in range(nq):
        last_row = min(Lq, 64 * qb + 64) - 1
        first_row = 64 * qb
        # keep the blocks of the diagonal keys of every row in the tile
        for i in (first_row, last_row):
            j = min(Lk - 1, i + (Lk - Lq)) if causal else Lk - 1
            bm[qb, j // 64] = 1
        if causal:
            for i in range(first_row, last_row + 1):
                bm[qb, min(Lk - 1, i + Lk - Lq) // 64] = 1
    return bm


def test_all_ones_block_mask_is_dense():
    q, k, v, do = rnd(1, 2, 130, 16), rnd(1, 1, 150, 16), rnd(1, 1, 150, 16), rnd(1, 2, 130, 16)
    for causal in (True, False):
        ones = np.ones((3, 3), dtype=np.uint8)
        a = oracle.backward(q, k, v, do, 0.25, causal, block=32)
        b = oracle.backward(q, k, v, do, 0.25, causal, block=32, block_mask=ones)
        for n in ("o", "lse", "dq", "dk", "dv"):
            assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("B,Hq,Hkv,Lq,Lk,D,causal,seed", [
    (1, 2, 1, 200, 200, 16, True, 1),
    (1, 4, 2, 130, 260, 8, True, 2),     # bottom-right causal, ragged tiles
    (2, 2, 2, 190, 140, 8, False, 3),    # dense, Lq > Lk
    (1, 2, 1, 256, 256, 8, False, 4),
])
def test_block_mask_matches_torch_float64(B, Hq, Hkv, Lq, Lk, D, causal, seed):
    q, k, v, do = rnd(B, Hq, Lq, D), rnd(B, Hkv, Lk, D), rnd(B, Hkv, Lk, D), rnd(B, Hq, Lq, D)
    bm = _random_block_mask(Lq, Lk, causal, seed)
    assert 0 < bm.sum() < bm.size  # some tiles kept, some skipped
    sc = 1.0 / math.sqrt(D)
    g = oracle.backward(q, k, v, do, sc, causal, block=48, block_mask=bm)
    t = _torch_masked(q, k, v, do, sc, _expand(bm, Lq, Lk, causal))
    for n in ("o", "lse", "dq", "dk", "dv"):
        np.testing.assert_allclose(g[n], t[n], rtol=1e-10, atol=1e-12, err_msg=n)


def test_block_mask_rows_without_keys():
    """A query tile whose mask row is all zero: its rows get O = 0, LSE = -inf
    and dQ = 0, and dK/dV equal those of the problem without those rows."""
    Lq = Lk = 192
    q, k, v, do = rnd(1, 2, Lq, 8), rnd(1, 1, Lk, 8), rnd(1, 1, Lk, 8), rnd(1, 2, Lq, 8)
    bm = np.ones((3, 3), dtype=np.uint8)
    bm[1, :] = 0
    g = oracle.backward(q, k, v, do, 0.3, False, block=40, block_mask=bm)
    empty = slice(64, 128)
    assert np.all(g["o"][:, :, empty] == 0) and np.all(g["dq"][:, :, empty] == 0)
    assert np.all(np.isneginf(g["lse"][:, :, empty]))
    keep = np.r_[0:64, 128:192]
    elem = np.ones((128, Lk), dtype=bool)
    t = _torch_masked(q[:, :, keep], k, v, do[:, :, keep], 0.3, elem)
    for n in ("o", "lse", "dq"):
        np.testing.assert_allclose(g[n][:, :, keep], t[n], rtol=1e-10, atol=1e-12, err_msg=n)
    for n in ("dk", "dv"):
        np.testing.assert_allclose(g[n], t[n], rtol=1e-10, atol=1e-12, err_msg=n)


def test_block_diagonal_mask_is_independent_blocks():
    """Non-causal block-diagonal mask: each 64-row tile attends only its own
    64 keys, i.e. independent attention per tile (closed-form split)."""
    L = 192
    q, k, v, do = rnd(1, 1, L, 8), rnd(1, 1, L, 8), rnd(1, 1, L, 8), rnd(1, 1, L, 8)
    bm = np.eye(3, dtype=np.uint8)
    g = oracle.backward(q, k, v, do, 0.5, False, block=64, block_mask=bm)
    for b in range(3):
        s = slice(64 * b, 64 * b + 64)
        t = _torch_masked(q[:, :, s], k[:, :, s], v[:, :, s], do[:, :, s], 0.5, np.ones((64, 64), dtype=bool))
        for n in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(g[n][:, :, s], t[n], rtol=1e-10, atol=1e-12, err_msg=n)
