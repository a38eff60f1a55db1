"""Plain fp64 attention forward/backward (test infrastructure only).

Every contraction is a numpy float64 matmul; the score matrix S, the
probabilities P, dP and dS are materialised explicitly for a block of query
rows, so the code reads as the definition.  See ``oracle/__init__.py`` for
the page passages each step follows.
"""
from __future__ import annotations

import numpy as np

_NEG_INF = -np.inf

# Granularity of a block-sparse mask: 64 query rows x 64 keys per entry.
MASK_BLOCK = 64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16/int16) to float64."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE binary16 bit patterns (uint16/int16) to float64
    (the float16 element type of "feat(attention): complete Flash Attention
    VJP implementation", summary)."""
    return np.ascontiguousarray(bits).view(np.float16).astype(np.float64)


def bits_to_f64(bits: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """bf16_bits_to_f64 or f16_bits_to_f64 by element type name."""
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    raise ValueError(f"unknown element type {dtype}")


def visible_mask(Lq: int, Lk: int, causal: bool, rows=None, block_mask=None) -> np.ndarray:
    """Boolean [len(rows), Lk]: may query row i attend to key j?

    Causal masking is bottom-right aligned: j <= i + (Lk - Lq)
    ("Add a fused full-attention path for head_dim 256 on NAX devices",
    Design, ragged causal inputs).  Without a causal mask every key is seen.

    ``block_mask`` ([ceil(Lq/64), ceil(Lk/64)], nonzero = kept) additionally
    hides every pair (i, j) whose entry [i // 64, j // 64] is 0: the sparse
    block masks of "feat(attention): complete Flash Attention VJP
    implementation", "Sparse Block Masks" (tile pairs with a 0 entry are
    skipped), at a fixed 64 x 64 granularity.
    """
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    if not causal:
        vis = np.ones((rows.shape[0], Lk), dtype=bool)
    else:
        off = Lk - Lq
        vis = np.arange(Lk)[None, :] <= (rows[:, None] + off)
    if block_mask is not None:
        bm = np.asarray(block_mask)
        if bm.shape != (-(-Lq // MASK_BLOCK), -(-Lk // MASK_BLOCK)):
            raise ValueError(f"block mask shape {bm.shape} does not match Lq={Lq}, Lk={Lk}")
        vis = vis & (bm[rows // MASK_BLOCK][:, np.arange(Lk) // MASK_BLOCK] != 0)
    return vis


def _scores(qb: np.ndarray, kh: np.ndarray, scale: float, vis: np.ndarray) -> np.ndarray:
    """S = scale * Q K^T, with -inf where the mask hides a key."""
    s = scale * (qb @ kh.T)
    return np.where(vis, s, _NEG_INF)


def _lse(s: np.ndarray, allow_empty: bool = False) -> np.ndarray:
    """Natural-log log-sum-exp of each row: m + log(sum exp(s - m)).

    A row that sees no key has no softmax.  Without a block mask that cannot
    happen for valid sizes and is an error; with one (``allow_empty``) such a
    row gets LSE = -inf (the log of an empty sum).
    """
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    if np.any(empty) and not allow_empty:
        raise ValueError("a query row sees no key; its softmax is undefined")
    safe = np.where(empty, 0.0, m)
    tot = np.exp(s - safe[:, None]).sum(axis=1)
    return np.where(empty, _NEG_INF, safe + np.log(np.where(empty, 1.0, tot)))


def _probs(s: np.ndarray, l: np.ndarray) -> np.ndarray:
    """P = exp(S - LSE) per row; all zero for a row that sees no key."""
    return np.where(np.isfinite(l)[:, None], np.exp(s - np.where(np.isfinite(l), l, 0.0)[:, None]), 0.0)


def _row_blocks(rows: np.ndarray, block: int):
    for i in range(0, rows.shape[0], block):
        yield rows[i:i + block]


def head_forward(qh, kh, vh, scale, causal, rows=None, block=256, block_mask=None):
    """One head: O and LSE for the given query rows (default: all rows).

    qh [Lq, D], kh/vh [Lk, D] float64.  Returns (o [n, D], lse [n]).  With a
    block mask, a row that sees no key gets O = 0 and LSE = -inf.
    """
    Lq, Lk = qh.shape[0], kh.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    o = np.empty((rows.shape[0], vh.shape[1]))
    lse = np.empty(rows.shape[0])
    pos = 0
    for rb in _row_blocks(rows, block):
        s = _scores(qh[rb], kh, scale, visible_mask(Lq, Lk, causal, rb, block_mask))
        l = _lse(s, allow_empty=block_mask is not None)
        p = _probs(s, l)                    # softmax rows, 0 where masked
        o[pos:pos + rb.shape[0]] = p @ vh   # O = P V
        lse[pos:pos + rb.shape[0]] = l
        pos += rb.shape[0]
    return o, lse


def head_forward_online(qh, kh, vh, scale, causal, block_n=32):
    """Forward from per-key-block softmax summaries (all rows of one head).

    Section 3 of "When the Bottleneck Moved" computes attention one key block
    at a time, keeping per query row only a small summary of the keys seen so
    far instead of the score matrix.  Here the summary of a set of keys is a
    triple (m, l, a): m the row's largest score over the set, l the sum of
    exp(s - m) and a the sum of exp(s - m) * v_j over it.  The set's softmax
    output is then a / l and its log-sum-exp m + log l, whatever m is, as long
    as every term uses the same m.  Each key block's own triple is formed
    directly; two triples combine by moving both onto the larger of their
    maxima (a factor exp(m_old - m_max) on each sum).  Folding the blocks in
    order gives the result; it is an independent route to the numbers of
    ``head_forward`` and pins the block-by-block schedule of the kernels.
    """
    Lq, Lk = qh.shape[0], kh.shape[0]
    D = vh.shape[1]
    vis = visible_mask(Lq, Lk, causal)
    m = np.full(Lq, _NEG_INF)     # the empty set: no maximum, zero sums
    l = np.zeros(Lq)
    a = np.zeros((Lq, D))
    for j0 in range(0, Lk, block_n):
        j1 = min(Lk, j0 + block_n)
        s = np.where(vis[:, j0:j1], scale * (qh @ kh[j0:j1].T), _NEG_INF)
        # this block's own summary (a row that sees none of its keys has the
        # empty summary)
        mb = s.max(axis=1)
        eb = np.exp(s - np.where(np.isfinite(mb), mb, 0.0)[:, None])
        lb, ab = eb.sum(axis=1), eb @ vh[j0:j1]
        # combine the two summaries on the larger maximum
        top = np.maximum(m, mb)
        ref = np.where(np.isfinite(top), top, 0.0)
        w_run = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
        w_blk = np.where(np.isfinite(mb), np.exp(mb - ref), 0.0)
        m, l, a = top, w_run * l + w_blk * lb, w_run[:, None] * a + w_blk[:, None] * ab
    return a / l[:, None], m + np.log(l)


def head_backward(qh, kh, vh, doh, scale, causal, rows=None, key_rows=None, block=256, block_mask=None):
    """One query head's backward by explicit recomputation.

    Per block of query rows: S, P from the row's own log-sum-exp, O = P V,
    delta_i = sum_d dO_id O_id, dP = dO V^T, dS = P * (dP - delta),
    dQ = scale * dS K, and this head's contributions
    dK += scale * dS^T Q, dV += P^T dO.

    ``rows`` limits the query rows (dK/dV are then partial sums over those
    rows only).  ``key_rows`` limits which key rows get dK/dV (dQ is then
    not computed).  Returns a dict with o, lse, delta, dq (rows) and dk, dv
    ([len(key_rows) or Lk, D]).  With a block mask, a row that sees no key
    has P = 0: O = 0, LSE = -inf, dQ = 0 and no share in dK/dV.
    """
    Lq, Lk = qh.shape[0], kh.shape[0]
    rows = np.arange(Lq) if rows is None else np.asarray(rows)
    kcols = np.arange(Lk) if key_rows is None else np.asarray(key_rows)
    full_keys = key_rows is None
    n = rows.shape[0]
    D = qh.shape[1]
    out = {
        "o": np.empty((n, D)),
        "lse": np.empty(n),
        "delta": np.empty(n),
        "dq": np.empty((n, D)) if full_keys else None,
        "dk": np.zeros((kcols.shape[0], D)),
        "dv": np.zeros((kcols.shape[0], D)),
    }
    pos = 0
    for rb in _row_blocks(rows, block):
        nb = rb.shape[0]
        qb, dob = qh[rb], doh[rb]
        s = _scores(qb, kh, scale, visible_mask(Lq, Lk, causal, rb, block_mask))
        l = _lse(s, allow_empty=block_mask is not None)
        p = _probs(s, l)
        o = p @ vh
        dl = (dob * o).sum(axis=1)                      # delta = rowsum(dO * O)
        pk = p[:, kcols]
        dp = dob @ vh[kcols].T                          # dP = dO V^T
        ds = pk * (dp - dl[:, None])                    # dS (scale applied below)
        if full_keys:
            out["dq"][pos:pos + nb] = scale * (ds @ kh)  # dQ = scale * dS K
        out["dk"] += scale * (ds.T @ qb)                # dK += scale * dS^T Q
        out["dv"] += pk.T @ dob                         # dV += P^T dO
        out["o"][pos:pos + nb] = o
        out["lse"][pos:pos + nb] = l
        out["delta"][pos:pos + nb] = dl
        pos += nb
    return out


def _check(q, k, v):
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if (Bk, Dk) != (B, D) or v.shape != k.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    return B, Hq, Hkv, Lq, Lk, D, Hq // Hkv


def forward(q, k, v, scale, causal, block=256, block_mask=None):
    """Full forward over [B, Hq, Lq, D] / [B, Hkv, Lk, D] float64 arrays
    (one block mask, if any, for every batch and head)."""
    B, Hq, Hkv, Lq, Lk, D, G = _check(q, k, v)
    o = np.empty((B, Hq, Lq, D))
    lse = np.empty((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, g], v[b, g], scale, causal, block=block,
                                              block_mask=block_mask)
    return o, lse


def backward(q, k, v, do, scale, causal, block=256, block_mask=None):
    """Full backward; dK/dV of a key/value head sum over its query heads."""
    B, Hq, Hkv, Lq, Lk, D, G = _check(q, k, v)
    res = {
        "o": np.empty((B, Hq, Lq, D)),
        "lse": np.empty((B, Hq, Lq)),
        "delta": np.empty((B, Hq, Lq)),
        "dq": np.empty((B, Hq, Lq, D)),
        "dk": np.zeros((B, Hkv, Lk, D)),
        "dv": np.zeros((B, Hkv, Lk, D)),
    }
    for b in range(B):
        for h in range(Hq):
            g = h // G
            r = head_backward(q[b, h], k[b, g], v[b, g], do[b, h], scale, causal, block=block,
                              block_mask=block_mask)
            for name in ("o", "lse", "delta", "dq"):
                res[name][b, h] = r[name]
            res["dk"][b, g] += r["dk"]
            res["dv"][b, g] += r["dv"]
    return res


def delta(o, do):
    """delta[..., i] = sum_d dO[..., i, d] * O[..., i, d] in float64."""
    return (np.asarray(do, dtype=np.float64) * np.asarray(o, dtype=np.float64)).sum(axis=-1)
