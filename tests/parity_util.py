"""Helpers shared by the GPU parity tests: move seeded bf16 bits to the GPU,
run the library's three calls, and compare against the fp64 oracle with the
stated tolerances.

Tolerances (per output tensor):
  LSE            max |gpu - ref| <= 1e-3 (absolute, natural-log units)
  O              max |gpu - ref| <= 1e-2 * max |ref|
  dQ, dK, dV     max |gpu - ref| <= 2e-2 * max |ref|
The median elementwise relative error (over |ref| >= 1e-3 * max |ref|) and the
relative L2 error are reported alongside.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"lse": ("abs", 1e-3), "o": ("rel_max", 1e-2), "dq": ("rel_max", 2e-2),
       "dk": ("rel_max", 2e-2), "dv": ("rel_max", 2e-2), "delta": ("rel_max", 1e-2)}


def to_gpu(bits: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_library(q, k, v, do, scale, causal, backward=True, block_mask=None):
    """Run fa_fwd (+ fa_bwd_delta + fa_bwd) on GPU tensors; return GPU tensors.
    With a (GPU uint8) block mask the *_block_sparse calls are used."""
    import causal_gqa_flashattention_amd as fa
    if block_mask is None:
        o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    else:
        o, lse = fa.fa_fwd_block_sparse(q, k, v, block_mask, scale=scale, causal=causal)
    out = {"o": o, "lse": lse}
    if backward:
        delta = fa.fa_bwd_delta(o, do)
        if block_mask is None:
            dq, dk, dv = fa.fa_bwd(q, k, v, o, lse, delta, do, scale=scale, causal=causal)
        else:
            dq, dk, dv = fa.fa_bwd_block_sparse(q, k, v, o, lse, delta, do, block_mask,
                                                scale=scale, causal=causal)
        out.update(delta=delta, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def stats(got: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(got - ref)
    amax = float(np.abs(ref).max()) if ref.size else 0.0
    sel = (np.abs(ref) >= 1e-3 * amax) & (np.abs(ref) > 0)
    med = float(np.median(err[sel] / np.abs(ref[sel]))) if sel.any() else 0.0
    l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    return {"max_abs": float(err.max()) if err.size else 0.0, "max_ref": amax, "median_rel": med, "rel_l2": l2}


def check(name: str, got: np.ndarray, ref: np.ndarray, label: str = "", atol: float = 0.0) -> dict:
    """Assert the tolerance for `name`; `atol` is an absolute floor used only
    where the exact result is identically zero (degenerate cases)."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label} {name}: non-finite values"
    st = stats(got, ref)
    kind, tol = TOL[name]
    bound = tol if kind == "abs" else max(tol * st["max_ref"], atol)
    print(f"[parity] {label} {name}: max_abs={st['max_abs']:.3e} bound={bound:.3e} "
          f"median_rel={st['median_rel']:.2e} rel_l2={st['rel_l2']:.2e}", flush=True)
    assert st["max_abs"] <= bound, f"{label} {name}: {st['max_abs']:.4e} > {bound:.4e}"
    return st


def oracle_full(bits: dict, scale: float, causal: bool, backward=True, block_mask=None,
                dtype: str = "bf16") -> dict:
    q = oracle.bits_to_f64(bits["q"], dtype)
    k = oracle.bits_to_f64(bits["k"], dtype)
    v = oracle.bits_to_f64(bits["v"], dtype)
    if not backward:
        o, lse = oracle.forward(q, k, v, scale, causal, block_mask=block_mask)
        return {"o": o, "lse": lse}
    do = oracle.bits_to_f64(bits["do"], dtype)
    return oracle.backward(q, k, v, do, scale, causal, block_mask=block_mask)


def check_masked(name: str, got: np.ndarray, ref: np.ndarray, label: str = "", empty=None) -> dict:
    """`check` for block-masked results.  `empty` (bool over the sequence
    axis: query rows for o, lse, dq; keys for dk, dv) marks the rows that see
    no key / keys that no row sees: there the GPU must give exactly what the
    oracle gives (LSE = -inf, zeros); the tolerance of `check` applies to the
    rest."""
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    if name == "lse":
        e = np.isneginf(ref)
        assert np.array_equal(np.isneginf(got), e), f"{label} lse: -inf rows differ"
        if empty is not None:
            assert np.array_equal(e, np.broadcast_to(empty, e.shape)), f"{label}: oracle -inf rows"
        return check(name, got[~e], ref[~e], label) if (~e).any() else {}
    if empty is not None and np.any(empty):
        sel = np.broadcast_to(np.asarray(empty)[:, None], got.shape[-2:])
        sel = np.broadcast_to(sel, got.shape)
        assert np.all(ref[sel] == 0.0), f"{label} {name}: oracle not zero where nothing is seen"
        assert np.all(got[sel] == 0.0), f"{label} {name}: not zero where nothing is seen"
        print(f"[parity] {label} {name}: {int(np.sum(empty))} empty rows exactly zero", flush=True)
    return check(name, got, ref, label)
