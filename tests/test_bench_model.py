"""Pins of bench.py's accounting against numbers the pages print
(tests/golden/*, each file names its page and table)."""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [list(map(float, ln.split())) for ln in f if ln.strip() and not ln.startswith("#")]


def test_flop_model_reproduces_printed_throughput():
    for Lq, Lk, ms, tf in _rows("d256_forward_timings.txt"):
        _, fwd = bench.model_flops(1, 16, int(Lq), int(Lk), 256, causal=True)
        assert round(fwd / (ms * 1e-3) / 1e12, 1) == pytest.approx(tf, abs=0.05)


def test_training_shape_flops():
    # 8192-token training shape: 0.5498 TFLOP forward + 2.5x backward
    total, fwd = bench.model_flops(1, 32, 8192, 8192, 128, causal=True)
    assert fwd == 4 * 32 * 8192 * 8192 * 128 / 2
    assert total == pytest.approx(3.5 * fwd)
    assert round(total / 1e12, 4) == 1.9241


def test_unfused_score_matrix_size():
    for L, mb in _rows("unfused_score_matrix_mb.txt"):
        assert round(bench.unfused_score_bytes(32, int(L), 2) / 1e6) == pytest.approx(mb, abs=1)


@pytest.mark.parametrize("Lq,Lk,causal", [(7, 7, True), (5, 9, True), (1, 4, True), (6, 3, False), (0, 5, True)])
def test_visible_pairs_brute_force(Lq, Lk, causal):
    want = sum(1 for i in range(Lq) for j in range(Lk) if (not causal) or j <= i + (Lk - Lq))
    assert bench.visible_pairs(Lq, Lk, causal) == want


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_executed_mfma_counts():
    """The kernels' analytic MFMA counts: exactly the algorithmic FLOPs / 32768
    for dense shapes whose lengths are whole tiles; a few percent above it for
    causal ones (diagonal tiles run whole); never below."""
    import bench
    from fa_synth import WORKLOADS
    for name in ("dense4k_d64", "dense4k_d96", "train8k", "d256_train8k", "long23k"):
        w = WORKLOADS[name]
        e = bench.executed_mfma(w)
        work = bench.kernel_work(w, bench.visible_pairs(w.Lq, w.Lk, w.causal))
        for k in ("fwd", "dq", "dkv"):
            ratio = e[k] * 32768 / work[k]
            if not w.causal:
                assert ratio == 1.0, (name, k, ratio)
            else:
                assert 1.0 <= ratio < 1.05, (name, k, ratio)


def test_visible_pairs_under_a_block_mask():
    """The bench's pair count under a block mask is the number of True entries
    of the oracle's visibility matrix, and reduces to the plain count for an
    all-ones mask."""
    import numpy as np

    import bench
    import oracle
    from fa_synth import random_block_mask, window_block_mask
    for Lq, Lk, causal, m in [
        (300, 300, True, random_block_mask(300, 300, 0.5, 1)),
        (200, 333, True, window_block_mask(200, 333, 100, 1)),
        (333, 200, False, random_block_mask(333, 200, 0.3, 2)),
        (257, 257, True, np.ones((5, 5), np.uint8)),
    ]:
        want = int(oracle.visible_mask(Lq, Lk, causal, block_mask=m).sum())
        assert bench.visible_pairs_masked(Lq, Lk, causal, m) == want
    assert bench.visible_pairs_masked(257, 257, True, np.ones((5, 5), np.uint8)) == bench.visible_pairs(257, 257, True)
