"""fp64 CPU oracle for causal grouped-query attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library; the only module both sides use is ``fa_synth`` (seeded input bits).

What it computes is the plain definition of attention and of its gradient,
with the score matrix materialised (one block of query rows at a time, so
memory stays bounded), in float64:

* forward — page "When the Bottleneck Moved: From Fused Cross-Entropy to
  FlashAttention on MLX", section 3 (scores = scale * Q K^T plus mask,
  softmax, P V; the saved log-sum-exp per query row); also page
  "feat(attention): complete Flash Attention VJP implementation",
  Background (the two forward matmuls);
* backward — the same Background section of the VJP page (five matmuls per
  block pair: recomputed scores, dP = dO V^T, dS = scale * P * (dP - delta),
  dQ = dS K, dK = dS^T Q, dV = P^T dO) and section 3 of "When the Bottleneck
  Moved" (P recomputed from the saved log-sum-exp, delta_i = dO_i . O_i);
* grouped-query heads: query head h reads key/value head h // (Hq/Hkv)
  (contiguous groups; the pages name only the group factor);
* causal mask, bottom-right aligned: key j is visible to query i iff
  j <= i + (Lk - Lq) — page "Add a fused full-attention path for head_dim
  256 on NAX devices", Design, "Ragged causal inputs" (the query offset is
  taken from the true lengths).  Masked scores are -inf, so they get exactly
  zero probability;
* optional block-sparse mask — page "feat(attention): complete Flash
  Attention VJP implementation", "Sparse Block Masks": a uint8 entry per
  (query tile, key tile) pair, 0 = the pair is skipped; here tiles are 64
  query rows by 64 keys, one mask for all batches and heads.  A row left
  with no visible key gets O = 0, LSE = -inf and no gradient share (the
  pages do not say; this is the reading that skipping every tile of the row
  gives).

The log-sum-exp is returned in natural-log units.  Pins for every function
live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

from .attention import (  # noqa: F401
    MASK_BLOCK,
    bf16_bits_to_f64,
    f16_bits_to_f64,
    bits_to_f64,
    visible_mask,
    head_forward,
    head_forward_online,
    head_backward,
    forward,
    backward,
    delta,
)
