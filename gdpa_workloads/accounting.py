"""Algorithmic work and traffic of a workload (for throughput and roofline reporting only).

Model flops count the two (forward) or four (backward) matrix products per unmasked score entry
(2*d flops each): forward 4*d*E, backward 8*d*E, where E is the number of unmasked
(query, key, head) entries. The backward recompute of the scores is not credited.

Minimum bytes count each input read once and each output written once per pass, at the
storage width (bf16 = 2 B, fp32 = 4 B; the gate and the log-sum-exp are fp32).
"""

from __future__ import annotations

from typing import Dict

import numpy as np


def _allowed_keys_per_query(lq: int, lk: int, left: int, right: int) -> int:
    """Number of (i, j) pairs with 0<=i<lq, 0<=j<lk and i-left <= j <= i+right (-1 = unbounded)."""
    if lq == 0 or lk == 0:
        return 0
    i = np.arange(lq, dtype=np.int64)
    lo = np.zeros(lq, np.int64) if left < 0 else np.maximum(0, i - left)
    hi = np.full(lq, lk - 1, np.int64) if right < 0 else np.minimum(lk - 1, i + right)
    return int(np.maximum(0, hi - lo + 1).sum())


def group_work(group) -> Dict[str, float]:
    s = group.spec
    h, d = s.num_heads, s.head_dim
    left, right = s.window
    e = 0
    for lq, lk in zip(group.lengths_q.tolist(), group.lengths_kv.tolist()):
        e += _allowed_keys_per_query(lq, lk, left, right)
    e *= h
    esize = 2 if s.dtype == "bf16" else 4
    tq, tk = group.total_q, group.total_kv
    qrows = int(group.q.shape[0])  # = tq, or S rows of a shared query matrix
    softmax = s.act == "softmax"
    gate_b = 4 * tk * h if s.gate else 0
    lse_b = 4 * tq * h if softmax else 0
    # forward: read Q, K, V (+G); write O (+LSE)
    fwd_bytes = esize * ((qrows + tq) * h * d + 2 * tk * h * d) + gate_b + lse_b
    # backward: read Q, K, V, dO (+G; softmax also LSE); write dQ, dK, dV (+dG). The softmax row
    # term D_i = sum_j p_ij dp_ij is formed from P and dP in the kernel, so O is not read.
    bwd_bytes = esize * ((2 * qrows + tq) * h * d + 4 * tk * h * d) + 2 * gate_b + lse_b
    return {
        "entries": float(e),
        "fwd_flops": 4.0 * d * e,
        "bwd_flops": 8.0 * d * e,
        "fwd_bytes": float(fwd_bytes),
        "bwd_bytes": float(bwd_bytes),
    }


def workload_work(workload) -> Dict[str, float]:
    tot: Dict[str, float] = {}
    for g in workload.groups:
        for k, v in group_work(g).items():
            tot[k] = tot.get(k, 0.0) + v
    return tot
