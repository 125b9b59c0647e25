"""Seeded input recipe for the six GDPA workloads and their reduced parity variants.

Draw order is part of the recipe: ``numpy.random.default_rng(seed)`` (PCG64), lengths first,
then the tensors in the order each builder lists them. Normal draws are made in float64 (the
context-to-weight maps in float32) and rounded once to the compute dtype with torch's
round-to-nearest-even cast. Both the oracle and the GPU receive exactly those rounded values.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

ACTS = ("gelu", "silu", "softmax")


@dataclasses.dataclass(frozen=True)
class GroupSpec:
    """Shape and operator settings of one event group (one GDPA problem)."""

    name: str
    num_seqs: int            # B
    num_heads: int           # H
    head_dim: int            # d
    len_range: Tuple[int, int]  # inclusive integer range of the jagged lengths L_b
    keys_per_seq: Optional[int]  # n for the cross-attention (PFFN) form; None = self-attention
    act: str                 # "gelu" | "silu" | "softmax"
    scale: float
    window: Tuple[int, int] = (-1, -1)  # (left, right); -1 = unbounded side
    gate: bool = False       # per-head, per-key gate G of the gated-softmax form
    dtype: str = "bf16"      # "bf16" | "fp32"
    shared_q: bool = False   # one [S, H, d] query matrix shared by every sequence (seed pooling)


@dataclasses.dataclass
class Group:
    """One group's inputs, already rounded to the compute dtype (torch CPU tensors)."""

    spec: GroupSpec
    lengths_q: np.ndarray    # int64 [B]
    lengths_kv: np.ndarray   # int64 [B]
    q_offsets: np.ndarray    # int64 [B+1]
    kv_offsets: np.ndarray   # int64 [B+1]
    q: torch.Tensor          # [total_q, H, d] (shared_q: [S, H, d])
    k: torch.Tensor          # [total_kv, H, d]
    v: torch.Tensor          # [total_kv, H, d]
    g: Optional[torch.Tensor]  # float32 [total_kv, H] or None
    dout: torch.Tensor       # [total_q, H, d]

    @property
    def total_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def total_kv(self) -> int:
        return int(self.kv_offsets[-1])

    def subset(self, seqs) -> "Group":
        """Return a new group holding only the listed sequences (in the given order).

        Sequences are independent in every output, so a subset is the way to sample outputs
        of a large workload for a slow reference."""
        seqs = [int(s) for s in seqs]
        qo, ko = self.q_offsets, self.kv_offsets
        qi = np.concatenate([np.arange(qo[s], qo[s + 1]) for s in seqs]) if seqs else np.zeros(0, np.int64)
        ki = np.concatenate([np.arange(ko[s], ko[s + 1]) for s in seqs]) if seqs else np.zeros(0, np.int64)
        lq = self.lengths_q[seqs] if seqs else np.zeros(0, np.int64)
        lk = self.lengths_kv[seqs] if seqs else np.zeros(0, np.int64)
        qit = torch.from_numpy(qi.astype(np.int64))
        kit = torch.from_numpy(ki.astype(np.int64))
        spec = dataclasses.replace(self.spec, num_seqs=len(seqs))
        return Group(
            spec=spec,
            lengths_q=lq.astype(np.int64),
            lengths_kv=lk.astype(np.int64),
            q_offsets=_offsets(lq),
            kv_offsets=_offsets(lk),
            q=self.q if self.spec.shared_q else self.q.index_select(0, qit),
            k=self.k.index_select(0, kit),
            v=self.v.index_select(0, kit),
            g=None if self.g is None else self.g.index_select(0, kit),
            dout=self.dout.index_select(0, qit),
        )


@dataclasses.dataclass
class Workload:
    name: str
    description: str
    groups: List[Group]
    passes: Tuple[str, ...]  # ("fwd",) or ("fwd", "bwd")
    seed: int


def _offsets(lengths: np.ndarray) -> np.ndarray:
    off = np.zeros(len(lengths) + 1, dtype=np.int64)
    if len(lengths):
        off[1:] = np.cumsum(lengths)
    return off


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "fp32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def widen(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact widening of a rounded tensor to float64 numpy (for the oracle)."""
    if t is None:
        return None
    return t.to(torch.float64).numpy()


def _lengths(rng, b: int, lo_hi: Tuple[int, int]) -> np.ndarray:
    lo, hi = lo_hi
    return rng.integers(lo, hi + 1, size=b).astype(np.int64)


# ----------------------------------------------------------------------------------------------
# Workload registry. Shapes follow the workload descriptions of the Kunlun review and README;
# where they leave a value open (dtype, score scale) the recipe takes one reading: bf16 for the
# training shapes, scale 1/L_max for the pointwise forms, 1/sqrt(d) for the softmax form.
# ----------------------------------------------------------------------------------------------
CONFIGS: Dict[str, str] = {
    "tiny_fp32": "tiny PFFN-form GDPA fp32: B=4, L in [1,64], H=2, d=32, n=64, GELU, fwd",
    "pffn_fwd": "PFFN-form GDPA bf16 fwd: B=256, L in [100,1000], H=4, d=64, n=256 generated from a "
            "512-dim context by a random linear map, SiLU",
    "pffn_train": "pffn_fwd shapes, bf16 fwd+bwd (dQ, dK, dV), upstream gradient N(0,1)",
    "causal_gated": "gated softmax self-attention bf16 fwd+bwd: B=128, L in [200,2000], H=8, d=64, "
            "scale 1/sqrt(d), log sigmoid gate G~N(0,1), causal sliding window 128",
    "grouped10": "10 event groups in one launch, bf16 fwd+bwd: each B=64, L in [100,1000], n=32; "
            "groups 0-4 H=8 d=128, groups 5-9 H=2 d=32; GELU",
    "seed_pool": "seed-query pooling (PMA / hierarchical seed pooling as GDPA) bf16 fwd+bwd: S=256 "
            "learnable seed queries shared by B=256 sequences, L in [100,1000] keys each, H=4, d=64, "
            "softmax, scale 1/sqrt(d); dQ summed over the sequences",
}


def _pffn_plain(rng, spec: GroupSpec, lengths: np.ndarray, std: float) -> Group:
    """Q, K, V, dO with independent N(0, std^2) entries (draw order: Q, K, V, dO)."""
    b, h, d, n = spec.num_seqs, spec.num_heads, spec.head_dim, spec.keys_per_seq
    lk = np.full(b, n, dtype=np.int64)
    t = int(lengths.sum())
    q = rng.standard_normal((t, h, d)) * std
    k = rng.standard_normal((b * n, h, d)) * std
    v = rng.standard_normal((b * n, h, d)) * std
    do = rng.standard_normal((t, h, d))
    return Group(spec, lengths, lk, _offsets(lengths), _offsets(lk), _cast(q, spec.dtype),
                 _cast(k, spec.dtype), _cast(v, spec.dtype), None, _cast(do, spec.dtype))


def _pffn_context(rng, spec: GroupSpec, lengths: np.ndarray, ctx_dim: int) -> Group:
    """K/V generated per sample from a context vector by a random linear map.

    Draw order: Q [T,H,d] ~ N(0,1); context c [B, ctx] ~ N(0,1); maps M_K, M_V
    [ctx, n*H*d] ~ N(0, 1/ctx) drawn in float32; K_b = reshape(c_b M_K, [n, H, d]) (V alike);
    dO [T,H,d] ~ N(0,1). With map variance 1/ctx the generated entries are ~N(0,1)."""
    b, h, d, n = spec.num_seqs, spec.num_heads, spec.head_dim, spec.keys_per_seq
    t = int(lengths.sum())
    q = rng.standard_normal((t, h, d))
    c = rng.standard_normal((b, ctx_dim)).astype(np.float32)
    m_k = (rng.standard_normal((ctx_dim, n * h * d), dtype=np.float32) / np.float32(math.sqrt(ctx_dim)))
    m_v = (rng.standard_normal((ctx_dim, n * h * d), dtype=np.float32) / np.float32(math.sqrt(ctx_dim)))
    k = (torch.from_numpy(c) @ torch.from_numpy(m_k)).reshape(b * n, h, d)
    v = (torch.from_numpy(c) @ torch.from_numpy(m_v)).reshape(b * n, h, d)
    do = rng.standard_normal((t, h, d))
    lk = np.full(b, n, dtype=np.int64)
    cast = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
    return Group(spec, lengths, lk, _offsets(lengths), _offsets(lk), _cast(q, spec.dtype),
                 k.to(cast).contiguous(), v.to(cast).contiguous(), None, _cast(do, spec.dtype))


def _self_attention(rng, spec: GroupSpec, lengths: np.ndarray) -> Group:
    """Self-attention: Q, K, V [T,H,d] ~ N(0,1); G [T,H] ~ N(0,1) fp32 (if gated); dO ~ N(0,1)."""
    h, d = spec.num_heads, spec.head_dim
    t = int(lengths.sum())
    q = rng.standard_normal((t, h, d))
    k = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    g = rng.standard_normal((t, h)) if spec.gate else None
    do = rng.standard_normal((t, h, d))
    off = _offsets(lengths)
    return Group(spec, lengths, lengths.copy(), off, off.copy(), _cast(q, spec.dtype),
                 _cast(k, spec.dtype), _cast(v, spec.dtype),
                 None if g is None else torch.from_numpy(g).to(torch.float32),
                 _cast(do, spec.dtype))


def _seed_pool(rng, spec: GroupSpec, lengths: np.ndarray, seeds: int) -> Group:
    """Shared seed queries over jagged sequences. Draw order: seed queries E [S,H,d] ~ N(0,1);
    sequence keys and values K, V [T,H,d] ~ N(0,1); dO [B*S,H,d] ~ N(0,1). Every sequence has
    S query rows (its pooled outputs) and L_b keys."""
    b, h, d = spec.num_seqs, spec.num_heads, spec.head_dim
    t = int(lengths.sum())
    q = rng.standard_normal((seeds, h, d))
    k = rng.standard_normal((t, h, d))
    v = rng.standard_normal((t, h, d))
    do = rng.standard_normal((b * seeds, h, d))
    lq = np.full(b, seeds, dtype=np.int64)
    return Group(spec, lq, lengths, _offsets(lq), _offsets(lengths), _cast(q, spec.dtype),
                 _cast(k, spec.dtype), _cast(v, spec.dtype), None, _cast(do, spec.dtype))


def make_workload(name: str, seed: int = 0, *, num_seqs: Optional[int] = None,
                  len_range: Optional[Tuple[int, int]] = None, scale: Optional[float] = None,
                  act: Optional[str] = None, ctx_dim: int = 512,
                  window: Optional[Tuple[int, int]] = None,
                  lengths: Optional[List[int]] = None, keys: Optional[int] = None,
                  seeds: Optional[int] = None) -> Workload:
    """Build a workload by config name.

    The keyword overrides shrink a config for parity tests (fewer sequences, shorter lengths)
    or change the score scale / activation / window while keeping the recipe's draw order.
    ``lengths`` replaces the length draw entirely (edge cases: zeros, ones, tile +- 1); ``keys``
    replaces the PFFN key count n and ``seeds`` the seed-query count S."""
    rng = np.random.default_rng(seed)

    def lens(b, lr):
        if lengths is not None:
            return np.asarray(lengths, dtype=np.int64)
        return _lengths(rng, b, lr)

    if name == "tiny_fp32":
        b = num_seqs or 4
        spec = GroupSpec("tiny_fp32", b, 2, 32, len_range or (1, 64), 64, act or "gelu",
                         1.0 / 64 if scale is None else scale, dtype="fp32")
        L = lens(b, spec.len_range)
        grp = _pffn_plain(rng, dataclasses.replace(spec, num_seqs=len(L)), L, 1.0 / math.sqrt(32))
        return Workload(name, CONFIGS[name], [grp], ("fwd",), seed)
    if name in ("pffn_fwd", "pffn_train"):
        b = num_seqs or 256
        spec = GroupSpec(name, b, 4, 64, len_range or (100, 1000), keys or 256, act or "silu",
                         1.0 / 1000 if scale is None else scale)
        L = lens(b, spec.len_range)
        grp = _pffn_context(rng, dataclasses.replace(spec, num_seqs=len(L)), L, ctx_dim)
        passes = ("fwd",) if name == "pffn_fwd" else ("fwd", "bwd")
        return Workload(name, CONFIGS[name], [grp], passes, seed)
    if name == "causal_gated":
        b = num_seqs or 128
        spec = GroupSpec("causal_gated", b, 8, 64, len_range or (200, 2000), None, act or "softmax",
                         1.0 / 8 if scale is None else scale,
                         window=(127, 0) if window is None else window, gate=True)
        L = lens(b, spec.len_range)
        grp = _self_attention(rng, dataclasses.replace(spec, num_seqs=len(L)), L)
        return Workload(name, CONFIGS[name], [grp], ("fwd", "bwd"), seed)
    if name == "grouped10":
        b = num_seqs or 64
        lr = len_range or (100, 1000)
        if lengths is not None:
            all_l = np.asarray(lengths, dtype=np.int64).reshape(10, -1)
        else:
            all_l = _lengths(rng, 10 * b, lr).reshape(10, b)
        groups = []
        for e in range(10):
            h, d = (8, 128) if e < 5 else (2, 32)
            spec = GroupSpec(f"grouped10.g{e}", all_l.shape[1], h, d, lr, 32, act or "gelu",
                             1.0 / 1000 if scale is None else scale)
            groups.append(_pffn_plain(rng, spec, all_l[e], 1.0))
        return Workload(name, CONFIGS[name], groups, ("fwd", "bwd"), seed)
    if name == "seed_pool":
        b = num_seqs or 256
        spec = GroupSpec("seed_pool", b, 4, 64, len_range or (100, 1000), None, act or "softmax",
                         1.0 / 8 if scale is None else scale, shared_q=True)
        L = lens(b, spec.len_range)
        grp = _seed_pool(rng, dataclasses.replace(spec, num_seqs=len(L)), L, seeds or 256)
        return Workload(name, CONFIGS[name], [grp], ("fwd", "bwd"), seed)
    raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
