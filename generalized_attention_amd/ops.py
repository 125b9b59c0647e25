"""Marshal torch device tensors into the libgdpa C ABI (no computation happens here).

torch allocates outputs and the workspace and supplies the current HIP stream; the library's
kernels do all of the operator's work.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import torch

from . import _lib

_ACTS = {"gelu": _lib.GDPA_ACT_GELU, "silu": _lib.GDPA_ACT_SILU, "softmax": _lib.GDPA_ACT_SOFTMAX}
_DTYPES = {torch.bfloat16: _lib.GDPA_DTYPE_BF16, torch.float32: _lib.GDPA_DTYPE_FP32}


@dataclasses.dataclass
class GroupArgs:
    """One GDPA problem: device tensors plus the shape hints the library needs."""

    q: torch.Tensor            # [total_q, H, d]; with shared_q one [S, H, d] matrix
    k: torch.Tensor            # [total_kv, H, d]
    v: torch.Tensor            # [total_kv, H, d]
    q_offsets: torch.Tensor    # int32 [B+1] on the device
    kv_offsets: torch.Tensor   # int32 [B+1] on the device
    act: str
    scale: float
    max_seqlen_q: int
    max_seqlen_kv: int
    window: Tuple[int, int] = (-1, -1)
    g: Optional[torch.Tensor] = None  # float32 [total_kv, H]
    self_attention: bool = False
    planned: bool = False  # the workspace holds a gdpa_plan() work list for this shape
    head_acts: Optional[torch.Tensor] = None  # int32 [H] on the device: activation per head
    shared_q: bool = False  # q is one query matrix shared by every sequence (rows of o: total_q)
    total_q: Optional[int] = None  # rows of o / lse / dout (default: rows of q)
    fp32_out: bool = False  # bf16 problem with float32 o, dq, dk, dv
    validate: bool = False  # enqueue the offsets-validation kernel first (GDPA_FLAG_VALIDATE)
    split_operands: bool = False  # P / dS as high + low bf16 pairs in every backward product

    @property
    def out_dtype(self) -> torch.dtype:
        return torch.float32 if self.fp32_out else self.q.dtype

    @property
    def rows(self) -> int:
        return self.q.shape[0] if self.total_q is None else int(self.total_q)

    @property
    def may_softmax(self) -> bool:
        return self.act == "softmax" or self.head_acts is not None

    def problem(self) -> _lib.gdpa_problem:
        p = _lib.gdpa_problem()
        p.num_seqs = self.q_offsets.numel() - 1
        p.num_heads = self.q.shape[1]
        p.head_dim = self.q.shape[2]
        p.dtype = _DTYPES[self.q.dtype]
        p.act = _ACTS[self.act]
        p.scale = float(self.scale)
        p.window_left, p.window_right = int(self.window[0]), int(self.window[1])
        p.total_q = self.rows
        p.total_kv = self.k.shape[0]
        p.max_seqlen_q = int(self.max_seqlen_q)
        p.max_seqlen_kv = int(self.max_seqlen_kv)
        p.self_attention = 1 if self.self_attention else 0
        p.flags = ((_lib.GDPA_FLAG_PLANNED if self.planned else 0) | (_lib.GDPA_FLAG_SHARED_Q if self.shared_q else 0)
                   | (_lib.GDPA_FLAG_FP32_OUT if self.fp32_out else 0)
                   | (_lib.GDPA_FLAG_VALIDATE if self.validate else 0)
                   | (_lib.GDPA_FLAG_SPLIT_OPERANDS if self.split_operands else 0))
        p.q_offsets = self.q_offsets.data_ptr()
        p.kv_offsets = self.kv_offsets.data_ptr()
        p.head_acts = 0 if self.head_acts is None else self.head_acts.data_ptr()
        return p


def make_group(q, k, v, q_offsets, kv_offsets, *, act, scale: float, window=(-1, -1), g=None,
               self_attention: Optional[bool] = None, lengths_q=None, lengths_kv=None,
               shared_q: bool = False, fp32_out: bool = False) -> GroupArgs:
    """Build GroupArgs from device tensors. Offsets may be given on the host (int64 numpy/torch)
    or the device; the max lengths come from host lengths when given (no device sync).
    act: an activation name, or a sequence with one name per head. shared_q: q is one [S, H, d]
    query matrix whose row i is query row i of every sequence (each sequence has <= S rows).
    fp32_out: a bf16 problem writes o, dq, dk, dv in float32."""
    dev = q.device
    head_acts = None
    if not isinstance(act, str):
        names = list(act)
        if len(names) != q.shape[1]:
            raise ValueError("one activation per head expected")
        head_acts = torch.tensor([_ACTS[a] for a in names], dtype=torch.int32).to(dev)
        act = names[0]

    def dev_off(o):
        t = torch.as_tensor(o)
        return t.to(device=dev, dtype=torch.int32).contiguous()

    qo, ko = dev_off(q_offsets), dev_off(kv_offsets)
    if lengths_q is None:
        lq = torch.as_tensor(q_offsets).cpu().long()
        lengths_q = (lq[1:] - lq[:-1]).tolist()
    if lengths_kv is None:
        lk = torch.as_tensor(kv_offsets).cpu().long()
        lengths_kv = (lk[1:] - lk[:-1]).tolist()
    if self_attention is None:
        self_attention = window != (-1, -1)
    max_q = q.shape[0] if shared_q else int(max(lengths_q, default=0))
    return GroupArgs(q=q, k=k, v=v, q_offsets=qo, kv_offsets=ko, act=act, scale=scale,
                     max_seqlen_q=max_q, max_seqlen_kv=int(max(lengths_kv, default=0)),
                     window=tuple(window), g=g, self_attention=bool(self_attention), head_acts=head_acts,
                     shared_q=bool(shared_q), total_q=int(sum(lengths_q)) if shared_q else None,
                     fp32_out=bool(fp32_out))


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def workspace(groups: Sequence[GroupArgs], pass_: int) -> torch.Tensor:
    n = _lib.gdpa_workspace_size([g.problem() for g in groups], pass_)
    if n == 0:
        raise _lib.GdpaError(_lib.GDPA_ERR_INVALID_ARGUMENT, "gdpa_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=groups[0].q.device)


def device_error(ws: torch.Tensor) -> int:
    """The device error word of a workspace after the calls that used it (GDPA_DEVICE_ERR_* bits;
    0 when every item's offsets passed). Synchronizes with the current stream."""
    off = _lib.GDPA_WS_ERROR_OFFSET
    return int(ws[off:off + 4].view(torch.int32).item())


def gdpa_plan(groups: Sequence[GroupArgs], ws: torch.Tensor) -> None:
    """Build the longest-first work list of `groups` into `ws` (reused by planned calls)."""
    rc = _lib.gdpa_plan([g.problem() for g in groups], ws.data_ptr(), ws.numel(), _stream(groups[0].q.device))
    if rc != _lib.GDPA_OK:
        raise _lib.GdpaError(rc, "gdpa_plan")


def _fwd_tensors(grp: GroupArgs, o, lse) -> _lib.gdpa_tensors:
    t = _lib.gdpa_tensors()
    t.q, t.k, t.v, t.g = _ptr(grp.q), _ptr(grp.k), _ptr(grp.v), _ptr(grp.g)
    t.o, t.lse = _ptr(o), _ptr(lse)
    return t


def _alloc_fwd(grp: GroupArgs):
    o = torch.empty((grp.rows,) + tuple(grp.q.shape[1:]), dtype=grp.out_dtype, device=grp.q.device)
    lse = None
    if grp.may_softmax:
        lse = torch.empty(grp.rows, grp.q.shape[1], dtype=torch.float32, device=grp.q.device)
    return o, lse


def gdpa_fwd(grp: GroupArgs, o=None, lse=None, ws=None):
    """Forward. Returns (o, lse); lse is None unless some head uses softmax."""
    if o is None:
        o, lse = _alloc_fwd(grp)
    if ws is None:
        ws = workspace([grp], 0)
    rc = _lib.gdpa_fwd(grp.problem(), _fwd_tensors(grp, o, lse), ws.data_ptr(), ws.numel(), _stream(grp.q.device))
    if rc != _lib.GDPA_OK:
        raise _lib.GdpaError(rc, "gdpa_fwd")
    return o, lse


def _bwd_tensors(grp: GroupArgs, dout, o, lse, dq, dk, dv, dg) -> _lib.gdpa_tensors:
    t = _lib.gdpa_tensors()
    t.q, t.k, t.v, t.g = _ptr(grp.q), _ptr(grp.k), _ptr(grp.v), _ptr(grp.g)
    t.o, t.lse, t.dout = _ptr(o), _ptr(lse), _ptr(dout)
    t.dq, t.dk, t.dv, t.dg = _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg)
    return t


def _alloc_bwd(grp: GroupArgs, want_dg: bool):
    dt = grp.out_dtype
    dq, dk, dv = (torch.empty_like(grp.q, dtype=dt), torch.empty_like(grp.k, dtype=dt),
                  torch.empty_like(grp.v, dtype=dt))
    dg = torch.empty_like(grp.g) if (want_dg and grp.g is not None) else None
    return dq, dk, dv, dg


def gdpa_bwd(grp: GroupArgs, dout, o=None, lse=None, want_dg: bool = False, out=None, ws=None) -> Dict[str, torch.Tensor]:
    """Backward for upstream gradient dout. The softmax form needs the forward's o and lse."""
    dq, dk, dv, dg = out if out is not None else _alloc_bwd(grp, want_dg)
    if ws is None:
        ws = workspace([grp], 1)
    rc = _lib.gdpa_bwd(grp.problem(), _bwd_tensors(grp, dout, o, lse, dq, dk, dv, dg), ws.data_ptr(), ws.numel(),
                       _stream(grp.q.device))
    if rc != _lib.GDPA_OK:
        raise _lib.GdpaError(rc, "gdpa_bwd")
    res = {"dq": dq, "dk": dk, "dv": dv}
    if dg is not None:
        res["dg"] = dg
    return res


def gdpa_fwd_grouped(groups: List[GroupArgs], outs=None, ws=None):
    """One launch over several problems. Returns a list of (o, lse)."""
    outs = outs if outs is not None else [_alloc_fwd(g) for g in groups]
    if ws is None:
        ws = workspace(groups, 0)
    rc = _lib.gdpa_fwd_grouped([g.problem() for g in groups],
                               [_fwd_tensors(g, o, l) for g, (o, l) in zip(groups, outs)],
                               ws.data_ptr(), ws.numel(), _stream(groups[0].q.device))
    if rc != _lib.GDPA_OK:
        raise _lib.GdpaError(rc, "gdpa_fwd_grouped")
    return outs


def gdpa_bwd_grouped(groups: List[GroupArgs], douts, fwd_outs=None, want_dg: bool = False, outs=None, ws=None):
    """One launch over several problems. Returns a list of gradient dicts."""
    outs = outs if outs is not None else [_alloc_bwd(g, want_dg) for g in groups]
    fwd_outs = fwd_outs if fwd_outs is not None else [(None, None)] * len(groups)
    if ws is None:
        ws = workspace(groups, 1)
    tens = [_bwd_tensors(g, do, o, l, *out) for g, do, (o, l), out in zip(groups, douts, fwd_outs, outs)]
    rc = _lib.gdpa_bwd_grouped([g.problem() for g in groups], tens, ws.data_ptr(), ws.numel(),
                               _stream(groups[0].q.device))
    if rc != _lib.GDPA_OK:
        raise _lib.GdpaError(rc, "gdpa_bwd_grouped")
    res = []
    for out in outs:
        d = {"dq": out[0], "dk": out[1], "dv": out[2]}
        if out[3] is not None:
            d["dg"] = out[3]
        res.append(d)
    return res
