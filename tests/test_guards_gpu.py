"""GPU checks of the boundary's device-side guards (through the C ABI).

Each case hands the library offsets or hints that break a documented precondition while keeping
every kernel in bounds: an item whose offsets fail its own check returns before touching any
tensor, and the work-list builder clamps its bucket index. What is checked:
  * the device error word (workspace header) reports the violation;
  * a refused item writes nothing (its outputs keep the NaN they were filled with);
  * every other item is computed as usual (compared with the fp64 oracle);
  * with the debug validation (GDPA_FLAG_VALIDATE, or GDPA_DEBUG=1), no output is touched at all.
"""

from __future__ import annotations

import dataclasses
import os

import numpy as np
import pytest
import torch

import oracle
from gdpa_workloads import make_workload
from gpu_harness import check, device_group, rows_of, to64

import generalized_attention_amd as ga
from generalized_attention_amd import _lib

pytestmark = pytest.mark.gpu

E_OFF, E_LEN = _lib.GDPA_DEVICE_ERR_OFFSETS, _lib.GDPA_DEVICE_ERR_LENGTH


def _nan_outputs(dev, want_dg=False):
    o, lse = ga.ops._alloc_fwd(dev)
    o.fill_(float("nan"))
    if lse is not None:
        lse.fill_(float("nan"))
    grads = ga.ops._alloc_bwd(dev, want_dg=want_dg)
    for t in grads:
        if t is not None:
            t.fill_(float("nan"))
    return (o, lse), grads


def _run(dev, dout, fwd_out, grads):
    """Forward and backward into the given outputs; returns the error word after each pass."""
    ws0 = ga.workspace([dev], 0)
    ga.gdpa_fwd(dev, o=fwd_out[0], lse=fwd_out[1], ws=ws0)
    e0 = ga.device_error(ws0)
    ws1 = ga.workspace([dev], 1)
    ga.gdpa_bwd(dev, dout, o=fwd_out[0], lse=fwd_out[1], out=grads, ws=ws1)
    e1 = ga.device_error(ws1)
    return e0, e1


def test_clean_calls_leave_no_error():
    w = make_workload("pffn_train", 81, num_seqs=5, len_range=(1, 300))
    g = w.groups[0]
    dev = device_group(g)
    fwd_out, grads = _nan_outputs(dev)
    print("[gpu] guard: clean call", flush=True)
    e0, e1 = _run(dev, g.dout.to("cuda:0"), fwd_out, grads)
    assert (e0, e1) == (0, 0)


def test_understated_key_hint_refuses_the_long_item():
    """max_seqlen_kv says 256 while one sample has 300 keys: the forward launch is the
    resident-keys build (at most 256 keys per item at d = 64) and the backward reserved no key-chunk
    rows, so both refuse that sample's items (LENGTH); the other samples are computed."""
    w = make_workload("pffn_train", 82, num_seqs=4, len_range=(1, 300), keys=256, ctx_dim=64)
    g = w.groups[0]
    # give sample 2 another 44 keys: rebuild K / V with the extra rows appended to that sample
    extra = 44
    ko = g.kv_offsets.copy()
    rows = [np.arange(ko[b], ko[b + 1]) for b in range(4)]
    rng = np.random.default_rng(5)
    add_k = torch.from_numpy(rng.standard_normal((extra, 4, 64))).to(torch.bfloat16)
    add_v = torch.from_numpy(rng.standard_normal((extra, 4, 64))).to(torch.bfloat16)
    ks, vs = [], []
    for b in range(4):
        ks.append(g.k[rows[b]])
        vs.append(g.v[rows[b]])
        if b == 2:
            ks.append(add_k)
            vs.append(add_v)
    g.k, g.v = torch.cat(ks).contiguous(), torch.cat(vs).contiguous()
    g.lengths_kv = g.lengths_kv.copy()
    g.lengths_kv[2] += extra
    g.kv_offsets = np.concatenate([[0], np.cumsum(g.lengths_kv)]).astype(np.int64)
    dev = device_group(g)
    assert dev.max_seqlen_kv == 300
    dev = dataclasses.replace(dev, max_seqlen_kv=256)  # the understated hint
    fwd_out, grads = _nan_outputs(dev)
    print("[gpu] guard: understated max_seqlen_kv", flush=True)
    e0, e1 = _run(dev, g.dout.to("cuda:0"), fwd_out, grads)
    assert e0 == E_LEN and e1 == E_LEN
    bad_q = rows_of(g.q_offsets, [2])
    bad_k = rows_of(g.kv_offsets, [2])
    assert torch.isnan(fwd_out[0][bad_q]).all()
    for t, r in ((grads[0], bad_q), (grads[1], bad_k), (grads[2], bad_k)):
        assert torch.isnan(t[r]).all()
    good = [0, 1, 3]
    sub = g.subset(good)
    ref = oracle.group_fwd(sub)
    rb = oracle.group_bwd(sub)
    qr, kr = rows_of(g.q_offsets, good), rows_of(g.kv_offsets, good)
    check("bf16", to64(fwd_out[0])[qr], ref["o"], "O of the other samples")
    for name, t, r in (("dq", grads[0], qr), ("dk", grads[1], kr), ("dv", grads[2], kr)):
        check("bf16", to64(t)[r], rb[name], name + " of the other samples")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decreasing_offsets_refuse_their_item(dtype):
    """Query offsets [0, 50, 40] over 100 rows: the second sequence's range decreases (OFFSETS)
    and is refused; the first is computed."""
    name = "pffn_train" if dtype == "bf16" else "tiny_fp32"
    w = make_workload(name, 83, lengths=[50, 50], keys=64) if dtype == "bf16" else make_workload(name, 83, lengths=[50, 50])
    g = w.groups[0]
    dev = device_group(g)
    bad = torch.tensor([0, 50, 40], dtype=torch.int32, device="cuda:0")
    dev = dataclasses.replace(dev, q_offsets=bad)
    fwd_out, _ = _nan_outputs(dev)
    print(f"[gpu] guard: decreasing offsets ({dtype})", flush=True)
    ws = ga.workspace([dev], 0)
    ga.gdpa_fwd(dev, o=fwd_out[0], lse=fwd_out[1], ws=ws)
    assert ga.device_error(ws) & E_OFF
    o = fwd_out[0]
    assert torch.isnan(o[50:]).all()  # rows no accepted item owns
    ref = oracle.group_fwd(g.subset([0]))
    check(dtype, to64(o[:50]), ref["o"], "O of the first sequence")


@pytest.mark.parametrize("how", ["flag", "env"])
def test_debug_validation_leaves_outputs_untouched(how, monkeypatch):
    """The validation kernel finds the understated max_seqlen_q (a sequence of 290 rows against a
    hint of 200) and the main kernels then return at once: every output keeps its NaN, in both
    passes; valid offsets validate clean."""
    w = make_workload("pffn_train", 84, lengths=[290, 10, 100], keys=64)
    g = w.groups[0]
    dev = device_group(g)
    dout = g.dout.to("cuda:0")
    if how == "flag":
        good = dataclasses.replace(dev, validate=True)
    else:
        monkeypatch.setenv("GDPA_DEBUG", "1")
        good = dev
    fwd_out, grads = _nan_outputs(good)
    print(f"[gpu] guard: debug validation ({how}), valid offsets", flush=True)
    assert _run(good, dout, fwd_out, grads) == (0, 0)
    assert not torch.isnan(fwd_out[0]).any() and not any(torch.isnan(t).any() for t in grads[:3])
    bad = dataclasses.replace(good, max_seqlen_q=200)
    fwd_out, grads = _nan_outputs(bad)
    print(f"[gpu] guard: debug validation ({how}), understated max_seqlen_q", flush=True)
    e0, e1 = _run(bad, dout, fwd_out, grads)
    assert e0 == E_LEN and e1 == E_LEN
    assert torch.isnan(fwd_out[0]).all()
    for t in grads[:3]:
        assert torch.isnan(t).all()


def test_planned_call_with_another_split_is_refused():
    """A work list that gdpa_plan built with a 24-key group in the short-key class, used by a
    planned call whose problems put that group in the other class (its max_seqlen_kv hint raised
    to 40): the list's signature differs from the call's, every kernel of the call returns at once
    (GDPA_DEVICE_ERR_PLAN), and no output is touched. The same list used by the problems it was
    built for computes as usual."""
    short = make_workload("pffn_train", 85, num_seqs=4, len_range=(1, 200), keys=24, scale=0.125).groups[0]
    long = make_workload("pffn_train", 86, num_seqs=3, len_range=(1, 200), keys=300, scale=0.125).groups[0]
    built = [device_group(short), device_group(long)]
    called = [dataclasses.replace(built[0], max_seqlen_kv=40), built[1]]
    douts = [short.dout.to("cuda:0"), long.dout.to("cuda:0")]
    for problems, expect in ((built, 0), (called, _lib.GDPA_DEVICE_ERR_PLAN)):
        ws = ga.workspace(problems, 1)
        ga.gdpa_plan(built, ws)
        planned = [dataclasses.replace(p, planned=True) for p in problems]
        outs = [_nan_outputs(p) for p in problems]
        print(f"[gpu] guard: planned call, expected error word {expect}", flush=True)
        ga.gdpa_fwd_grouped(planned, outs=[o[0] for o in outs], ws=ws)
        ga.gdpa_bwd_grouped(planned, douts, fwd_outs=[o[0] for o in outs], outs=[o[1] for o in outs], ws=ws)
        torch.cuda.synchronize()
        assert ga.device_error(ws) == expect
        for (o, _), grads in outs:
            tensors = [o] + [t for t in grads[:3] if t is not None]
            if expect:
                assert all(torch.isnan(t).all() for t in tensors)
            else:
                assert all(torch.isfinite(t).all() for t in tensors)
