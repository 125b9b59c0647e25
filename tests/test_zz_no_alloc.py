"""gdpa_bwd_noalloc (the backward with the library's own device scratch) against gdpa_bwd with a
caller workspace: bit-identical gradients on two calls in a row, the second with a smaller
problem, through the C ABI."""

from __future__ import annotations

import pytest
import torch

from gdpa_workloads import make_workload
from gpu_harness import device_group

import generalized_attention_amd as ga
from generalized_attention_amd import _lib

pytestmark = pytest.mark.gpu


def _noalloc(dev, dout, fwd_out, want_dg):
    dq, dk, dv, dg = ga.ops._alloc_bwd(dev, want_dg=want_dg)
    for t in (dq, dk, dv, dg):
        if t is not None:
            t.fill_(float("nan"))
    t = ga.ops._bwd_tensors(dev, dout, fwd_out[0], fwd_out[1], dq, dk, dv, dg)
    rc = _lib.gdpa_bwd_noalloc(dev.problem(), t, torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.GDPA_OK, _lib.strerror(rc)
    out = {"dq": dq, "dk": dk, "dv": dv}
    if dg is not None:
        out["dg"] = dg
    return out


@pytest.mark.parametrize("cases", [
    (("pffn_train", dict(num_seqs=24, len_range=(1, 700))), ("pffn_train", dict(num_seqs=5, len_range=(1, 200)))),
    (("causal_gated", dict(num_seqs=6, len_range=(1, 900))), ("causal_gated", dict(num_seqs=3, len_range=(1, 300)))),
    (("pffn_train", dict(num_seqs=6, len_range=(1, 300), keys=600, act="gelu", scale=0.125)),
     ("pffn_train", dict(num_seqs=2, len_range=(1, 100), keys=300, act="silu", scale=0.125))),
], ids=["pffn", "causal_gated", "key_chunks"])
def test_noalloc_matches_workspace_backward(cases):
    for call, (name, kw) in enumerate(cases):
        w = make_workload(name, 90 + call, **kw)
        g = w.groups[0]
        dev = device_group(g)
        dout = g.dout.to("cuda:0")
        want_dg = g.g is not None
        print(f"[gpu] noalloc call {call}: {name} {kw}", flush=True)
        o, lse = ga.gdpa_fwd(dev)
        ref = ga.gdpa_bwd(dev, dout, o=o, lse=lse, want_dg=want_dg)
        got = _noalloc(dev, dout, (o, lse), want_dg)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(ref[k], got[k]), (call, k)
