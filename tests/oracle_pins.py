"""Checks that pin the fp64 oracle to things other than itself.

Each check takes an oracle module-like object (``fwd``/``bwd`` callables with the signatures of
``oracle.fwd``/``oracle.bwd``) so that the same checks run against the real oracle
(``test_oracle_pins.py``) and against deliberately broken copies of it
(``test_oracle_mutants.py``). Every check raises AssertionError on failure.

What they compare against (none of it re-types the oracle's formulas):
  * torch library routines in float64: ``torch.nn.functional.gelu`` (exact erf form),
    ``silu``, ``logsigmoid``, ``scaled_dot_product_attention`` and autograd;
  * closed-form worked examples (``tests/golden/worked_examples.json``);
  * identities the sources state: the element-wise form equals the back-to-back product
    act(X W1) W2 (Kunlun review, section 2.3 / Figure 2; substack breakdown, "Core
    Architecture"), softmax rows sum to one, a gate of +inf reduces the gated form to plain
    scaled dot-product attention (reproduction README, "Core equations"), a window at least as
    long as the sequence equals full attention (review, section 2.5);
  * central finite differences of the oracle's own forward for its backward;
  * invariants: sample independence, permutation equivariance over sequences, zero upstream
    gradient, zero-sum key gradients of softmax.
"""

from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_examples.json")


def offsets(lengths):
    o = np.zeros(len(lengths) + 1, dtype=np.int64)
    o[1:] = np.cumsum(lengths)
    return o


def rand_problem(seed, lq, lk=None, h=2, d=8, std=1.0, gate=False, shared_rows=0):
    """Small jagged problem with float64 entries; lk=None means self-attention (lk = lq).
    shared_rows > 0: q is one [shared_rows, h, d] query matrix shared by every sequence."""
    rng = np.random.default_rng(seed)
    lk = lq if lk is None else lk
    tq, tk = int(sum(lq)), int(sum(lk))
    q = rng.standard_normal((shared_rows if shared_rows else tq, h, d)) * std
    k = rng.standard_normal((tk, h, d)) * std
    v = rng.standard_normal((tk, h, d))
    g = rng.standard_normal((tk, h)) * 2.0 if gate else None
    do = rng.standard_normal((tq, h, d))
    return dict(q=q, k=k, v=v, g=g, do=do, qo=offsets(lq), ko=offsets(lk))


def _mask(lq, lk, window):
    left, right = window
    i = torch.arange(lq)[:, None]
    j = torch.arange(lk)[None, :]
    m = torch.ones(lq, lk, dtype=torch.bool)
    if left >= 0:
        m &= j >= i - left
    if right >= 0:
        m &= j <= i + right
    return m


def torch_reference(pb, act, scale, window=(-1, -1), need_grad=False, shared=False):
    """Per (sequence, head) dense evaluation with torch library routines in float64.

    Element-wise form: act(scale * Q_h K_h^T) V_h with masked entries dropped (the PFFN product
    with W1 = K_h^T, W2 = V_h). Softmax form: scaled_dot_product_attention with an additive
    float mask log sigmoid(G) (and -inf outside the window). act may list one form per head.
    shared: every sequence takes its query rows from the top of the one query matrix; autograd
    then sums that matrix's gradient over the sequences."""
    _, h, d = pb["q"].shape
    q = torch.tensor(pb["q"], requires_grad=need_grad)
    k = torch.tensor(pb["k"], requires_grad=need_grad)
    v = torch.tensor(pb["v"], requires_grad=need_grad)
    g = None if pb["g"] is None else torch.tensor(pb["g"], requires_grad=need_grad)
    outs = [None] * (len(pb["qo"]) - 1)
    for b in range(len(pb["qo"]) - 1):
        q0, q1 = int(pb["qo"][b]), int(pb["qo"][b + 1])
        k0, k1 = int(pb["ko"][b]), int(pb["ko"][b + 1])
        m = _mask(q1 - q0, k1 - k0, window)
        heads = []
        for hh in range(h):
            Q = q[0:q1 - q0, hh] if shared else q[q0:q1, hh]
            K = k[k0:k1, hh]
            V = v[k0:k1, hh]
            act_h = act if isinstance(act, str) else act[hh]
            if act_h == "softmax":
                bias = torch.zeros(q1 - q0, k1 - k0, dtype=torch.float64)
                if g is not None:
                    bias = bias + F.logsigmoid(g[k0:k1, hh])[None, :]
                bias = bias.masked_fill(~m, float("-inf"))
                if q1 - q0 == 0 or k1 - k0 == 0:
                    heads.append(torch.zeros(q1 - q0, d, dtype=torch.float64))
                    continue
                o = F.scaled_dot_product_attention(Q[None], K[None], V[None], attn_mask=bias[None],
                                                   scale=scale)[0]
                heads.append(o)
            else:
                S = scale * (Q @ K.T)
                if g is not None:
                    S = S + F.logsigmoid(g[k0:k1, hh])[None, :]
                fn = F.gelu if act_h == "gelu" else F.silu
                P = torch.where(m, fn(S), torch.zeros((), dtype=torch.float64))
                heads.append(P @ V)
        outs[b] = torch.stack(heads, dim=1) if heads else torch.zeros(q1 - q0, 0, d)
    o = torch.cat(outs, dim=0) if outs else torch.zeros(0, h, d, dtype=torch.float64)
    if not need_grad:
        return {"o": o.detach().numpy()}
    (o * torch.tensor(pb["do"])).sum().backward()
    res = {"o": o.detach().numpy(), "dq": q.grad.numpy(), "dk": k.grad.numpy(),
           "dv": v.grad.numpy()}
    if g is not None:
        res["dg"] = g.grad.numpy()
    return res


def close(a, b, rtol=1e-11, atol=1e-12, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    bound = atol + rtol * (np.max(np.abs(b)) if b.size else 0.0)
    assert err <= bound, f"{what}: max err {err:.3e} > {bound:.3e}"


# ---------------------------------------------------------------------------------------------
# The checks
# ---------------------------------------------------------------------------------------------

def check_worked_examples(orc):
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        q = np.asarray(c["q"], np.float64)[:, None, :]
        k = np.asarray(c["k"], np.float64)[:, None, :]
        v = np.asarray(c["v"], np.float64)[:, None, :]
        g = None if c["g"] is None else np.asarray(c["g"], np.float64)[:, None]
        r = orc.fwd(q, k, v, [0, len(q)], [0, len(k)], act=c["act"], scale=c["scale"], g=g,
                    window=tuple(c["window"]))
        close(r["o"][:, 0, :], np.asarray(c["o"]), rtol=1e-14, atol=1e-15, what=c["name"])
        if "lse" in c:
            close(r["lse"][:, 0], np.asarray(c["lse"]), rtol=1e-14, atol=1e-15, what=c["name"] + " lse")


def check_forward_vs_library(orc, act, scale, window=(-1, -1), gate=False, seed=0, self_attn=False):
    lq = [5, 0, 1, 9, 3]
    lk = None if self_attn else [7, 4, 0, 6, 2]
    pb = rand_problem(seed, lq, lk, gate=gate, h=2 if isinstance(act, str) else len(act))
    r = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=scale, g=pb["g"],
                window=window)
    ref = torch_reference(pb, act, scale, window)
    close(r["o"], ref["o"], what=f"fwd {act} {window} gate={gate}")


def check_backward_vs_autograd(orc, act, scale, window=(-1, -1), gate=False, seed=1, self_attn=False):
    lq = [4, 0, 6, 1]
    lk = None if self_attn else [5, 3, 0, 2]
    pb = rand_problem(seed, lq, lk, gate=gate, h=2 if isinstance(act, str) else len(act))
    r = orc.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act=act, scale=scale,
                g=pb["g"], window=window, want_dg=gate)
    ref = torch_reference(pb, act, scale, window, need_grad=True)
    for name in ("dq", "dk", "dv") + (("dg",) if gate else ()):
        close(r[name], ref[name], rtol=1e-10, atol=1e-12, what=f"bwd {name} {act} {window}")


def check_shared_queries(orc, act, scale, gate=False, seed=5):
    """One query matrix (6 rows) attending over five jagged sequences of keys: forward and all
    gradients against torch autograd, which sums the shared matrix's gradient by itself."""
    lq = [5, 0, 3, 5, 1]
    lk = [7, 4, 0, 9, 2]
    pb = rand_problem(seed, lq, lk, gate=gate, shared_rows=6)
    r = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=scale, g=pb["g"], shared_q=True)
    rb = orc.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act=act, scale=scale, g=pb["g"],
                 want_dg=gate, shared_q=True)
    ref = torch_reference(pb, act, scale, need_grad=True, shared=True)
    close(r["o"], ref["o"], what=f"shared-query fwd {act}")
    for name in ("dq", "dk", "dv") + (("dg",) if gate else ()):
        close(rb[name], ref[name], rtol=1e-10, atol=1e-12, what=f"shared-query bwd {name} {act}")


def check_finite_differences(orc, act, scale, window=(-1, -1), gate=False, seed=2, self_attn=True):
    """Central differences of L = sum(dO * O) through the oracle's own forward."""
    lq = [3, 2]
    lk = None if self_attn else [4, 3]
    pb = rand_problem(seed, lq, lk, h=1, d=3, gate=gate)
    r = orc.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act=act, scale=scale,
                g=pb["g"], window=window, want_dg=gate)

    def loss(q, k, v, g):
        o = orc.fwd(q, k, v, pb["qo"], pb["ko"], act=act, scale=scale, g=g, window=window)["o"]
        return float((o * pb["do"]).sum())

    eps = 1e-6
    names = ["q", "k", "v"] + (["g"] if gate else [])
    for name in names:
        base = {n: (None if pb[n] is None else pb[n].copy()) for n in ("q", "k", "v", "g")}
        grad = np.zeros_like(base[name])
        it = np.nditer(base[name], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            plus = {n: (None if base[n] is None else base[n].copy()) for n in base}
            minus = {n: (None if base[n] is None else base[n].copy()) for n in base}
            plus[name][idx] += eps
            minus[name][idx] -= eps
            grad[idx] = (loss(plus["q"], plus["k"], plus["v"], plus["g"]) -
                         loss(minus["q"], minus["k"], minus["v"], minus["g"])) / (2 * eps)
        close(r["d" + name], grad, rtol=1e-6, atol=1e-8, what=f"fd d{name} {act}")


def check_pffn_identity(orc, act):
    """act(X W1) W2 for a generated weight pair equals GDPA with Q=X, K=W1^T, V=W2, scale 1."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 6))     # 11 tokens of one sequence, width 6
    w1 = rng.standard_normal((6, 9))     # generated first-layer weight: width -> 9 hidden units
    w2 = rng.standard_normal((9, 6))
    fn = F.gelu if act == "gelu" else F.silu
    ref = (fn(torch.tensor(x) @ torch.tensor(w1)) @ torch.tensor(w2)).numpy()
    r = orc.fwd(x[:, None, :], w1.T.copy()[:, None, :], w2[:, None, :], [0, 11], [0, 9], act=act,
                scale=1.0)
    close(r["o"][:, 0, :], ref, what=f"PFFN identity {act}")


def check_softmax_rows_sum_to_one(orc):
    pb = rand_problem(4, [6, 1, 0, 8], None, gate=True)
    ones = np.ones_like(pb["v"])
    r = orc.fwd(pb["q"], pb["k"], ones, pb["qo"], pb["ko"], act="softmax", scale=0.7, g=pb["g"],
                window=(2, 1))
    close(r["o"], np.ones_like(pb["q"]), rtol=0, atol=1e-13, what="rows sum to one")
    # lse = log sum exp of the allowed scores (scipy-free: torch.logsumexp is the library routine)
    qo = pb["qo"]
    for b in range(len(qo) - 1):
        for hh in range(pb["q"].shape[1]):
            Q = torch.tensor(pb["q"][qo[b]:qo[b + 1], hh])
            K = torch.tensor(pb["k"][qo[b]:qo[b + 1], hh])
            G = torch.tensor(pb["g"][qo[b]:qo[b + 1], hh])
            S = 0.7 * Q @ K.T + F.logsigmoid(G)[None, :]
            S = S.masked_fill(~_mask(len(Q), len(K), (2, 1)), float("-inf"))
            if len(Q):
                close(r["lse"][qo[b]:qo[b + 1], hh], torch.logsumexp(S, dim=1).numpy(), what="lse")


def check_rows_without_keys(orc):
    """A query row that sees no key: its softmax lse is log of an empty sum (torch.logsumexp of an
    all -inf score row gives -inf) and its output is the empty sum, zero, in every form. Rows of a
    sample with no keys (cross-attention, n_b = 0) and rows that a window moves past the last key
    (cross-attention with window (0, 0): row i sees only key i) are both such rows."""
    lq, lk = [3, 5, 2], [0, 2, 4]
    pb = rand_problem(12, lq, lk, gate=True)
    for window in ((-1, -1), (0, 0)):
        for act in ("softmax", "gelu"):
            r = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=0.6, g=pb["g"],
                        window=window)
            for b in range(len(lq)):
                for i in range(lq[b]):
                    row = int(pb["qo"][b]) + i
                    allowed = _mask(lq[b], lk[b], window)[i] if lk[b] else torch.zeros(0, dtype=torch.bool)
                    if bool(allowed.any()):
                        continue
                    assert np.all(r["o"][row] == 0.0), f"o of a row without keys ({act}, {window})"
                    if act == "softmax":
                        empty = torch.full((max(lk[b], 1),), float("-inf"), dtype=torch.float64)
                        want = float(torch.logsumexp(empty, dim=0))
                        got = r["lse"][row]
                        assert np.all(got == want), f"lse of a row without keys: {got} vs {want}"
    # and a row with keys keeps a finite lse
    r = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act="softmax", scale=0.6, g=pb["g"])
    assert np.all(np.isfinite(r["lse"][int(pb["qo"][1]):])), "rows with keys"


def check_rejects_bad_arguments(orc):
    """Arguments outside the definition are refused (ValueError) instead of read: offsets that
    decrease or do not start at zero, and a sequence with more rows than a shared query matrix
    holds. The shared matrix is a view into a larger buffer, so a wrongly accepted call reads
    memory that exists."""
    q = np.zeros((2, 1, 4))
    for qo, ko in (([0, 2, 1], [0, 1, 2]), ([1, 2], [0, 2])):
        try:
            orc.fwd(q, q, q, qo, ko, act="gelu", scale=1.0)
        except ValueError:
            pass
        else:
            raise AssertionError(f"offsets {qo} / {ko} accepted")
    big = np.zeros((8, 1, 4))
    shared = big[:3]  # S = 3 rows
    kv = np.zeros((6, 1, 4))
    for lq in ([3, 2], [2, 4]):
        try:
            orc.fwd(shared, kv, kv, offsets(lq), offsets([3, 3]), act="softmax", scale=1.0, shared_q=True)
        except ValueError:
            assert max(lq) > 3, "a sequence within the shared rows was refused"
        else:
            assert max(lq) <= 3, f"a sequence of {max(lq)} rows over a 3-row shared query matrix accepted"


def check_gate_infinity_is_sdpa(orc):
    pb = rand_problem(5, [7, 3], None, gate=False)
    g = np.full((pb["k"].shape[0], pb["k"].shape[1]), 40.0)
    r = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act="softmax", scale=0.3, g=g,
                window=(-1, 0))
    ref = torch_reference(pb, "softmax", 0.3, (-1, 0))  # no gate at all
    close(r["o"], ref["o"], rtol=1e-12, what="G=+inf -> SDPA")
    # a very negative gate on one key removes it
    g2 = np.full_like(g, 40.0)
    g2[2, :] = -800.0
    r2 = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act="softmax", scale=0.3, g=g2)
    keep = [j for j in range(pb["k"].shape[0]) if j != 2]
    pb2 = dict(pb)
    pb2["k"], pb2["v"] = pb["k"][keep], pb["v"][keep]
    pb2["ko"] = offsets([6, 3])
    pb2["qo"] = pb["qo"]
    # rows of sequence 1 are unaffected (key 2 belongs to sequence 0)
    ref2 = torch_reference(dict(pb2, qo=offsets([7, 3])), "softmax", 0.3)
    close(r2["o"], ref2["o"], rtol=1e-12, what="G=-inf removes the key")


def check_window_covering_sequence_is_full(orc):
    pb = rand_problem(6, [9, 4, 1], None, gate=True)
    for act in ("softmax", "gelu"):
        full = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=0.5, g=pb["g"])
        wide = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=0.5, g=pb["g"],
                       window=(9, 9))
        close(wide["o"], full["o"], rtol=0, atol=0, what="window >= L equals full")
        causal_full = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=0.5,
                              g=pb["g"], window=(-1, 0))
        causal_wide = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act=act, scale=0.5,
                              g=pb["g"], window=(8, 0))
        close(causal_wide["o"], causal_full["o"], rtol=0, atol=0, what="causal window >= L")


def check_invariants(orc):
    # zero upstream gradient gives zero gradients
    pb = rand_problem(7, [5, 2], [3, 4], gate=True)
    r = orc.bwd(pb["q"], pb["k"], pb["v"], np.zeros_like(pb["do"]), pb["qo"], pb["ko"], act="silu",
                scale=0.9, g=pb["g"], want_dg=True)
    for n in ("dq", "dk", "dv", "dg"):
        assert np.all(r[n] == 0.0), n
    # softmax: sum_j ds_ij = 0  =>  sum_j dk_j = 0 per (sequence, head)
    pb = rand_problem(8, [6, 5], None, gate=True)
    r = orc.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act="softmax", scale=0.8,
                g=pb["g"], window=(3, 0), want_dg=True)
    for b in range(2):
        s = r["dk"][pb["ko"][b]:pb["ko"][b + 1]].sum(axis=0)
        close(s, np.zeros_like(s), rtol=0, atol=1e-12, what="sum_j dk_j = 0")
    # sample independence: perturbing sequence 1 changes nothing of sequence 0
    pb = rand_problem(9, [4, 3], [5, 2])
    base = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act="gelu", scale=0.6)["o"]
    k2 = pb["k"].copy()
    k2[5:] += 1.0
    pert = orc.fwd(pb["q"], k2, pb["v"], pb["qo"], pb["ko"], act="gelu", scale=0.6)["o"]
    assert np.array_equal(base[:4], pert[:4])
    assert not np.array_equal(base[4:], pert[4:])
    # permutation equivariance: the sequences in reverse order give the same per-sequence results
    lq, lk = [3, 0, 5, 2], [4, 2, 3, 1]
    pb = rand_problem(10, lq, lk, gate=True)
    fw = orc.fwd(pb["q"], pb["k"], pb["v"], pb["qo"], pb["ko"], act="silu", scale=0.7, g=pb["g"])
    bw = orc.bwd(pb["q"], pb["k"], pb["v"], pb["do"], pb["qo"], pb["ko"], act="silu", scale=0.7, g=pb["g"],
                 want_dg=True)
    order = [3, 2, 1, 0]

    def rows(off, b):
        return np.arange(off[b], off[b + 1])

    qi = np.concatenate([rows(pb["qo"], b) for b in order])
    ki = np.concatenate([rows(pb["ko"], b) for b in order])
    qo2, ko2 = offsets([lq[b] for b in order]), offsets([lk[b] for b in order])
    fw2 = orc.fwd(pb["q"][qi], pb["k"][ki], pb["v"][ki], qo2, ko2, act="silu", scale=0.7, g=pb["g"][ki])
    bw2 = orc.bwd(pb["q"][qi], pb["k"][ki], pb["v"][ki], pb["do"][qi], qo2, ko2, act="silu", scale=0.7,
                  g=pb["g"][ki], want_dg=True)
    assert np.array_equal(fw["o"][qi], fw2["o"]) and np.array_equal(bw["dq"][qi], bw2["dq"])
    for n in ("dk", "dv", "dg"):
        assert np.array_equal(bw[n][ki], bw2[n]), n


def check_activation_closed_forms(lib):
    import math
    # Phi(1), Phi(-1), Phi(2) of the standard normal; GELU(x) = x Phi(x)
    assert abs(lib.gdpa_oracle_phi(0, 1.0) - 0.8413447460685429) < 1e-15
    assert abs(lib.gdpa_oracle_phi(0, -1.0) + 0.15865525393145707) < 1e-15
    assert abs(lib.gdpa_oracle_phi(0, 2.0) - 2 * 0.9772498680518208) < 1e-14
    # GELU'(0) = Phi(0) = 1/2; GELU'(1) = Phi(1) + phi(1)
    assert abs(lib.gdpa_oracle_phi_grad(0, 0.0) - 0.5) < 1e-15
    assert abs(lib.gdpa_oracle_phi_grad(0, 1.0) - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    # SiLU(1) = e/(1+e); SiLU'(0) = 1/2; SiLU'(1) = s(1)(1 + (1 - s(1)))
    s1 = math.e / (1 + math.e)
    assert abs(lib.gdpa_oracle_phi(1, 1.0) - s1) < 1e-15
    assert abs(lib.gdpa_oracle_phi_grad(1, 0.0) - 0.5) < 1e-15
    assert abs(lib.gdpa_oracle_phi_grad(1, 1.0) - s1 * (2 - s1)) < 1e-15
    # log sigmoid: log(1/2) at 0, ~x for very negative x, ~-exp(-x) for large x
    assert abs(lib.gdpa_oracle_log_sigmoid(0.0) + math.log(2)) < 1e-15
    assert lib.gdpa_oracle_log_sigmoid(-700.0) == -700.0
    assert abs(lib.gdpa_oracle_log_sigmoid(30.0) + math.exp(-30.0)) < 1e-25


FAST_CHECKS = [
    ("worked examples", lambda o: check_worked_examples(o)),
    ("fwd gelu", lambda o: check_forward_vs_library(o, "gelu", 0.7)),
    ("fwd silu", lambda o: check_forward_vs_library(o, "silu", 0.7)),
    ("fwd softmax gated window", lambda o: check_forward_vs_library(o, "softmax", 0.5, (2, 0), True, self_attn=True)),
    ("fwd gelu gated window", lambda o: check_forward_vs_library(o, "gelu", 0.5, (1, 2), True, self_attn=True)),
    ("bwd gelu", lambda o: check_backward_vs_autograd(o, "gelu", 0.8)),
    ("bwd silu", lambda o: check_backward_vs_autograd(o, "silu", 0.8)),
    ("bwd softmax gated window", lambda o: check_backward_vs_autograd(o, "softmax", 0.6, (2, 0), True, self_attn=True)),
    ("bwd silu gated window", lambda o: check_backward_vs_autograd(o, "silu", 0.6, (1, 1), True, self_attn=True)),
    ("fwd per-head acts", lambda o: check_forward_vs_library(o, ["gelu", "softmax", "silu"], 0.7, (3, 1), True, self_attn=True)),
    ("bwd per-head acts", lambda o: check_backward_vs_autograd(o, ["softmax", "silu", "gelu"], 0.7, gate=True)),
    ("PFFN identity gelu", lambda o: check_pffn_identity(o, "gelu")),
    ("PFFN identity silu", lambda o: check_pffn_identity(o, "silu")),
    ("rows sum to one", lambda o: check_softmax_rows_sum_to_one(o)),
    ("rows without keys", lambda o: check_rows_without_keys(o)),
    ("rejects bad arguments", lambda o: check_rejects_bad_arguments(o)),
    ("gate inf is sdpa", lambda o: check_gate_infinity_is_sdpa(o)),
    ("window covering sequence", lambda o: check_window_covering_sequence_is_full(o)),
    ("invariants", lambda o: check_invariants(o)),
    ("shared queries softmax gated", lambda o: check_shared_queries(o, "softmax", 0.6, gate=True)),
    ("shared queries silu", lambda o: check_shared_queries(o, "silu", 0.9)),
]
