"""The C-ABI boundary on the CPU: the library loads, exports what include/gdpa.h declares, its
structures match the ctypes mirrors, and invalid requests are rejected before any HIP call."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from generalized_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdpa.h")


@pytest.fixture(scope="module")
def lib():
    # GDPA_TEST_LIB: another build of the library to check (the sanitizer test's host-only build)
    path = os.environ.get("GDPA_TEST_LIB", _lib.LIB_PATH)
    if path == _lib.LIB_PATH and not os.path.exists(path):
        from generalized_attention_amd import build
        build.build()
    return _lib.load(path)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdpa_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_header():
    prog = r'''
#include <stdio.h>
#include <stddef.h>
#include "gdpa.h"
int main(void) {
  printf("%zu %zu\n", sizeof(gdpa_problem), sizeof(gdpa_tensors));
  printf("%zu %zu %zu %zu\n", offsetof(gdpa_problem, total_q), offsetof(gdpa_problem, q_offsets),
         offsetof(gdpa_problem, kv_offsets), offsetof(gdpa_tensors, dg));
  return 0;
}
'''
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "t.c")
        exe = os.path.join(tmp, "t")
        open(c, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()
    got = [int(x) for x in out]
    want = [ctypes.sizeof(_lib.gdpa_problem), ctypes.sizeof(_lib.gdpa_tensors),
            _lib.gdpa_problem.total_q.offset, _lib.gdpa_problem.q_offsets.offset,
            _lib.gdpa_problem.kv_offsets.offset, _lib.gdpa_tensors.dg.offset]
    assert got == want


FAKE = 0x10000  # never dereferenced: every case below fails validation on the host first


def good_problem(**kw):
    p = _lib.gdpa_problem()
    p.num_seqs, p.num_heads, p.head_dim = 2, 4, 64
    p.dtype, p.act, p.scale = _lib.GDPA_DTYPE_BF16, _lib.GDPA_ACT_SILU, 1e-3
    p.window_left = p.window_right = -1
    p.total_q, p.total_kv = 100, 512
    p.max_seqlen_q, p.max_seqlen_kv = 60, 256
    p.self_attention, p.flags = 0, 0
    p.q_offsets = p.kv_offsets = FAKE
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def good_tensors(**kw):
    t = _lib.gdpa_tensors()
    for f, _ in _lib.gdpa_tensors._fields_:
        setattr(t, f, 0)
    t.q = t.k = t.v = t.o = FAKE
    t.dout = t.dq = t.dk = t.dv = FAKE
    for k, v in kw.items():
        setattr(t, k, v)
    return t


def test_workspace_size(lib):
    n0 = _lib.gdpa_workspace_size([good_problem()], 0)
    n1 = _lib.gdpa_workspace_size([good_problem()], 1)
    assert n0 > 0 and n1 >= n0 and n0 % 256 == 0
    # softmax backward reserves per-row space
    sm = good_problem(act=_lib.GDPA_ACT_SOFTMAX)
    assert _lib.gdpa_workspace_size([sm], 1) >= n1
    assert _lib.gdpa_workspace_size([good_problem(head_dim=48)], 0) == 0
    assert _lib.gdpa_workspace_size([good_problem()] * 17, 0) == 0  # more than GDPA_MAX_GROUPS
    assert _lib.gdpa_workspace_size([good_problem()], 2) == 0


def test_workspace_size_key_chunks(lib):
    """Backward workspace grows by the fp32 dQ rows (and softmax row terms) exactly when some
    sequence may have more keys than a workgroup holds, or the queries are shared."""
    base = _lib.gdpa_workspace_size([good_problem()], 1)
    long_kv = good_problem(max_seqlen_kv=600, total_kv=1200)
    n = _lib.gdpa_workspace_size([long_kv], 1)
    assert n - base >= 100 * 4 * 64 * 4  # total_q x H x d floats
    assert _lib.gdpa_workspace_size([long_kv], 0) == _lib.gdpa_workspace_size([good_problem()], 0)
    sm = _lib.gdpa_workspace_size([good_problem(max_seqlen_kv=600, total_kv=1200, act=_lib.GDPA_ACT_SOFTMAX)], 1)
    assert sm - n >= 100 * 4 * 4  # plus D_i per (row, head)
    shared = good_problem(flags=_lib.GDPA_FLAG_SHARED_Q, max_seqlen_q=64)
    assert _lib.gdpa_workspace_size([shared], 1) - base >= 2 * 64 * 4 * 64 * 4  # B x S x H x d floats
    # a causal window narrow enough for the resident ring needs no chunk rows
    ring = good_problem(self_attention=1, total_q=1200, total_kv=1200, max_seqlen_q=600, max_seqlen_kv=600,
                        window_left=127, window_right=0)
    assert _lib.gdpa_workspace_size([ring], 1) == base
    wide = good_problem(self_attention=1, total_q=1200, total_kv=1200, max_seqlen_q=600, max_seqlen_kv=600,
                        window_left=300, window_right=0)
    assert _lib.gdpa_workspace_size([wide], 1) - base >= 1200 * 4 * 64 * 4


def test_fp32_output_flag():
    """float32 outputs change no workspace, in either pass, and are accepted (a no-op) in fp32."""
    for pass_ in (0, 1):
        base = _lib.gdpa_workspace_size([good_problem()], pass_)
        assert _lib.gdpa_workspace_size([good_problem(flags=_lib.GDPA_FLAG_FP32_OUT)], pass_) == base
    assert _lib.gdpa_workspace_size([good_problem(flags=_lib.GDPA_FLAG_FP32_OUT, dtype=_lib.GDPA_DTYPE_FP32)], 0) > 0


INVALID_PROBLEMS = [
    ("negative seqs", dict(num_seqs=-1), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("zero heads", dict(num_heads=0), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("257 heads", dict(num_heads=257), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("head dim 48", dict(head_dim=48), _lib.GDPA_ERR_UNSUPPORTED),
    ("bad dtype", dict(dtype=7), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("bad act", dict(act=3), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("nan scale", dict(scale=float("nan")), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("window below -1", dict(window_left=-2), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("window on cross-attention", dict(window_left=8), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("unknown flag", dict(flags=32), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("shared queries in self-attention", dict(flags=_lib.GDPA_FLAG_SHARED_Q, self_attention=1, total_kv=100,
                                              max_seqlen_kv=60), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("shared queries in fp32", dict(flags=_lib.GDPA_FLAG_SHARED_Q, dtype=_lib.GDPA_DTYPE_FP32), _lib.GDPA_ERR_UNSUPPORTED),
    ("null offsets", dict(q_offsets=0), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("max len above total", dict(max_seqlen_q=101), _lib.GDPA_ERR_INVALID_ARGUMENT),
    ("self-attention with unequal totals", dict(self_attention=1), _lib.GDPA_ERR_INVALID_ARGUMENT),
]


@pytest.mark.parametrize("name,kw,code", INVALID_PROBLEMS, ids=[c[0] for c in INVALID_PROBLEMS])
def test_invalid_problem_rejected(lib, name, kw, code):
    for fn in (_lib.gdpa_fwd, _lib.gdpa_bwd):
        assert fn(good_problem(**kw), good_tensors(), FAKE * 16, 1 << 20, 0) == code


INVALID_TENSORS = [
    ("null q", dict(q=0)),
    ("misaligned k", dict(k=FAKE + 2)),
    ("dg without g", dict(dg=FAKE)),
]


@pytest.mark.parametrize("name,kw", INVALID_TENSORS, ids=[c[0] for c in INVALID_TENSORS])
def test_invalid_tensors_rejected(lib, name, kw):
    for fn in (_lib.gdpa_fwd, _lib.gdpa_bwd):
        assert fn(good_problem(), good_tensors(**kw), FAKE * 16, 1 << 20, 0) == _lib.GDPA_ERR_INVALID_ARGUMENT


def test_forward_specific_checks(lib):
    # softmax forward needs lse; forward rejects a dg pointer
    sm = good_problem(act=_lib.GDPA_ACT_SOFTMAX)
    assert _lib.gdpa_fwd(sm, good_tensors(), FAKE * 16, 1 << 20, 0) == _lib.GDPA_ERR_INVALID_ARGUMENT
    assert _lib.gdpa_fwd(good_problem(), good_tensors(g=FAKE, dg=FAKE), FAKE * 16, 1 << 20, 0) == \
        _lib.GDPA_ERR_INVALID_ARGUMENT
    # softmax backward needs the forward's lse
    assert _lib.gdpa_bwd(sm, good_tensors(lse=0), FAKE * 16, 1 << 20, 0) == _lib.GDPA_ERR_INVALID_ARGUMENT


def test_per_head_activation_needs_lse(lib):
    # with an activation per head, some heads may be softmax: lse is required in both passes
    p = good_problem()
    p.head_acts = FAKE
    assert _lib.gdpa_fwd(p, good_tensors(), FAKE * 16, 1 << 20, 0) == _lib.GDPA_ERR_INVALID_ARGUMENT
    assert _lib.gdpa_bwd(p, good_tensors(lse=0), FAKE * 16, 1 << 20, 0) == _lib.GDPA_ERR_INVALID_ARGUMENT


def test_workspace_checks(lib):
    for fn in (_lib.gdpa_fwd, _lib.gdpa_bwd):
        assert fn(good_problem(), good_tensors(), 0, 1 << 20, 0) == _lib.GDPA_ERR_WORKSPACE
        assert fn(good_problem(), good_tensors(), FAKE * 16 + 8, 1 << 20, 0) == _lib.GDPA_ERR_WORKSPACE
        assert fn(good_problem(), good_tensors(), FAKE * 16, 16, 0) == _lib.GDPA_ERR_WORKSPACE


def test_any_key_length_accepted(lib):
    # every window and key length is accepted: a narrow window streams keys through the resident
    # ring; wider windows and unbounded long key ranges run in key chunks
    for wl, wr in ((127, 0), (200, 0), (-1, 0), (-1, -1), (300, 300)):
        p = good_problem(self_attention=1, total_q=5000, total_kv=5000, max_seqlen_q=2000, max_seqlen_kv=2000,
                         window_left=wl, window_right=wr, act=_lib.GDPA_ACT_SOFTMAX)
        assert _lib.gdpa_workspace_size([p], 0) > 0
        assert _lib.gdpa_workspace_size([p], 1) > 0
    cross = good_problem(total_kv=50000, max_seqlen_kv=30000)
    assert _lib.gdpa_workspace_size([cross], 1) > 0


def test_empty_problem_accepted(lib):
    """No sequences (and then no rows and no keys): every tensor pointer may be null, and the
    calls return GDPA_OK with nothing enqueued, so no HIP call is made here."""
    for act in (_lib.GDPA_ACT_SILU, _lib.GDPA_ACT_SOFTMAX):
        p = good_problem(num_seqs=0, total_q=0, total_kv=0, max_seqlen_q=0, max_seqlen_kv=0, act=act,
                         q_offsets=0, kv_offsets=0)
        none = good_tensors(q=0, k=0, v=0, o=0, dout=0, dq=0, dk=0, dv=0)
        for pass_ in (0, 1):
            assert _lib.gdpa_workspace_size([p], pass_) > 0
        assert _lib.gdpa_plan([p], FAKE * 16, 1 << 20, 0) == _lib.GDPA_OK
        assert _lib.gdpa_fwd(p, none, FAKE * 16, 1 << 20, 0) == _lib.GDPA_OK
        assert _lib.gdpa_bwd(p, none, FAKE * 16, 1 << 20, 0) == _lib.GDPA_OK
        assert _lib.gdpa_fwd_grouped([p, p], [none, none], FAKE * 16, 1 << 20, 0) == _lib.GDPA_OK
    # rows without sequences are inconsistent
    assert _lib.gdpa_workspace_size([good_problem(num_seqs=0)], 0) == 0


def test_grouped_requires_same_dtype(lib):
    a = good_problem()
    b = good_problem(dtype=_lib.GDPA_DTYPE_FP32)
    assert _lib.gdpa_fwd_grouped([a, b], [good_tensors(), good_tensors()], FAKE * 16, 1 << 20, 0) == \
        _lib.GDPA_ERR_INVALID_ARGUMENT


def test_strerror_and_version(lib):
    for code in (0, -1, -2, -3, -4, 99):
        assert isinstance(_lib.strerror(code), str)
    assert lib.gdpa_version() >= 200  # float32 outputs


def test_product_path_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "missing.so"))


def test_binding_fp32_outputs_marshalling():
    """The binding sets GDPA_FLAG_FP32_OUT and allocates float32 outputs for it (host tensors:
    marshalling only, nothing is launched)."""
    import torch
    import generalized_attention_amd as ga

    q = torch.zeros(10, 2, 32, dtype=torch.bfloat16)
    k = torch.zeros(6, 2, 32, dtype=torch.bfloat16)
    for fp32_out in (False, True):
        grp = ga.make_group(q, k, k, [0, 4, 10], [0, 3, 6], act="silu", scale=0.5, fp32_out=fp32_out)
        flags = grp.problem().flags
        assert bool(flags & _lib.GDPA_FLAG_FP32_OUT) == fp32_out
        o, lse = ga.ops._alloc_fwd(grp)
        dq, dk, dv, dg = ga.ops._alloc_bwd(grp, want_dg=False)
        want = torch.float32 if fp32_out else torch.bfloat16
        assert o.dtype == dq.dtype == dk.dtype == dv.dtype == want and lse is None and dg is None
        assert o.shape == q.shape and dk.shape == k.shape


def _offsets(lengths):
    import numpy as np
    o = np.zeros(len(lengths) + 1, dtype=np.int32)
    o[1:] = np.cumsum(lengths)
    return o


def test_validate_offsets_host(lib):
    """The offsets rules that the kernels' own item checks and the debug validation kernel apply,
    run on host arrays: each kind of violation sets its bit, and valid offsets give 0."""
    import numpy as np
    E_OFF, E_LEN, E_SELF = _lib.GDPA_DEVICE_ERR_OFFSETS, _lib.GDPA_DEVICE_ERR_LENGTH, _lib.GDPA_DEVICE_ERR_SELF
    qo, ko = _offsets([40, 60]), _offsets([256, 256])
    p = good_problem()  # B=2, total_q=100, total_kv=512, max 60 / 256
    assert _lib.gdpa_validate_offsets(p, qo, ko) == 0
    cases = [
        ("decreasing", np.array([0, 50, 40], np.int32), ko, E_OFF),
        ("not starting at 0", np.array([5, 45, 100], np.int32), ko, E_OFF),
        ("not ending at total_q", np.array([0, 40, 90], np.int32), ko, E_OFF),
        ("past total_kv", qo, np.array([0, 256, 600], np.int32), E_OFF | E_LEN),
        ("longer than max_seqlen_q", np.array([0, 30, 100], np.int32), ko, E_LEN),
        ("longer than max_seqlen_kv", qo, np.array([0, 200, 512], np.int32), E_LEN),
        ("negative start", np.array([-4, 40, 100], np.int32), ko, E_OFF),
    ]
    for name, q_off, kv_off, bits in cases:
        assert _lib.gdpa_validate_offsets(p, q_off, kv_off) == bits, name
    # self-attention: the two offset arrays must coincide
    sp = good_problem(self_attention=1, total_kv=100, max_seqlen_kv=60)
    assert _lib.gdpa_validate_offsets(sp, qo, qo) == 0
    assert _lib.gdpa_validate_offsets(sp, qo, np.array([0, 60, 100], np.int32)) == E_SELF
    # a shared query matrix bounds every sequence's rows by its own row count max_seqlen_q
    shared = good_problem(flags=_lib.GDPA_FLAG_SHARED_Q, max_seqlen_q=64, total_q=128)
    assert _lib.gdpa_validate_offsets(shared, _offsets([64, 64]), ko) == 0
    assert _lib.gdpa_validate_offsets(shared, _offsets([65, 63]), ko) == E_LEN
    # an invalid problem is refused as such
    assert _lib.gdpa_validate_offsets(good_problem(head_dim=48), qo, ko) == _lib.GDPA_ERR_UNSUPPORTED


def test_validate_flag_accepted(lib):
    """GDPA_FLAG_VALIDATE changes no workspace; the error word sits in the workspace header."""
    for pass_ in (0, 1):
        base = _lib.gdpa_workspace_size([good_problem()], pass_)
        assert _lib.gdpa_workspace_size([good_problem(flags=_lib.GDPA_FLAG_VALIDATE)], pass_) == base
        assert base >= 256 + 4  # header (error word) + a work list
    assert _lib.GDPA_WS_ERROR_OFFSET == 0


def test_noalloc_rejections_on_host(lib):
    """gdpa_bwd_noalloc checks everything before its first HIP call: a workspace beyond the 16 MiB
    scratch (a shared query matrix's fp32 partials) and a planned call are refused, as is an
    invalid problem."""
    big = good_problem(flags=_lib.GDPA_FLAG_SHARED_Q, num_seqs=600, max_seqlen_q=256, total_q=600 * 256,
                       total_kv=512, max_seqlen_kv=256)
    assert _lib.gdpa_workspace_size([big], 1) > _lib.GDPA_NOALLOC_SCRATCH_BYTES
    assert _lib.gdpa_bwd_noalloc(big, good_tensors(), 0) == _lib.GDPA_ERR_WORKSPACE
    assert _lib.gdpa_bwd_noalloc(good_problem(flags=_lib.GDPA_FLAG_PLANNED), good_tensors(), 0) == \
        _lib.GDPA_ERR_INVALID_ARGUMENT
    assert _lib.gdpa_bwd_noalloc(good_problem(head_dim=48), good_tensors(), 0) == _lib.GDPA_ERR_UNSUPPORTED
    assert _lib.gdpa_bwd_noalloc(good_problem(), good_tensors(dq=0), 0) == _lib.GDPA_ERR_INVALID_ARGUMENT
