"""Helpers shared by the GPU parity tests: move a seeded workload group to the device, run the
HIP path through the C ABI, and compare with the fp64 oracle by the tolerance rules below.

Tolerance rules (stated as numbers):
  * fp32 tensors: max |gpu - ref| <= 1e-5.
  * bf16 tensors: |gpu_i - ref_i| <= 2e-2 * RMS(ref) + 1/2 ulp_bf16(max(|ref_i|, |gpu_i|)) for
    every element, i.e. the stated 2e-2-of-RMS bound on the kernel's arithmetic plus the rounding
    of the stored bf16 result itself (which alone can exceed 2e-2 of RMS on large tensors: an
    exactly computed result rounded to bf16 deviates by up to 2^-9 relative to its own magnitude).
    The literal ratio max|gpu - ref| / RMS(ref) is returned for reporting.
  * float32 outputs of a bf16 problem: max |gpu - ref| <= 2e-2 * RMS(ref), the stated rule
    literally (nothing is rounded to bf16 on the way out).
"""

from __future__ import annotations

import numpy as np
import torch

import generalized_attention_amd as ga


def device_group(grp, dev="cuda:0", fp32_out=False):
    """GroupArgs on `dev` for a gdpa_workloads.Group (inputs copied bit-exactly)."""
    s = grp.spec
    q = grp.q.to(dev)
    k = grp.k.to(dev)
    v = grp.v.to(dev)
    g = None if grp.g is None else grp.g.to(dev)
    return ga.make_group(q, k, v, grp.q_offsets, grp.kv_offsets, act=s.act, scale=s.scale, window=s.window, g=g,
                         self_attention=s.keys_per_seq is None and not s.shared_q, shared_q=s.shared_q,
                         lengths_q=grp.lengths_q.tolist(),
                         lengths_kv=grp.lengths_kv.tolist(), fp32_out=fp32_out)


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def half_ulp_bf16(x):
    a = np.abs(x)
    out = np.zeros_like(a)
    nz = a > 0
    e = np.floor(np.log2(a[nz]))
    out[nz] = np.exp2(e - 8.0)
    return out


def check_bf16(gpu, ref, what, rel=2e-2):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(gpu - ref)
    bound = rel * rms + half_ulp_bf16(np.maximum(np.abs(ref), np.abs(gpu)))
    bad = err > bound
    literal = float(err.max() / rms) if rms > 0 else float(err.max())
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        where = np.argwhere(bad)
        rows = np.unique(where[:, 0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance in {len(rows)} rows "
                             f"(first rows {rows[:12].tolist()}); worst at {i}: gpu={gpu[i]!r} "
                             f"ref={ref[i]!r} bound={bound[i]:.3e} rms={rms:.3e} literal={literal:.4f}")
    return literal


def check_fp32(gpu, ref, what, atol=1e-5):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape
    if ref.size == 0:
        return 0.0
    err = float(np.max(np.abs(gpu - ref)))
    assert err <= atol, f"{what}: max abs err {err:.3e} > {atol:.1e}"
    return err


def check_bf16_fp32_out(gpu, ref, what, rel=2e-2):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = float(np.max(np.abs(gpu - ref)))
    literal = err / rms if rms > 0 else err
    assert err <= rel * rms, f"{what}: max err {err:.3e} > {rel} x rms {rms:.3e} (literal {literal:.4f})"
    return literal


def check(dtype, gpu, ref, what):
    """dtype: "fp32", "bf16", or "bf16/f32" (a bf16 problem with float32 outputs)."""
    if dtype == "fp32":
        return check_fp32(gpu, ref, what)
    if dtype == "bf16/f32":
        return check_bf16_fp32_out(gpu, ref, what)
    return check_bf16(gpu, ref, what)


def rows_of(offsets, seqs):
    return np.concatenate([np.arange(offsets[s], offsets[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, int)
