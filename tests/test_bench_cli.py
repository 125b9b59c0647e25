"""bench.py's command line on the CPU: more than one GPU is refused with a message (the path is
measured on one GPU), and the kernel-source hash that keys the committed traffic figures is
stable and covers each main kernel's sources."""

from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash():
    sys.path.insert(0, ROOT)
    import bench

    for kernel in ("fwd", "bwd"):
        h = bench.kernel_source_hash(kernel)
        assert len(h) == 16 and h == bench.kernel_source_hash(kernel)
        for f in bench.KERNEL_SOURCES[kernel]:
            assert os.path.exists(os.path.join(ROOT, "generalized_attention_amd", "csrc", f)), f
    assert bench.kernel_source_hash("fwd") != bench.kernel_source_hash("bwd")
