"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle is rebuilt with g++ ``-fsanitize=address,undefined`` and every fast pin of
  ``oracle_pins.py`` runs against it in a child interpreter that preloads gcc's sanitizer runtimes.
* Every unit of libgdpa.so is rebuilt host-only (hipcc ``--offload-host-only``: the argument
  checks, workspace layout, offsets validation and launch set-up, with empty device images in place
  of the kernels) with clang's sanitizers, and the CPU boundary tests (``test_boundary.py``) run against that library in a child
  interpreter that preloads clang's runtime. Those tests never reach a kernel launch.

Any sanitizer report fails the child (``halt_on_error``, no recovery from undefined behaviour),
and the reports' banners are also looked for in its output.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
REPORTS = ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer", "UndefinedBehaviorSanitizer")

pytestmark = pytest.mark.slow


def _run_child(args, env_extra, timeout=900):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, *args], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=timeout)
    out = r.stdout + r.stderr
    bad = [m for m in REPORTS if m in out]
    assert r.returncode == 0 and not bad, f"exit {r.returncode}, reports {bad}:\n{out[-6000:]}"
    return out


def _gcc_runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"gcc's {name} is not installed")
    return path


_ORACLE_CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle
from oracle_pins import FAST_CHECKS
lib = oracle.load({lib!r})
class Sanitized:
    def fwd(self, *a, **kw): return oracle.fwd(*a, lib=lib, **kw)
    def bwd(self, *a, **kw): return oracle.bwd(*a, lib=lib, **kw)
s = Sanitized()
for name, check in FAST_CHECKS:
    check(s)
    print("pin ok:", name, flush=True)
"""


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    oracle.build(out=lib, extra_flags=("-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                                       "-fno-sanitize-recover=undefined"))
    preload = _gcc_runtime("libasan.so") + ":" + _gcc_runtime("libubsan.so")
    code = _ORACLE_CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    out = _run_child(["-c", code], {"LD_PRELOAD": preload})
    from oracle_pins import FAST_CHECKS
    assert out.count("pin ok:") == len(FAST_CHECKS)


def _clang_asan_runtime():
    rt = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True,
                        check=True).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        rt = subprocess.run([CLANG, "--print-runtime-dir"], capture_output=True, text=True,
                            check=True).stdout.strip()
        rt = os.path.join(os.path.dirname(rt), "linux", "libclang_rt.asan-x86_64.so")
    assert os.path.exists(rt), "clang's AddressSanitizer runtime is missing"
    return rt


def _host_only_library(tmp_path, runtime):
    from generalized_attention_amd import build

    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer", "-I", build.INCLUDE, "-I", build.CSRC,
             "--offload-host-only", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-shared-libasan"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        cmd = [HIPCC, *flags, "-x", "hip", "-c", os.path.join(build.CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"host-only build of {src} failed:\n{r.stdout}{r.stderr}"
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, build.SOURCES))
    # A host-only object refers to its unit's device image by an external symbol. Stand in an empty
    # offload bundle for each: the runtime registers the images but never loads one, since no kernel
    # is launched.
    nm = subprocess.run(["nm", "-u", *objs], capture_output=True, text=True, check=True).stdout
    images = sorted(set(re.findall(r"__hip_fatbin_[0-9a-f]+", nm)))
    stub = tmp_path / "device_images.c"
    stub.write_text("".join(f'__attribute__((aligned(4096))) const unsigned char {n}[32] = '
                            f'"__CLANG_OFFLOAD_BUNDLE__";\n' for n in images))
    subprocess.run(["gcc", "-c", "-fPIC", str(stub), "-o", str(tmp_path / "device_images.o")], check=True)
    objs.append(str(tmp_path / "device_images.o"))
    lib = str(tmp_path / "libgdpa_host_san.so")
    cmd = [HIPCC, "--offload-host-only", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", "-Wl,-rpath," + os.path.dirname(runtime),
           *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"link failed:\n{r.stdout}{r.stderr}"
    return lib


def test_boundary_checks_under_sanitizers(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    rt = _clang_asan_runtime()
    lib = _host_only_library(tmp_path, rt)
    out = _run_child(["-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      os.path.join("tests", "test_boundary.py")],
                     {"LD_PRELOAD": rt, "GDPA_TEST_LIB": lib})
    assert " passed" in out and " failed" not in out, out[-3000:]
