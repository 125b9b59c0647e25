"""Plant plausible mistakes in a copy of the oracle and check that the pins catch every one.

Each mutant is a single textual substitution in ``oracle/gdpa_oracle.cpp`` (a dropped term, a
wrong sign, a wrong operand or index, an off-by-one window edge), compiled into a temporary
library. The pin checks of ``oracle_pins.py`` run against it; at least one must fail. The real
oracle source is never modified.
"""

import os
import subprocess
import tempfile

import pytest

import oracle
from oracle_pins import FAST_CHECKS, check_finite_differences

MUTANTS = [
    ("drop gate", "if (p.g) sij += log_sigmoid", "if (false) sij += log_sigmoid"),
    ("log sigmoid sign", "return x - std::log1p(std::exp(x));", "return x + std::log1p(std::exp(x));"),
    ("gelu grad sign", "+ x * kInvSqrt2Pi", "- x * kInvSqrt2Pi"),
    ("gelu wrong erf argument", "return x * 0.5 * (1.0 + std::erf(x / kSqrt2));",
     "return x * 0.5 * (1.0 + std::erf(x * kSqrt2));"),
    ("silu grad", "(1.0 + x * (1.0 - s))", "(1.0 + x * (1.0 + s))"),
    ("dv uses q", "dvj[c] += pij * doi[c];", "dvj[c] += pij * qi[c];"),
    ("dk missing scale", "dkj[c] += p.scale * dsij * qi[c];", "dkj[c] += dsij * qi[c];"),
    ("dq uses v", "dqi[c] += p.scale * dsij * kj[c];",
     "dqi[c] += p.scale * dsij * p.v[((k0 + j) * H + h) * d + c];"),
    ("softmax drops D", "ds[t] = pr[t] * (dp[t] - D);", "ds[t] = pr[t] * dp[t];"),
    ("window left off by one", "if (p.wl >= 0 && i - p.wl > a) a = i - p.wl;",
     "if (p.wl >= 0 && i - p.wl - 1 > a) a = i - p.wl - 1;"),
    ("window right ignored", "if (p.wr >= 0 && i + p.wr < b) b = i + p.wr;", ""),
    ("lse without log", "return m + std::log(l);", "return m + l;"),
    ("query row of the key sequence", "(p.shared_q > 0 ? 0 : p.q_off[b]) + i;",
     "(p.shared_q > 0 ? 0 : p.kv_off[b]) + i;"),
    ("shared query rows shifted", "(p.shared_q > 0 ? 0 : p.q_off[b]) + i;", "(p.shared_q > 0 ? 1 : p.q_off[b]) + i;"),
    ("shared query gradient not summed", "acc += part[", "acc = part["),
    ("head index swapped", "double sij = p.scale * dot(qi, kj, d);",
     "double sij = p.scale * dot(qi, p.k + ((k0 + j) * H + (H - 1 - h)) * d, d);"),
    ("dg missing sigmoid", "+= sigmoid(-p.g[(k0 + j) * H + h]) * dsij", "+= dsij"),
    ("per-head activation ignored", "return p.head_acts ? p.head_acts[h] : p.act;", "return p.act;"),
    ("lse of an empty row is zero", "if (n <= 0) return -std::numeric_limits<double>::infinity();",
     "if (n <= 0) return 0.0;"),
    ("empty softmax row not zeroed", "for (int c = 0; c < d; ++c) oi[c] = 0.0;", "for (int c = 0; c < d; ++c) oi[c] = (hi < lo) ? 1.0 : 0.0;"),
    ("shared query row bound dropped", "if (p.q_off[b + 1] - p.q_off[b] > p.shared_q) return false;",
     "if (false) return false;"),
    ("offsets start unchecked", "if (p.q_off[0] != 0 || p.kv_off[0] != 0) return false;", ""),
    ("v transposed", "oi[c] += pr[j - lo] * vj[c];", "oi[c] += pr[j - lo] * p.v[((k0 + c % (hi - lo + 1)) * H + h) * d + (j % d)];"),
]


class _Mutant:
    def __init__(self, lib):
        self.lib = lib

    def fwd(self, *a, **kw):
        return oracle.fwd(*a, lib=self.lib, **kw)

    def bwd(self, *a, **kw):
        return oracle.bwd(*a, lib=self.lib, **kw)


def _caught(mut) -> bool:
    for _, check in FAST_CHECKS:
        try:
            check(mut)
        except (AssertionError, ValueError):
            return True
    for args in [("gelu", (-1, -1), True, False), ("softmax", (1, 0), True, True)]:
        try:
            check_finite_differences(mut, args[0], 0.9, args[1], args[2], self_attn=args[3])
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique/absent"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, "mutant.cpp")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib_path = os.path.join(tmp, "libmutant.so")
        subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-pthread", path, "-o",
                        lib_path], check=True)
        mut = _Mutant(oracle.load(lib_path))
        assert _caught(mut), f"no pin caught mutant {name!r}"
