"""The oracle's pins catch planted mistakes (CPU).

Each case copies the oracle (``oracle.cpp`` and the float64 numpy
``reference.py``) into a scratch directory, plants one plausible mistake --
a dropped term, a wrong sign, index or operand, an off-by-one, a swapped tie
rule -- rebuilds the C++ library there and runs ``test_oracle_pins.py``
against the copy.  The pins must fail for every planted mistake and pass for
the unchanged copy and for rewrites that change nothing (the page min/max
loop bounded by the length twice; a prefix longer than the sequence left
unclamped, which every later use bounds by the length anyway).  Mistakes are planted in the oracle only,
never in the HIP path.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CPP, NP = "oracle/oracle.cpp", "oracle/reference.py"
# (file, text, replacement, what the mistake is)
MUTATIONS = [
    (CPP, "const double a = v[k - 1].s, b = v[k].s;", "const double a = v[k].s, b = v[std::min(k + 1, C - 1)].s;",
     "selection margin taken one rank low"),
    (CPP, "q_bits[((size_t)b * hq + g * G + h) * D + i]", "q_bits[((size_t)b * hq + h * hkv + g) * D + i]",
     "query heads dealt round-robin to KV heads"),
    (CPP, "const uint32_t u = (uint32_t)bits << 16;", "const uint32_t u = (uint32_t)bits << 15;",
     "bf16 bits shifted by 15"),
    (CPP, "best = std::max(best, quest_bound_one(in.q + (size_t)h * D, m + p * stride, M + p * stride, D));",
     "best = (h == 0 ? 0.0 : best) + quest_bound_one(in.q + (size_t)h * D, m + p * stride, M + p * stride, D);",
     "group score summed, not maximised"),
    (CPP, "return a.page < b.page;", "return a.page > b.page;", "ties to the higher page id"),
    (CPP, "*Ws = std::max(0, L - W);", "*Ws = std::max(0, L - W + 1);", "window one token short"),
    (CPP, "m[(size_t)p * D + i] = lo + 0.0;", "m[(size_t)p * D + i] = lo;", "minimum keeps a -0"),
    (CPP, "z[j] = scale * dot;", "z[j] = dot;", "softmax scale dropped"),
    (CPP, "return (Ws + S - 1) / S - Pe / S;", "return Ws / S - Pe / S;", "partial last candidate page dropped"),
    (CPP, "u += std::max(q[i] * m[i], q[i] * M[i]);", "u += q[i] * M[i];", "bound ignores the minimum"),
    (CPP, "u += std::max(q[i] * m[i], q[i] * M[i]);", "u += std::min(q[i] * m[i], q[i] * M[i]);",
     "bound takes the smaller product"),
    (CPP, "const size_t phys = (size_t)pt_row[t / S];", "const size_t phys = (size_t)(t / S);", "page table ignored"),
    (CPP, "return bf16_value(pool[((phys * hkv + g) * S + t % S) * D + i]);",
     "return bf16_value(pool[((phys * hkv + g) * S + (t + 1) % S) * D + i]);", "token slot off by one"),
    (CPP, "for (int i = 0; i < D; ++i) num[i] += w * vals(toks[j], i);",
     "for (int i = 0; i < D; ++i) num[i] += w * keys(toks[j], i);", "values read from the keys"),
    (CPP, "for (int i = 0; i < D; ++i) out[(size_t)h * D + i] = num[i] / den;",
     "for (int i = 0; i < D; ++i) out[(size_t)h * D + i] = num[i];", "softmax not normalised"),
    (CPP, "for (int t = sel[j] * S; t < std::min(sel[j] * S + S, L); ++t) mask[t] = 1;",
     "for (int t = sel[j] * S; t < std::min(sel[j] * S + S - 1, L); ++t) mask[t] = 1;",
     "selected page's last token dropped"),
    (NP, "return float((s[k - 1] - s[k]) / max(abs(s[k - 1]), 1e-300))",
     "return float((s[k] - s[min(k + 1, len(s) - 1)]) / max(abs(s[k]), 1e-300))",
     "numpy: selection margin one rank low"),
    (NP, "q = bf16_to_f64(qb[b, g * G:(g + 1) * G])", "q = bf16_to_f64(qb[b, g::wl.hkv])",
     "numpy: query heads round-robin"),
    (NP, "return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)",
     "return (b.astype(np.uint32) << 15).view(np.float32).astype(np.float64)", "numpy: bf16 bits shifted by 15"),
]
# rewrites that must change nothing (the pins must still pass)
EQUIVALENT = [
    (CPP, "for (int t = p * S + 1; t < t_end; ++t) {",
     "for (int t = p * S + 1; t < p * S + S && t < t_end + 1 && t < L; ++t) {", "min/max loop bounded twice"),
    (CPP, "*Pe = std::min(P, L);", "*Pe = P;", "prefix left unclamped (every use is bounded by the length)"),
]


def _run(case, tmp):
    path, old, new, what = case
    d = os.path.join(tmp, "".join(ch if ch.isalnum() else "_" for ch in what))
    os.makedirs(d)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.so"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(d, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(d, "tests"))
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(d, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(d, "tests", "golden"))
    if old is not None:
        f = os.path.join(d, path)
        s = open(f).read()
        assert s.count(old) == 1, f"anchor for '{what}' not found once in {path}"
        open(f, "w").write(s.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    subprocess.run([sys.executable, "-c", "import oracle; oracle.build_lib()"], cwd=d, env=env, check=True,
                   capture_output=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_oracle_pins.py"], cwd=d, env=env, capture_output=True, text=True)
    tail = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else r.stderr[-300:]
    return r.returncode, tail


@pytest.fixture(scope="module")
def results(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("mutants"))
    cases = [(None, None, None, "unchanged")] + EQUIVALENT + MUTATIONS
    with ThreadPoolExecutor(max_workers=4) as ex:
        outs = list(ex.map(lambda c: _run(c, tmp), cases))
    return {c[3]: o for c, o in zip(cases, outs)}


def test_unchanged_and_equivalent_copies_pass(results):
    for what in ["unchanged"] + [c[3] for c in EQUIVALENT]:
        rc, tail = results[what]
        assert rc == 0 and "passed" in tail and "failed" not in tail, (what, tail)


@pytest.mark.parametrize("what", [c[3] for c in MUTATIONS])
def test_planted_mistake_fails_a_pin(results, what):
    rc, tail = results[what]
    # a genuine catch: the pins ran and at least one of them failed (not an
    # import or build error)
    assert rc == 1 and " failed" in tail, (what, tail)
