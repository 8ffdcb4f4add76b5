"""The C-ABI library loads, exports every entry point of include/fsa.h, and
rejects bad host arguments before touching a GPU (no device needed)."""
import ctypes
import glob
import os
import re

import pytest

import free_sparse_attention_amd as fsa
from free_sparse_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fsa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libfsa.so is not built (run python -m free_sparse_attention_amd.build)")
    return fsa.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def _d(**kw):
    base = dict(batch=1, num_q_heads=8, num_kv_heads=2, head_dim=64, max_pages_per_seq=256, num_pool_pages=256)
    base.update(kw)
    return fsa.dims(**base)


def test_workspace_sizing_and_bad_shapes(lib):
    c = fsa.cfg(64, 256, 32)
    assert fsa.sparse_decode_workspace_bytes(_d(), c, 4096) > 0
    assert fsa.dense_decode_workspace_bytes(_d(), 4096) > 0
    assert fsa.max_work_items(_d(), c, 4096) == 4 + 32 + 17
    assert fsa.meta_bytes(_d()) == 1 * 2 * 16 * 16 * 2 * 64 * 2
    for bad, status in ((dict(head_dim=96), _lib.FSA_ERR_UNSUPPORTED), (dict(num_q_heads=7), _lib.FSA_ERR_INVALID_ARG),
                        (dict(num_q_heads=34, num_kv_heads=2), _lib.FSA_ERR_UNSUPPORTED),
                        (dict(batch=0), _lib.FSA_ERR_INVALID_ARG)):
        assert lib.fsa_sparse_decode_workspace_bytes(ctypes.byref(_d(**bad)), c, 4096) == 0
        with pytest.raises(fsa.FsaError) as e:
            fsa.sparse_decode_workspace_bytes(_d(**bad), c, 4096)
        assert "dims" in str(e.value)
        st = lib.fsa_quest_scores(ctypes.byref(_d(**bad)), c, 4096, None, None, None, None, None)
        assert st == status
    # page size other than 16
    assert lib.fsa_build_page_meta(ctypes.byref(_d(page_size=32)), None, None, None, None, None) == _lib.FSA_ERR_UNSUPPORTED


def test_bad_cfg_len_and_pointers(lib):
    d = _d()
    p = ctypes.c_void_p(16)  # never dereferenced: every check runs before a launch
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(0, 0, 0), 4096, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"attends to nothing" in lib.fsa_last_error()
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(-1, 0, 4), 4096, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(64, 256, 32), 4097, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_quest_scores(ctypes.byref(d), fsa.cfg(64, 256, 32), 4096, p, None, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"meta" in lib.fsa_last_error()
    assert lib.fsa_append_kv(ctypes.byref(d), 0, p, p, p, p, None, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_kv(ctypes.byref(d), 1, p, p, p, p, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"alias" in lib.fsa_last_error()
    need = fsa.sparse_decode_workspace_bytes(d, fsa.cfg(64, 256, 32), 4096)
    st = lib.fsa_sparse_decode_attn(ctypes.byref(d), fsa.cfg(64, 256, 32), 0.125, 4096, p, p, p, p, p, p, p, None,
                                    p, need - 1, None)
    assert st == _lib.FSA_ERR_WORKSPACE
    st = lib.fsa_sparse_decode_attn(ctypes.byref(d), fsa.cfg(64, 256, 32), 0.0, 4096, p, p, p, p, p, p, p, None,
                                    p, need, None)
    assert st == _lib.FSA_ERR_INVALID_ARG
    st = lib.fsa_dense_decode_attn(ctypes.byref(d), 0.125, 4096, p, p, p, p, p, p, p, 0, None)
    assert st == _lib.FSA_ERR_WORKSPACE
    # combined append + decode: the append's and the step's checks, before any launch
    c = fsa.cfg(64, 256, 32)
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 0, p, p, p, p, c, 0.125, 4096, p, p, p, p, p, p, None, p, need,
                                      None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, p, c, 0.125, 4096, p, p, p, p, p, p, None, p, need,
                                      None) == _lib.FSA_ERR_INVALID_ARG
    assert b"alias" in lib.fsa_last_error()
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, None, c, 0.125, 4096, p, p, p, p, p, p, None, p,
                                      need, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_append_decode_attn(ctypes.byref(d), 1, p, p, p, ctypes.c_void_p(32), c, 0.125, 4096, p, p, p, p,
                                      p, p, None, p, need - 1, None) == _lib.FSA_ERR_WORKSPACE
    # the validator checks its host arguments before any launch
    assert lib.fsa_validate_inputs(ctypes.byref(d), 0, 4096, p, p, p, None, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"scratch" in lib.fsa_last_error()
    assert lib.fsa_validate_inputs(ctypes.byref(d), 0, 0, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_validate_inputs(ctypes.byref(d), -1, 4096, p, p, p, p, None) == _lib.FSA_ERR_INVALID_ARG
    assert b"n_new" in lib.fsa_last_error()


def _plan(B, hq, hkv, D, L, P, W, budget):
    n = (L + 15) // 16 + 8
    return fsa.describe_step(fsa.dims(B, hq, hkv, D, n, B * n), fsa.cfg(P, W, budget), L)


def test_step_plans_on_256_cus(lib):
    """Host-side planning (no device here: the library assumes MI355X's 256
    CUs).  Shapes of the 64k, 256k and ragged serving workloads, a short
    context and a many-replica case."""
    p = _plan(4, 16, 4, 128, 65536, 128, 1024, 128)
    assert (p["plan"], p["replicas"], p["per_replica"], p["xcd_grouped"], p["prefetch"], p["select_cols"]) == \
        ("wide", 8, 16, 1, 1, 4)
    assert p["slots"] == p["pw_workgroups"] + p["replicas"]
    p = _plan(4, 32, 4, 128, 262144, 128, 4096, 256)  # one XCD's share of selected K/V (4 MiB) > half its L2
    assert (p["plan"], p["replicas"], p["per_replica"], p["xcd_grouped"], p["prefetch"], p["select_cols"]) == \
        ("wide", 8, 32, 1, 0, 16)
    p = _plan(16, 32, 8, 128, 262144, 128, 2048, 256)  # 128 units: replicas would not fit
    assert (p["plan"], p["replicas"], p["xcd_grouped"], p["prefetch"]) == ("narrow", 0, 0, 0)
    p = _plan(9, 8, 1, 64, 6400, 32, 256, 224)  # 9 x 14 replicas fit, but 28 per XCD do not fit half an XCD
    assert (p["plan"], p["replicas"], p["xcd_grouped"], p["prefetch"]) == ("wide", 14, 0, 0)
    p = _plan(4, 16, 4, 128, 2048, 128, 1024, 128)  # every candidate fits the budget
    assert p["plan"] == "dense" and p["replicas"] == 0
    assert _plan(1, 8, 1, 128, 400001, 128, 4096, 256)["select_cols"] == 32


def test_describe_step_rejects_bad_arguments(lib):
    d = fsa.dims(1, 8, 2, 64, 100, 100)
    buf = (ctypes.c_int32 * 8)()
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 1600, None, 8) == -1
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 1600, buf, 3) == 3
    assert lib.fsa_describe_step(ctypes.byref(d), fsa.cfg(16, 64, 4), 10 ** 9, buf, 8) == -1


def test_measurement_helpers_check_their_arguments(lib):
    sink = ctypes.c_void_p(256)  # never dereferenced: every call below fails before any launch
    for buf, nbytes in ((None, 1024), (ctypes.c_void_p(4096), 0), (ctypes.c_void_p(4096), 1000),
                        (ctypes.c_void_p(4104), 1024)):
        assert lib.fsa_read_probe(buf, nbytes, sink, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_read_probe(ctypes.c_void_p(4096), 1024, None, None) == _lib.FSA_ERR_INVALID_ARG
    assert lib.fsa_device_memory(None, 4) == -1
    info = (ctypes.c_int32 * 4)()
    n = lib.fsa_device_memory(info, 4)
    if n == -1:  # no device here
        assert lib.fsa_last_error()
    else:
        assert n == 4 and info[0] > 0 and info[1] > 0 and info[2] > 0


def test_missing_library_fails_loudly(monkeypatch):
    """Without the built library the binding raises; nothing falls back to a CPU path."""
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load("/nonexistent/libfsa.so")


def _pw_items_needed(L, P, W):
    """Prefix and window items of a sequence of length L (brute force over its tokens):
    each page meeting the prefix [0, min(P, L)) is one item, and each page meeting the
    window's part past the prefix, [max(L - W, min(P, L)), L), is another."""
    Pe = min(P, L)
    w0 = max(L - W, Pe)
    pre = {t // 16 for t in range(0, Pe)}
    win = {t // 16 for t in range(w0, L)}
    return len(pre) + len(win)


@pytest.mark.parametrize("msl,P,W,budget", [
    (249, 5, 231, 1),    # prefix end and window start on one page at every length: n_pages + 1 items
    (241, 1, 228, 0),
    (16 * 1024, 16 * 3 + 5, 16 * 1019, 2),   # prefix + window nearly cover 1024 pages
    (16 * 1024, 16 * 1020 + 9, 40, 1),
    (4000, 64, 256, 8), (65536, 128, 1024, 128), (3000, 300, 5000, 7)])
def test_prefix_window_plan_holds_every_item(lib, msl, P, W, budget):
    """The prefix/window workgroups the planner sizes from the host length bound hold
    every prefix and window item of every length up to that bound (host only)."""
    for B, hq, hkv in ((2, 8, 2), (16, 32, 8)):
        n = (msl + 15) // 16
        p = fsa.describe_step(fsa.dims(B, hq, hkv, 128, n, B * n), fsa.cfg(P, W, budget), msl)
        if p["plan"] == "dense":
            continue
        cap = p["pw_workgroups"] * 16 * p["pw_items_per_wave"]
        # every length for short bounds; otherwise the top 64 lengths (every residue of
        # L mod 16 with the window past the prefix, where the count is largest)
        lens = range(1, msl + 1) if msl <= 5000 else range(msl - 64, msl + 1)
        need = max(_pw_items_needed(L, P, W) for L in lens)
        assert cap >= need, (p, need)


def test_noalloc_step_checks_size_before_any_device_call(lib):
    """The allocation-free step rejects a step whose workspace exceeds its fixed
    scratch, and bad arguments, before any HIP call (so this runs without a GPU)."""
    p = ctypes.c_void_p(16)  # never dereferenced
    d = fsa.dims(64, 64, 8, 128, 32768, 64 * 32768)
    c = fsa.cfg(128, 1024, 128)
    assert fsa.sparse_decode_workspace_bytes(d, c, 32768 * 16) > fsa.NOALLOC_SCRATCH_BYTES
    st = lib.fsa_sparse_decode_attn_noalloc(ctypes.byref(d), c, 0.1, 32768 * 16, p, p, p, p, p, p, p, None, None)
    assert st == _lib.FSA_ERR_WORKSPACE and b"allocation-free" in lib.fsa_last_error()
    small = _d()
    for args, status in (((fsa.cfg(0, 0, 0), 0.1, 4096), _lib.FSA_ERR_INVALID_ARG),
                         ((fsa.cfg(64, 256, 32), 0.0, 4096), _lib.FSA_ERR_INVALID_ARG),
                         ((fsa.cfg(64, 256, 32), 0.1, 4097), _lib.FSA_ERR_INVALID_ARG)):
        assert lib.fsa_sparse_decode_attn_noalloc(ctypes.byref(small), *args, p, p, p, p, p, p, p, None,
                                                  None) == status
    assert lib.fsa_sparse_decode_attn_noalloc(ctypes.byref(small), fsa.cfg(64, 256, 32), 0.1, 4096, p, p, p, None,
                                              p, p, p, None, None) == _lib.FSA_ERR_INVALID_ARG
    # the sizes the decode workloads need fit
    for B, hq, hkv, L, cfg in ((4, 16, 4, 65536, (128, 1024, 128)), (4, 32, 4, 262144, (128, 4096, 256)),
                               (16, 32, 8, 262144 + 64, (128, 2048, 256))):
        n = (L + 15) // 16
        assert fsa.sparse_decode_workspace_bytes(fsa.dims(B, hq, hkv, 128, n, B * n), fsa.cfg(*cfg), L) <= \
            fsa.NOALLOC_SCRATCH_BYTES


def test_launch_range_call_checks_its_arguments(lib):
    """The measurement call that runs some launches of a step rejects a range
    outside the step's launches, and the step's own bad arguments, before any launch."""
    d = _d()
    c = fsa.cfg(64, 256, 32)
    p = ctypes.c_void_p(256)  # never dereferenced
    need = fsa.sparse_decode_workspace_bytes(d, c, 4096)
    for first, last in ((-1, 0), (0, 3), (2, 1), (3, 3)):  # 4096 tokens, 64 / 256 / 32: the wide plan, 3 launches
        assert lib.fsa_sparse_decode_attn_launches(ctypes.byref(d), c, 0.1, 4096, p, p, p, p, p, p, p, None, p, need,
                                                   first, last, None) == -1
        assert b"launches" in lib.fsa_last_error()
    assert lib.fsa_sparse_decode_attn_launches(ctypes.byref(d), c, 0.1, 4096, p, p, p, p, p, p, p, None, p, need - 1,
                                               0, 0, None) == -1
    assert b"workspace" in lib.fsa_last_error()


@pytest.mark.parametrize("trace", ["1", None])
def test_trace_ranges_open_roctx_only_on_request(trace):
    """FSA_TRACE=1 makes the entry points open roctx ranges: the roctx library is
    loaded at run time on the first traced call (here one that fails its
    argument check before any launch); without it nothing is loaded."""
    import subprocess
    import sys
    code = (
        "import sys\n"
        f"sys.path.insert(0, {os.path.dirname(os.path.dirname(os.path.abspath(__file__)))!r})\n"
        "from free_sparse_attention_amd import _lib\n"
        "L = _lib.load()\n"
        "rc = L.fsa_quest_scores(None, _lib.LayerCfg(0, 0, 0), 0, None, None, None, None, None)\n"
        "maps = open('/proc/self/maps').read()\n"
        "print(rc, int('rocprofiler-sdk-roctx' in maps))\n")
    env = {k: v for k, v in os.environ.items() if k != "FSA_TRACE"}
    if trace:
        env["FSA_TRACE"] = trace
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    rc, loaded = r.stdout.split()
    assert int(rc) == _lib.FSA_ERR_INVALID_ARG
    if trace and not os.path.exists("/opt/rocm/lib/librocprofiler-sdk-roctx.so.1"):
        pytest.skip("no roctx library in this ROCm install")
    assert int(loaded) == (1 if trace else 0)


def test_fast_division_is_exact(tmp_path):
    """The kernels' division by launch-invariant divisors (fsa_internal.h
    make_fastdiv / fdiv), built for the host with hipcc: equal to n / d for
    every 16-bit numerator at divisors 1..1024 and for edge and random 32-bit
    numerators at divisors up to 2^32 - 1."""
    import subprocess
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc is not installed")
    csrc = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "free_sparse_attention_amd",
                        "csrc")
    src = tmp_path / "fastdiv.cpp"
    src.write_text(r'''
#include <cstdio>
#include <cstdint>
#include "fsa_internal.h"
int main() {
  uint64_t bad = 0, s = 88172645463325252ull;
  auto next = [&]() { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return (uint32_t)s; };
  for (uint32_t d = 1; d <= 1024; ++d) {
    const fsa::FastDiv f = fsa::make_fastdiv(d);
    for (uint32_t n = 0; n < 65536; ++n) bad += fsa::fdiv(n, f) != n / d;
  }
  const uint32_t ds[] = {1, 2, 3, 7, 8, 100, 65535, 65536, 65537, 1u << 20, 2147483647u, 2147483648u, 4294967295u};
  for (uint32_t d : ds) {
    const fsa::FastDiv f = fsa::make_fastdiv(d);
    const uint32_t edge[] = {0, 1, d - 1, d, d + 1, 2 * d - 1, 4294967295u, 4294967294u};
    for (uint32_t n : edge) bad += fsa::fdiv(n, f) != n / d;
    for (int i = 0; i < 1000000; ++i) { const uint32_t n = next(); bad += fsa::fdiv(n, f) != n / d; }
  }
  printf("%llu\n", (unsigned long long)bad);
  return 0;
}
''')
    exe = tmp_path / "fastdiv"
    r = subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950", "-I", csrc, "-o", str(exe),
                        str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.strip() == "0", (out.stdout, out.stderr[-500:])


def test_one_launch_plan_modes(lib):
    """The one-launch form of the wide plan (on 256 CUs, the count assumed
    without a device): off by default; mode 1 for unit counts that are
    multiples of 8 up to 64, mode 2 for any count up to 64."""
    def plan(units, mode):
        old = fsa.set_one_launch(mode)
        try:
            d = fsa.dims(units // 4, 16, 4, 128, 4096, units // 4 * 4096)
            return fsa.describe_step(d, fsa.cfg(128, 1024, 32 if units == 64 else 128), 65536)
        finally:
            fsa.set_one_launch(old)
    for units, want in ((16, 1), (64, 1), (8, 1), (12, 0), (4, 0)):
        got = plan(units, 1)
        assert got["plan"] == "wide" and got["one_launch"] == want, (units, got)
        assert (got["score_tasks"] > 0) == (want == 1)
    assert plan(12, 2)["one_launch"] == 1 and plan(4, 2)["one_launch"] == 1
    assert plan(16, 0)["one_launch"] == 0
    d = fsa.dims(4, 16, 4, 128, 4096, 4 * 4096)
    assert fsa.describe_step(d, fsa.cfg(128, 1024, 128), 65536)["one_launch"] == 0  # the default
    # scoring tasks of 16 waves, an XCD's at most one round of its 32 CUs:
    # 65536 tokens, window 1024 -> candidate pages 8 .. 4031 in tiles 0 .. 251,
    # 16 tasks of one tile per wave for 2 units per XCD, 4 for 8 units per XCD
    p = plan(16, 1)
    assert p["score_tasks"] == 16 and p["replicas"] == 8
    assert plan(64, 1)["score_tasks"] == 4
