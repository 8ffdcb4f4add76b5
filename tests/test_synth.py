"""The seeded input generator: determinism, thread-count independence, distributions."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_same_seed_same_bits_and_streams_differ():
    a = synth.normal_bf16(synth.stream_key(1, 2), 1000)
    b = synth.normal_bf16(synth.stream_key(1, 2), 1000)
    c = synth.normal_bf16(synth.stream_key(1, 3), 1000)
    assert (a == b).all() and (a != c).mean() > 0.9


def test_counter_mode_offsets_agree():
    k = synth.stream_key(5, 9)
    full = synth.normal_f64(k, 100)
    part = synth.normal_f64(k, 30, idx0=70)
    assert (full[70:] == part).all()


def test_normal_moments():
    x = synth.normal_f64(synth.stream_key(0, 1), 200000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = synth.uniform(synth.stream_key(0, 1), 100000)
    assert (u > 0).all() and (u < 1).all() and abs(u.mean() - 0.5) < 0.005


def test_bf16_rounding_nearest_even():
    # 1 + 2^-8 lies halfway between bf16 1.0 and 1 + 2^-7: ties to even (1.0)
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 3.140625])
    bits = synth.f64_to_bf16_bits(x)
    back = synth.bf16_bits_to_f64(bits)
    assert back.tolist() == [1.0, 1.0, 1 + 2**-6, -2.5, 3.140625]


def test_thread_count_does_not_change_values():
    code = ("import synth,sys;w=synth.make_workload('tiny',permuted=True);"
            "sys.stdout.write(str(int(w.k_pool.astype('uint64').sum())) + ' ' + str(int(w.v_pool.astype('uint64').sum())))")
    outs = set()
    for n in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.add(subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, check=True,
                                capture_output=True, text=True).stdout)
    assert len(outs) == 1


def test_tiny_workload_shape_and_needles():
    w = synth.make_workload("tiny")
    assert w.q.shape == (1, 8, 64) and w.k_pool.shape == (256, 2, 16, 64)
    assert len(w.needles[0]) == 8
    # needles lie in full pages of the middle region [prefix, L - window)
    assert (w.needles[0] >= 64).all() and (w.needles[0] < 4096 - 256).all()
    assert len(set((w.needles[0] // 16).tolist())) == 8


def test_ragged_lengths_in_range():
    L = synth.workloads.ragged_lens(4, 16, 16384, 262144)
    assert L.min() >= 16384 and L.max() <= 262144 and len(set(L.tolist())) == 16
