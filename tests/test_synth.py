"""The seeded generator: order independence, thread independence, moments."""
import os
import subprocess
import sys

import numpy as np

import synth
from synth import configs as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_slices_equal_whole():
    whole = synth.normal_f64(3, 5, 10001)
    for s, n in ((0, 1), (1, 1), (7, 100), (9990, 11), (5000, 3333)):
        assert np.array_equal(synth.normal_f64(3, 5, n, start=s), whole[s:s + n])
    b = synth.normal_stored(3, 5, 10001, 0.5, "bf16")
    assert np.array_equal(b[77:1077], synth.normal_stored(3, 5, 1000, 0.5, "bf16", start=77))
    assert np.array_equal(b, synth.round_to(0.5 * whole, "bf16"))


def test_independent_of_thread_count():
    code = ("import sys; sys.path.insert(0, %r); import synth, hashlib;"
            "a = synth.normal_stored(11, 3, 3_000_001, 0.1, 'bf16');"
            "print(hashlib.sha256(a.tobytes()).hexdigest())") % ROOT
    outs = set()
    for n in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        outs.add(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                capture_output=True, text=True).stdout.strip())
    assert len(outs) == 1


def test_moments_and_streams():
    n = 2_000_000
    x = synth.normal_f64(0, 1, n)
    assert abs(x.mean()) < 4 / np.sqrt(n)
    assert abs(x.var() - 1) < 4 * np.sqrt(2 / n)
    assert abs(np.mean(x ** 4) - 3) < 0.05           # Gaussian kurtosis
    y = synth.normal_f64(0, 2, n)
    assert abs(np.corrcoef(x, y)[0, 1]) < 4 / np.sqrt(n)
    z = synth.normal_f64(1, 1, n)
    assert not np.array_equal(x[:100], z[:100])


def test_splitmix64_reference_values():
    # SplitMix64 seeded with state 0: first outputs as published with the
    # algorithm (Steele, Lea, Flood 2014; also Vigna's reference C code).
    assert synth.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix64(0, 2) == 0x06C45D188009454F


def test_config_recipes_shapes():
    cfg = C.TINY
    assert cfg.u().shape == (16, 64) and cfg.u().dtype == np.float32
    assert cfg.w_route().shape == (4, 64)
    g, u, d = cfg.expert(3)
    assert g.shape == (128, 64) and u.shape == (128, 64) and d.shape == (64, 128)
    assert np.array_equal(cfg.expert_tensor("down")[3], d)
    m = C.MCU_BATCH
    assert m.u().dtype == np.uint16 and m.w_route().dtype == np.float32
    rows = np.array([5, 4095, 0])
    assert np.array_equal(m.u(rows), m.u()[rows])
    sw = C.SWITCH_SKEWED.with_(T=4, d=64, h=64)
    w = synth.normal_f64(sw.seed, synth.TID_W_ROUTE, sw.N * sw.d, 1 / 8).reshape(sw.N, sw.d)
    w[:2] *= 6
    assert np.array_equal(sw.w_route(), synth.round_to(w, "bf16"))
