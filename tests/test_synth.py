"""Pins for the seeded input generator (`synth/`), the one module both the
oracle side and the GPU side consume. It holds none of the method's
arithmetic; these tests tie it to the published definitions it states.

 - SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): the reference sequence of
   the published algorithm for seed 1234567, and a restatement of it here;
 - the uniform in (0,1) from the top 53 bits, the Box-Muller pair, and
   round-to-nearest-even BF16, each restated and compared element by element;
 - the moments of the normal stream, and the per-head scale workload's scales.
"""
import math
import struct

import numpy as np

import synth

M64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def _mix64(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def _splitmix(seed, n):
    return _mix64((seed + (n + 1) * GAMMA) & M64)


def test_splitmix64_reference_sequence():
    # the first five outputs of the reference generator seeded with 1234567
    ref = [6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
           16408922859458223821]
    lib = synth._load()
    assert [int(lib.synth_splitmix64(1234567, n)) for n in range(5)] == ref
    rng = np.random.default_rng(1)
    for seed in [0, 1, 20261230, int(rng.integers(0, 2 ** 63))]:
        for n in [0, 1, 2, 1000, 2 ** 32 + 5, int(rng.integers(0, 2 ** 40))]:
            assert int(lib.synth_splitmix64(seed, n)) == _splitmix(seed, n)


def _uniform(seed, n):
    return ((_splitmix(seed, n) >> 11) + 0.5) * 2.0 ** -53


def _normal(seed, n):
    p = n >> 1
    u1, u2 = _uniform(seed, 2 * p), _uniform(seed, 2 * p + 1)
    r = math.sqrt(-2.0 * math.log(u1))
    return r * (math.sin(2 * math.pi * u2) if n & 1 else math.cos(2 * math.pi * u2))


def test_uniform_and_box_muller_restated():
    for seed in (7, 20261210):
        for n in list(range(20)) + [12345, 2 ** 33 + 1]:
            u = synth.uniform(seed, n)
            assert u == _uniform(seed, n) and 0.0 < u < 1.0
            z = synth.normal(seed, n)
            assert abs(z - _normal(seed, n)) <= 4e-16 * max(1.0, abs(z))


def _bf16_rne(x):
    u = struct.unpack("<I", struct.pack("<f", x))[0]   # the double rounded to float first
    return (u + 0x7FFF + ((u >> 16) & 1)) >> 16


def test_tensor_elements_are_the_normals_rounded_to_bf16():
    w = synth.custom(2, 37, 3, D=128, base_seed=555)
    q = synth.tensor(w, "q")
    assert q.shape == (2, 37, 3, 128) and q.dtype == np.uint16
    rng = np.random.default_rng(2)
    for _ in range(200):
        b, s, h, d = (int(rng.integers(0, n)) for n in q.shape)
        idx = ((b * 37 + s) * 3 + h) * 128 + d
        assert int(q[b, s, h, d]) == _bf16_rne(_normal(555, idx))


def test_normal_stream_moments():
    z = synth.bf16_to_float(synth.tensor(synth.custom(1, 4096, 2, base_seed=99), "v")).astype(np.float64).ravel()
    n = z.size   # 1 048 576 draws
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1.0) < 5 * math.sqrt(2.0 / n) + 2 ** -8   # BF16 rounding adds ~2^-9 relative
    assert abs(np.mean(z ** 3)) < 5 * math.sqrt(15.0 / n)
    assert abs(np.mean(np.abs(z) > 3.0) - 0.0026998) < 5 * math.sqrt(0.0027 / n)


def test_per_head_scale_workload():
    # the long-sequence workload draws an independent U[0.5, 3] scale per head for Q and for K
    w = synth.WORKLOADS["C3"]
    for which in "qk":
        stds = []
        for h in (0, 5, 27):
            x = synth.bf16_to_float(synth.head(w, which, 0, h, 0, 4096)).astype(np.float64)
            stds.append(x.std())
        assert all(0.45 < s_ < 3.1 for s_ in stds), (which, stds)
        assert max(stds) / min(stds) > 1.05   # the heads do differ
