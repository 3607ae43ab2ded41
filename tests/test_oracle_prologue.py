"""Pins for the oracle's prologue: INT8 per-32-row-block quantization of Q/K,
the fp64 key mean (smooth_k), and FP8 E4M3 per-channel quantization of V.

Pinned against hand-worked blocks, torch's half-to-even rounding and float8
conversion (library routines), math.fsum (a correctly rounded sum), closed
forms and error invariants; none of them re-runs the oracle's own formulas.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def bf16(x):
    """float -> BF16 bits via torch (exact for the values used here)."""
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------ INT8 blocks
def test_int8_block_hand_worked_ramp():
    # x = (i - 2048) / 16 over a 32 x 128 block: absmax 128 -> scale 128/127,
    # inv = 127/128 = 0.9921875 exactly.  Worked by hand:
    #   x = -128      -> -127
    #   x = 127.9375  -> 126.937988... -> 127
    #   x = 0.5       -> 0.49609375    -> 0
    #   x = 1.5625    -> 1.55029296875 -> 2
    #   x = -64.5     -> -63.99609375  -> -64
    x = ((np.arange(32 * 128, dtype=np.float32) - 2048) / 16).reshape(32, 128)
    q, s = oracle.quant_block_int8(x)
    assert s == np.float32(128.0) / np.float32(127.0)
    flat = q.ravel()
    def at(v):
        return int(flat[int(v * 16 + 2048)])
    assert at(-128) == -127 and at(127.9375) == 127 and at(0.5) == 0 and at(1.5625) == 2 and at(-64.5) == -64
    assert flat.min() == -127 and flat.max() == 127


def test_int8_block_single_spike_and_zero_block():
    x = np.zeros((32, 128), np.float32)
    x[7, 99] = -3.0
    q, s = oracle.quant_block_int8(x)
    assert s == np.float32(3.0) / np.float32(127.0)
    assert q[7, 99] == -127 and np.count_nonzero(q) == 1
    q0, s0 = oracle.quant_block_int8(np.zeros((32, 128), np.float32))
    assert s0 == 0.0 and not q0.any()


def test_int8_ties_round_half_to_even():
    # absmax 127 -> inv = 1 exactly, so codes are rint(x) directly
    x = np.zeros((32, 128), np.float32)
    x[0, 0] = 127.0
    vals = [2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5, 126.5, -126.5]
    for i, v in enumerate(vals):
        x[1, i] = v
    q, s = oracle.quant_block_int8(x)
    assert s == 1.0
    assert list(q[1, :len(vals)]) == [2, 4, -2, -4, 0, 0, 2, 126, -126]


def test_int8_codes_match_torch_round_half_even():
    import torch
    rng = np.random.default_rng(3)
    for rows in (32, 17, 1):
        x = (rng.standard_normal((rows, 128)) * rng.uniform(0.01, 50)).astype(np.float32)
        q, s = oracle.quant_block_int8(x)
        a = np.float32(np.abs(x).max())
        inv = np.float32(127.0) / a
        ref = torch.round(torch.from_numpy(x) * torch.tensor(inv, dtype=torch.float32)).to(torch.int8).numpy()
        assert np.array_equal(q, ref)
        assert s == a / np.float32(127.0)


def test_int8_error_bound_invariant():
    rng = np.random.default_rng(4)
    for _ in range(20):
        x = (rng.standard_normal((32, 128)) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        q, s = oracle.quant_block_int8(x)
        err = np.abs(x.astype(np.float64) - q.astype(np.float64) * np.float64(s))
        assert err.max() <= np.float64(s) * (0.5 + 2.0 ** -15)
        assert np.abs(q).max() == 127


# ------------------------------------------------------------ whole prologue of a head
def _head_inputs(S, seed, scale=1.0, D=128):
    rng = np.random.default_rng(seed)
    return [bf16((rng.standard_normal((S, D)) * scale).astype(np.float32)) for _ in range(3)]


@pytest.mark.parametrize("S", [1, 31, 32, 33, 96, 300])
def test_prepare_head_layout_and_tail_blocks(S):
    q, k, v = _head_inputs(S, S)
    out = oracle.prepare_head(q, k, v, smooth_k=False)
    nb = -(-S // 32)
    assert out["q_scale"].shape == (nb,) and out["v8t"].shape == (128, oracle.s_pad(S))
    assert not out["v8t"][:, S:].any()           # padding keys are zero codes
    assert not out["k_mean"].any()               # smooth_k off: nothing subtracted
    # each block (tail included) is quantized on its own rows only
    for n in range(nb):
        r0, r1 = 32 * n, min(S, 32 * n + 32)
        xq = synth.bf16_to_float(q[r0:r1])
        qb, sb = oracle.quant_block_int8(xq)
        assert out["q_scale"][n] == sb and np.array_equal(out["q8"][r0:r1], qb)


def test_k_mean_is_correctly_rounded_fp64_mean():
    w = synth.WORKLOADS["C2"]
    k = synth.head(w, "k", 0, 5)
    q = synth.head(w, "q", 0, 5)
    v = synth.head(w, "v", 0, 5)
    out = oracle.prepare_head(q, k, v, smooth_k=True)
    kf = synth.bf16_to_float(k).astype(np.float64)
    for d in range(128):
        exact = math.fsum(kf[:, d].tolist())          # correctly rounded sum
        assert out["k_mean"][d] == np.float32(exact / k.shape[0]), d


def test_smooth_k_subtracts_the_per_channel_mean():
    # K whose every channel sums to exactly 0 (second half = -first half), so the
    # fp64 mean is exactly 0 and smooth_k on must equal smooth_k off; adding a
    # per-channel constant c (BF16-exact) must then give bit-identical codes.
    rng = np.random.default_rng(9)
    S = 256
    half = np.round(np.clip(rng.standard_normal((S // 2, 128)), -7, 7) * 16) / 16
    kf = np.concatenate([half, -half]).astype(np.float32)
    c = np.round(rng.uniform(-3, 3, 128)).astype(np.float32)
    q, _, v = _head_inputs(S, 10)
    k0 = bf16(kf)
    kc = bf16(kf + c[None, :])
    assert np.array_equal(synth.bf16_to_float(kc), kf + c[None, :])   # shift is exact in BF16
    off = oracle.prepare_head(q, k0, v, smooth_k=False)
    on0 = oracle.prepare_head(q, k0, v, smooth_k=True)
    onc = oracle.prepare_head(q, kc, v, smooth_k=True)
    assert not on0["k_mean"].any()
    assert np.array_equal(onc["k_mean"], c)
    for key in ("k8", "k_scale"):
        assert np.array_equal(off[key], on0[key]) and np.array_equal(on0[key], onc[key])
    # Q and V do not depend on smooth_k
    for key in ("q8", "q_scale", "v8t", "v_scale"):
        assert np.array_equal(off[key], onc[key])


def test_constant_channel_mean_is_exact():
    S = 1000
    q, k, v = _head_inputs(S, 21)
    kf = synth.bf16_to_float(k).copy()
    kf[:, 3] = np.float32(1.7265625)     # BF16-exact constant
    out = oracle.prepare_head(q, bf16(kf), v, smooth_k=True)
    assert out["k_mean"][3] == np.float32(1.7265625)
    assert not out["k8"][:, 3].any()     # K' = 0 in that channel


def test_v_per_channel_fp8_matches_torch_and_bounds():
    import torch
    S = 300
    q, k, v = _head_inputs(S, 31, scale=3.0)
    out = oracle.prepare_head(q, k, v, smooth_k=False)
    vf = synth.bf16_to_float(v)
    a = np.abs(vf).max(axis=0)
    assert np.array_equal(out["v_scale"], a / np.float32(448.0))
    inv = (np.float32(448.0) / a).astype(np.float32)
    y = torch.from_numpy(vf) * torch.from_numpy(inv)[None, :]           # float products
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()           # torch's RNE conversion
    assert np.array_equal(out["v8t"][:, :S].T, ref)
    # the channel maximum maps to +-448 exactly
    amax_rows = np.abs(vf).argmax(axis=0)
    codes = out["v8t"][np.arange(128), amax_rows]
    assert np.all((codes & 0x7F) == 0x7E)
    # half-ulp error bound of E4M3 (relative 2^-4, subnormal floor 2^-10 of the scale)
    dec = oracle.e4m3_decode_table()[out["v8t"][:, :S].T].astype(np.float64)
    sc = out["v_scale"].astype(np.float64)[None, :]
    err = np.abs(vf.astype(np.float64) - dec * sc)
    assert np.all(err <= (2.0 ** -4) * np.abs(vf) * (1 + 2 ** -20) + (2.0 ** -10) * sc * (1 + 2 ** -20))


def test_zero_channel_and_zero_head():
    S = 64
    z = np.zeros((S, 128), np.uint16)
    out = oracle.prepare_head(z, z, z, smooth_k=True)
    assert not out["q8"].any() and not out["k8"].any() and not out["v8t"].any()
    assert not out["q_scale"].any() and not out["k_scale"].any() and not out["v_scale"].any()
    # negative zeros are zeros: a block or channel of +-0 has scale 0 and codes 0
    nz = z.copy()
    nz[::3] = 0x8000
    out = oracle.prepare_head(nz, nz, nz, smooth_k=False)
    assert not out["q8"].any() and not out["k8"].any() and not out["v8t"].any() and not out["v_scale"].any()


def test_full_tensor_prepare_matches_per_head():
    w = synth.custom(2, 70, 3, smooth_k=True)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    full = oracle.prepare(q, k, v, True)
    for b in range(2):
        for h in range(3):
            one = oracle.prepare_head(q[b, :, h], k[b, :, h], v[b, :, h], True)
            for key in one:
                assert np.array_equal(full[key][b, h], one[key]), key


# ------------------------------------------------------------ blocks and channels of tiny values
def test_int8_tiny_block_hand_worked():
    # a = 2^-130 (a BF16 subnormal): 127/a overflows a float, so the block is
    # lifted by 2^64 first.  Worked by hand from x * 127 / a:
    #   2^-130     -> 127
    #   -2^-131    -> -63.5  -> -64 (tie to even)
    #   3 * 2^-133 -> 47.625 -> 48
    #   2^-132     -> 31.75  -> 32
    #   0          -> 0
    x = np.zeros((32, 128), np.float32)
    x[0, 0], x[0, 1], x[5, 7], x[31, 127] = 2.0 ** -130, -(2.0 ** -131), 3 * 2.0 ** -133, 2.0 ** -132
    assert np.array_equal(synth.bf16_to_float(bf16(x)), x)          # all BF16-exact
    q, s = oracle.quant_block_int8(x)
    assert (q[0, 0], q[0, 1], q[5, 7], q[31, 127]) == (127, -64, 48, 32)
    assert np.count_nonzero(q) == 4
    assert s == np.float32(2.0 ** -130) / np.float32(127.0)


@pytest.mark.parametrize("exp", [-149, -140, -133, -126, -100, -70])
def test_int8_tiny_block_codes_are_scale_invariant(exp):
    # integer-valued blocks times 2^exp are exact floats down to the smallest
    # subnormal; a power-of-two scale cannot change the codes, and at 2^0 the
    # quotient 127/a is an ordinary float
    rng = np.random.default_rng(100 - exp)
    for rows in (32, 7):
        xi = rng.integers(-255, 256, size=(rows, 128)).astype(np.float32)
        xi[rng.random(xi.shape) < 0.3] = 0
        ref, _ = oracle.quant_block_int8(xi)
        tiny = (xi * np.float32(2.0 ** exp)).astype(np.float32)
        assert np.array_equal(tiny.astype(np.float64) * 2.0 ** -exp, xi)   # exact
        q, s = oracle.quant_block_int8(tiny)
        assert np.array_equal(q, ref)
        assert s == np.float32(np.abs(tiny).max()) / np.float32(127.0)


def test_v_tiny_channel_codes_and_output_are_finite_and_scale_invariant():
    S = 200
    q, k, v = _head_inputs(S, 77)
    vf = synth.bf16_to_float(v).copy()
    # channel 5: absmax about 5e-37 (448/a overflows a float), its small values
    # BF16 subnormals; channel 9: lifted, though 448/a would be finite
    vf[:, 5] = synth.bf16_to_float(bf16(vf[:, 5] * np.float32(2.0 ** -122)))
    vf[:, 9] = vf[:, 9] * np.float32(2.0 ** -60)
    vt = bf16(vf)
    assert np.array_equal(synth.bf16_to_float(vt), vf)
    assert np.abs(vf[:, 5]).max() < 448.0 / np.finfo(np.float32).max
    # the same channels scaled back up by exact powers of two: ordinary inputs
    vr = vf.copy()
    vr[:, 5] *= np.float32(2.0 ** 122)
    vr[:, 9] *= np.float32(2.0 ** 60)
    v = bf16(vr)
    assert np.array_equal(synth.bf16_to_float(v), vr)
    out = oracle.prepare_head(q, k, vt, smooth_k=False)
    ref = oracle.prepare_head(q, k, v, smooth_k=False)
    for d in (5, 9):
        a = np.float32(np.abs(vf[:, d]).max())
        assert out["v_scale"][d] == a / np.float32(448.0)
        assert np.array_equal(out["v8t"][d], ref["v8t"][d])         # codes unchanged by the 2^-k factor
    assert np.all((out["v8t"] & 0x7F) != 0x7F)                       # no NaN codes
    o = oracle.bf16_bits_to_f64(oracle.attn_rows_head(out, np.arange(S), 1 / np.sqrt(128)))
    o_ref = oracle.bf16_bits_to_f64(oracle.attn_rows_head(ref, np.arange(S), 1 / np.sqrt(128)))
    assert np.all(np.isfinite(o))
    # channel 9 stays a normal float: exactly the scaled output; channel 5's
    # output lies among BF16 subnormals (spacing 2^-133), so up to that spacing
    assert np.array_equal(o[:, 9], o_ref[:, 9] * 2.0 ** -60)
    assert np.max(np.abs(o[:, 5] - o_ref[:, 5] * 2.0 ** -122)) <= 2.0 ** -133 * (1 + 1e-6)


# ------------------------------------------------------------ the exact fp64 key sum
def _bf16_exactly(vals):
    vals = np.asarray(vals, np.float64)
    bits = bf16(vals.astype(np.float32))
    assert np.array_equal(synth.bf16_to_float(bits).astype(np.float64), vals)
    return bits


def test_exact_sum_on_adversarial_channels_matches_fsum():
    rng = np.random.default_rng(2026)
    chans = [
        [2.0 ** 60, 1.0, -(2.0 ** 60), 1.0] * 50,               # ascending fp64 sum gives 1, exact 100
        [2.0 ** 100, 2.0 ** -100, -(2.0 ** 100), 3 * 2.0 ** -98],
        [2.0 ** 53, 1.0],                                       # tie: rounds to even (2^53)
        [2.0 ** 53, 1.0, 2.0 ** -100],                          # just above the tie: 2^53 + 2
        [2.0 ** 127, -(2.0 ** 127), 2.0 ** -133],               # largest and smallest magnitudes
        [2.0 ** -133] * 7 + [-(2.0 ** -131)],                   # subnormals cancelling to 3 * 2^-133
        [1.5, -1.5, 0.0, -0.0],                                 # exact zero
    ]
    for _ in range(40):                                         # random signs and exponents over the whole range
        n = int(rng.integers(1, 3000))
        # normal BF16 values m * 2^e (8-bit significand m) and some subnormals m * 2^-133
        m = rng.integers(128, 256, n).astype(np.float64)
        e = rng.integers(-133, 121, n).astype(np.float64)
        sub = rng.random(n) < 0.1
        m[sub], e[sub] = rng.integers(1, 128, int(sub.sum())), -133
        sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
        chans.append(list(sign * m * 2.0 ** e))
    for vals in chans:
        bits = _bf16_exactly(vals)
        exact = math.fsum(vals)                                 # correctly rounded sum
        assert oracle.bf16_exact_sum(bits) == exact, vals[:4]
    # the ascending-order fp64 sum differs on the first channel, so the pin discriminates
    acc = 0.0
    for x in chans[0]:
        acc += x
    assert acc != math.fsum(chans[0])


def test_k_mean_of_adversarial_channels_is_the_rounded_exact_mean():
    S = 96
    rng = np.random.default_rng(5)
    kf = rng.standard_normal((S, 128)).astype(np.float32)
    kf[:, 0] = np.tile(np.array([2.0 ** 60, 1.0, -(2.0 ** 60)], np.float32), S // 3)
    kf[:, 1] = np.where(np.arange(S) % 2 == 0, np.float32(2.0 ** 70), np.float32(2.0 ** -70)) * \
        np.where(np.arange(S) % 4 < 2, 1, -1).astype(np.float32)
    kf[:, 2] = np.float32(2.0 ** -130) * (np.arange(S) % 5 - 2)
    k = bf16(kf)
    q, _, v = _head_inputs(S, 6)
    out = oracle.prepare_head(q, k, v, smooth_k=True)
    kd = synth.bf16_to_float(k).astype(np.float64)
    for d in range(128):
        assert out["k_mean"][d] == np.float32(math.fsum(kd[:, d].tolist()) / S), d
    assert out["k_mean"][0] == np.float32(32.0 / S)
