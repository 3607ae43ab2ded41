"""Pins for the oracle's number codecs (BF16 and OCP FP8 E4M3).

Each pin compares the oracle with something that is not the oracle: torch's
own bfloat16 / float8_e4m3fn conversions (library routines) and a brute-force
nearest-code search over the 256-entry code table written here.
"""
import math

import numpy as np
import pytest

import oracle


def torch_e4m3_table(torch):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()


# ------------------------------------------------------------------ BF16
def test_bf16_decode_all_patterns(torch_cpu):
    torch = torch_cpu
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = np.array([oracle.lib().oracle_bf16_decode(int(b)) for b in bits[::7]], np.float32)
    ref = torch.from_numpy(bits[::7].view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_matches_torch_rne(torch_cpu):
    torch = torch_cpu
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(5000) * 1e-30).astype(np.float32),
        (rng.standard_normal(5000) * 1e30).astype(np.float32),
        # exact ties: bf16 value plus half an ulp, both parities
        (((np.arange(4000, dtype=np.uint32) + 0x3F80) << 16) | 0x8000).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-45], np.float32),
    ])
    ours = oracle.bf16_encode_array(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_all_codes_match_torch(torch_cpu):
    ours = oracle.e4m3_decode_table()
    ref = torch_e4m3_table(torch_cpu)
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.all((ours == ref) | both_nan)
    # format facts from the OCP spec: NaN only at S.1111.111, largest 448, smallest subnormal 2^-9
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.isnan(ours).sum() == 2
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert math.copysign(1.0, float(ours[0x80])) < 0


def _nearest_codes(xs: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Brute force over the code table: nearest finite code, ties to the even
    code, magnitudes above 448 saturate, the sign (also of zero) is kept."""
    xs = np.asarray(xs, np.float64)
    finite = np.asarray(table[:0x7F], np.float64)  # codes 0x00..0x7E
    a = np.abs(xs)
    dist = np.abs(finite[None, :] - a[:, None])
    dmin = dist.min(axis=1, keepdims=True)
    cand = dist == dmin
    even = cand & ((np.arange(0x7F) & 1) == 0)[None, :]
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    pick = np.where(a > 448.0, 0x7E, pick)
    sign = np.where(np.signbit(xs), 0x80, 0)
    out = (pick | sign).astype(np.uint8)
    return np.where(np.isnan(xs), 0x7F, out).astype(np.uint8)


def _probe_values(table):
    vals = []
    pos = [float(table[c]) for c in range(0x7F)]
    for i, v in enumerate(pos):
        f = np.float32(v)
        vals += [f, np.nextafter(f, np.float32(1e9)), np.nextafter(f, np.float32(-1e9))]
        if i + 1 < len(pos):
            mid = np.float32((v + pos[i + 1]) / 2.0)  # exact: midpoints have few bits
            vals += [mid, np.nextafter(mid, np.float32(1e9)), np.nextafter(mid, np.float32(-1e9))]
    vals += [np.float32(v) for v in (448.0, 456.0, 464.0, 465.0, 1e4, 1e38, 2.0 ** -10, 2.0 ** -11, 1e-40)]
    vals += [np.nextafter(np.float32(448.0), np.float32(1e9))]
    return np.array(vals, np.float32)


def test_e4m3_encode_boundaries_vs_brute_force(torch_cpu):
    table = torch_e4m3_table(torch_cpu)
    xs = _probe_values(table)
    xs = np.concatenate([xs, -xs, np.array([0.0, -0.0, np.inf, -np.inf, np.nan], np.float32)])
    assert np.array_equal(oracle.e4m3_encode_array(xs), _nearest_codes(xs, table))


def test_e4m3_encode_random_vs_brute_force(torch_cpu):
    table = torch_e4m3_table(torch_cpu)
    rng = np.random.default_rng(11)
    mags = np.exp2(rng.uniform(-12, 9.2, 60000)).astype(np.float32)
    xs = mags * np.where(rng.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode_array(xs), _nearest_codes(xs, table))


def test_e4m3_encode_matches_torch_in_range(torch_cpu):
    torch = torch_cpu
    rng = np.random.default_rng(12)
    mags = np.exp2(rng.uniform(-14, np.log2(448.0), 200000)).astype(np.float32)
    xs = mags * np.where(rng.random(mags.size) < 0.5, -1, 1).astype(np.float32)
    xs = np.concatenate([xs, _probe_values(torch_e4m3_table(torch))])
    xs = xs[np.abs(xs) <= 448.0]
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = oracle.e4m3_encode_array(xs)
    assert np.array_equal(ours, ref)


def test_e4m3_roundtrip_every_finite_code():
    table = oracle.e4m3_decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(float(table[c])) == c


def test_e4m3_saturation_and_specials():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(float(np.nextafter(np.float32(448), np.float32(1e9)))) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E and oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(float("inf")) == 0x7E and oracle.e4m3_encode(float("-inf")) == 0xFE
    assert oracle.e4m3_encode(float("nan")) == 0x7F
    assert oracle.e4m3_encode(-0.0) == 0x80 and oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-1e-30) == 0x80           # underflow keeps the sign
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00        # tie between 0 and 2^-9 goes to even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02    # tie between 1 and 2 (x 2^-9) goes to 2
