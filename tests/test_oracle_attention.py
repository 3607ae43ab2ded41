"""Pins for the oracle's quantized attention and its fp64 exact attention.

 - hand-worked cases in which every quantity is exactly representable, so the
   method must equal softmax attention computed here in rational arithmetic
   (several key tiles, running-max rescaling, FP8 P, v_scale, 448 scaling);
 - a hand-worked case where P is not representable (RNE to E4M3 by hand) and
   one where a tiny probability underflows FP8 but still counts in l;
 - closed-form special cases (one key; all scores equal; V = 1 gives the
   softmax row sum; one key far above the rest gives that key's value);
 - fp64 exact attention against torch's scaled_dot_product_attention in
   float64 (a library routine);
 - the quantized method against fp64 exact attention within an error bound
   derived from the quantization steps (not from the pages).
"""
import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
import synth

LOG2E_F32 = np.float32(1.4426950408889634)


def unit_sm_scale():
    """A float sm_scale with float32(sm_scale * log2(e)) == 1 exactly, so scores are exact integers."""
    s = np.float32(1.0 / float(LOG2E_F32))
    for _ in range(64):
        if np.float32(s * LOG2E_F32) == np.float32(1.0):
            return float(s)
        s = np.nextafter(s, np.float32(1.0))
    raise AssertionError("no unit sm_scale found")


def e4m3_code(value: float) -> int:
    """Code of an exactly representable E4M3 value (looked up in torch's table)."""
    import torch
    table = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    hits = [c for c in range(256) if table[c] == value and not (value == 0 and c == 0x80)]
    assert hits, value
    return hits[0]


def make_head(S, D=128):
    return dict(q8=np.zeros((S, D), np.int8), q_scale=np.ones(-(-S // 32), np.float32),
                k8=np.zeros((S, D), np.int8), k_scale=np.ones(-(-S // 32), np.float32),
                v8t=np.zeros((D, oracle.s_pad(S, 4) if S % 4 else S), np.uint8), v_scale=np.ones(D, np.float32))


def correctly_rounded_f32(val: np.float32, exact: Fr) -> bool:
    v = Fr(float(val))
    up = Fr(float(np.nextafter(val, np.float32(np.inf))))
    dn = Fr(float(np.nextafter(val, np.float32(-np.inf))))
    return abs(v - exact) <= abs(up - exact) and abs(v - exact) <= abs(dn - exact)


def bf16_of(x: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- hand-worked, exact
def test_three_tiles_with_rescaling_equals_exact_softmax():
    # Scores (log2 units) for one query over 12 keys, tiles of T=4:
    #   tile 0: 0 -1 -2 -3   (running max 0)
    #   tile 1: 2  0 -1  1   (max rises to 2: alpha = 1/4)
    #   tile 2: -5 -4 2 -10  (max stays 2: alpha = 1)
    # Every 448*p is an E4M3 value (448, 224, 112, 56, 3.5, 7, 0.109375), every
    # sum is exact in float, so the result must be the exact softmax
    # sum_j 2^(t_j - 2) v_j / sum_j 2^(t_j - 2), rounded once at the division.
    S, T = 12, 4
    t = [0, -1, -2, -3, 2, 0, -1, 1, -5, -4, 2, -10]
    rng = np.random.default_rng(1)
    vals = [0.5, 1.0, 1.5, 2.0, 3.0, -0.5, -1.0, -1.5, -2.0, -3.0, 0.25, 0.75]
    V = rng.choice(vals, size=(S, 128))
    h = make_head(S)
    h["q8"][0, 0] = 1
    for j in range(S):
        h["k8"][j, 0] = t[j]
        for d in range(128):
            h["v8t"][d, j] = e4m3_code(V[j, d])
    h["v_scale"][:] = 1.0
    ob, of = oracle.attn_rows_head(h, [0], unit_sm_scale(), T=T, want_f32=True)
    w = [Fr(2) ** (tj - 2) for tj in t]
    den = sum(w)
    assert den == Fr(3367431640625, 10 ** 12)  # 3.367431640625 = 0.46875 + 1.875 + 1.023681640625
    for d in range(128):
        exact = sum(wj * Fr(float(V[j, d])) for j, wj in enumerate(w)) / den
        assert correctly_rounded_f32(of[0, d], exact), d
    assert np.array_equal(ob[0], bf16_of(of[0]))


def test_later_tile_below_running_max_is_quantized_against_running_max():
    # T=4. Tile 0 scores 0 -1 -2 -3 set the running max to 0. Tile 1 scores
    # -20 -21 -22 -23 stay below it, so their p = 2^-20..2^-23 are taken
    # against the running max: 448 p < 2^-10 underflows E4M3 to zero (no PV
    # contribution) while l still gains 1.875 * 2^-20. Against the tile's own
    # max they would have been 448, 224, 112, 56.
    S, T = 8, 4
    t = [0, -1, -2, -3, -20, -21, -22, -23]
    h = make_head(S)
    h["q8"][0, 0] = 1
    V = [1.0, 2.0, -1.5, 3.0, 448.0, 448.0, -448.0, 448.0]
    for j in range(S):
        h["k8"][j, 0] = t[j]
        h["v8t"][0, j] = e4m3_code(V[j])
    ob, of = oracle.attn_rows_head(h, [0], unit_sm_scale(), T=T, want_f32=True)
    num = sum(Fr(2) ** t[j] * Fr(V[j]) for j in range(4))
    den = Fr(15, 8) * (1 + Fr(1, 2 ** 20))
    assert correctly_rounded_f32(of[0, 0], num / den)


def test_block_scales_use_the_query_and_key_block_of_each_pair():
    # S=64: query 40 lies in q block 1 (scale 1); q block 0 has scale 1000 so a
    # wrong block would blow the scores up. All keys have acc = -1; key block 1
    # has k_scale 2, so scores are -1 (keys 0..31) and -2 (keys 32..63).
    # Exact: (32*1*1 + 32*0.5*3) / (32 + 16) = 5/3 in channel 0.
    S = 64
    h = make_head(S)
    h["q_scale"][:] = [1000.0, 1.0]
    h["k_scale"][:] = [1.0, 2.0]
    h["q8"][40, 0] = 1
    h["k8"][:, 0] = -1
    h["v8t"][0, :32] = e4m3_code(1.0)
    h["v8t"][0, 32:] = e4m3_code(3.0)
    ob, of = oracle.attn_rows_head(h, [40], unit_sm_scale(), T=128, want_f32=True)
    assert correctly_rounded_f32(of[0, 0], Fr(5, 3))
    assert np.all(of[0, 1:] == 0)


def test_p_rounds_to_nearest_even_e4m3_by_hand():
    # Two keys, scores 0 and -1/2 (acc 0 and -1, q_scale 1/2): p = 1 and 2^-0.5.
    # 448 * 2^-0.5 = 316.78...; E4M3 neighbours at exponent 8 are 288, 320 (step
    # 32): nearest is 320. So O = (448 v0 + 320 v1) / (448 l), l = 1 + 2^-0.5.
    S = 2
    h = make_head(S)
    h["q_scale"][:] = 0.5
    h["q8"][0, 0] = 1
    h["k8"][1, 0] = -1
    h["v8t"][0, 0] = e4m3_code(1.0)
    h["v8t"][0, 1] = e4m3_code(2.0)
    ob, of = oracle.attn_rows_head(h, [0], unit_sm_scale(), T=128, want_f32=True)
    l = np.float32(1.0) + np.float32(2.0 ** -0.5)
    expected = (448.0 + 320.0 * 2.0) / (448.0 * float(l))
    assert abs(float(of[0, 0]) - expected) <= 2e-7 * expected
    unquantized = (448.0 + 448.0 * 2.0 ** -0.5 * 2.0) / (448.0 * float(l))
    assert abs(float(of[0, 0]) - unquantized) > 1e-3   # P really went through FP8


def test_underflowing_probability_counts_in_l_but_not_in_pv():
    # Scores 0 and -20: 448 * 2^-20 < 2^-10 rounds to E4M3 zero, but l = 1 + 2^-20.
    S = 2
    h = make_head(S)
    h["q8"][0, 0] = 1
    h["k8"][1, 0] = -20
    h["v8t"][0, 0] = e4m3_code(1.0)
    h["v8t"][0, 1] = e4m3_code(448.0)
    ob, of = oracle.attn_rows_head(h, [0], unit_sm_scale(), T=128, want_f32=True)
    assert correctly_rounded_f32(of[0, 0], Fr(1) / (1 + Fr(1, 2 ** 20)))


@pytest.mark.parametrize("jstar", [5, 200, 299])
def test_one_hot_row_returns_that_keys_value(jstar):
    # One key 30 log2 units (about 20.8 in natural log) above all others, with
    # real V codes everywhere: the others' 448 * 2^-30 rounds to E4M3 zero once
    # the maximum is known, so the row is that key's dequantized V; keys seen
    # before it (p = 1 while their tile's maximum was 0) come in rescaled by
    # 2^-30. |O - v*| <= 2^-30 (S max|v| + S |v*|) plus a few float roundings.
    S = 300
    h = make_head(S)
    h["q8"][0, 0] = 1
    h["k8"][jstar, 0] = 30
    rng = np.random.default_rng(90 + jstar)
    codes = rng.integers(0, 0x7F, size=(128, S)).astype(np.uint8) | (rng.integers(0, 2, size=(128, S)) << 7).astype(np.uint8)
    h["v8t"][:, :S] = codes
    ob, of = oracle.attn_rows_head(h, [0], unit_sm_scale(), T=128, want_f32=True)
    dec = oracle.e4m3_decode_table()[h["v8t"][:, :S]].astype(np.float64)    # [D, S]
    vstar = dec[:, jstar]
    vmax = np.abs(dec).max(axis=1)
    bound = 2.0 ** -30 * S * (vmax + np.abs(vstar)) + 4 * 2.0 ** -24 * np.abs(vstar) + 1e-30
    assert np.all(np.abs(of[0].astype(np.float64) - vstar) <= bound)
    # and it is not the plain mean: the other keys really are there
    assert not np.allclose(vstar, dec.mean(axis=1))


# ---------------------------------------------------------------- closed forms on prologue output
def _prep_head(S, seed, smooth_k=False, qscale=1.0):
    w = synth.custom(1, S, 1, smooth_k=smooth_k, base_seed=seed)
    q, k, v = (synth.tensor(w, x)[0, :, 0] for x in "qkv")
    if qscale != 1.0:
        q = bf16_of(synth.bf16_to_float(q) * qscale)
    return q, k, v, oracle.prepare_head(q, k, v, smooth_k)


def test_single_key_returns_its_dequantized_value():
    q, k, v, p = _prep_head(1, 5)
    ob, of = oracle.attn_rows_head(p, [0], 0.088, want_f32=True)
    dec = oracle.e4m3_decode_table()[p["v8t"][:, 0]].astype(np.float64) * p["v_scale"].astype(np.float64)
    assert np.allclose(of[0], dec, rtol=3e-7, atol=0)


@pytest.mark.parametrize("S", [5, 200, 300])
def test_equal_scores_give_the_mean_of_dequantized_v(S):
    q, k, v, p = _prep_head(S, 6, qscale=0.0)     # Q = 0: every score is 0
    assert not p["q8"].any()
    ob, of = oracle.attn_rows_head(p, np.arange(S), 0.088, want_f32=True)
    dec = oracle.e4m3_decode_table()[p["v8t"][:, :S]].astype(np.float64)       # [D, S]
    mean = dec.mean(axis=1) * p["v_scale"].astype(np.float64)
    assert np.allclose(of, mean[None, :], rtol=S * 2.0 ** -22, atol=1e-12)


@pytest.mark.parametrize("S", [50, 257])
def test_v_all_ones_gives_the_fp8_softmax_row_sum(S):
    q, k, v, p = _prep_head(S, 7, qscale=3.0)
    p = dict(p)
    p["v8t"] = np.where(np.arange(p["v8t"].shape[1])[None, :] < S, e4m3_code(1.0), 0).astype(np.uint8)
    p["v8t"] = np.ascontiguousarray(np.broadcast_to(p["v8t"], (128, p["v8t"].shape[1])))
    p["v_scale"] = np.ones(128, np.float32)
    ob, of = oracle.attn_rows_head(p, np.arange(S), 0.088, want_f32=True)
    # sum_j dec(p8_j) alpha / (448 l) is within the E4M3 half-ulp of 1, minus underflow
    assert np.all(of <= 1 + 2.0 ** -4 + 1e-6)
    assert np.all(of >= 1 - 2.0 ** -4 - S * 2.0 ** -10 / 448 - 1e-6)
    assert np.all(of[:, 0:1] == of)   # identical over channels


def test_tile_size_is_irrelevant_within_one_tile_and_relevant_across():
    q, k, v, p = _prep_head(128, 8, qscale=2.5)
    a = oracle.attn_rows_head(p, np.arange(128), 0.088, T=128)
    b = oracle.attn_rows_head(p, np.arange(128), 0.088, T=1024)
    assert np.array_equal(a, b)
    c = oracle.attn_rows_head(p, np.arange(128), 0.088, T=16)
    assert not np.array_equal(a, c)   # the key-tile schedule is part of the result


def test_v_times_power_of_two_scales_output_exactly():
    S = 96
    w = synth.custom(1, S, 2, smooth_k=True, base_seed=40)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    v4 = bf16_of(synth.bf16_to_float(v) * 4.0)
    o1 = oracle.attn(oracle.prepare(q, k, v, True), w.sm_scale)
    o4 = oracle.attn(oracle.prepare(q, k, v4, True), w.sm_scale)
    assert np.array_equal(synth.bf16_to_float(o1) * 4.0, synth.bf16_to_float(o4))


# ---------------------------------------------------------------- fp64 exact attention
def test_exact_rows_match_torch_sdpa_float64():
    import torch
    w = synth.custom(1, 77, 2, base_seed=50)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    ours = oracle.exact(q, k, v, 0.3)
    tq, tk, tv = (torch.from_numpy(synth.bf16_to_float(a).astype(np.float64)).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3).permute(0, 2, 1, 3).numpy()
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-13)


def test_exact_attention_is_invariant_to_a_per_channel_key_shift():
    # softmax cancels a key-independent score offset: exact attention with K and
    # K + c (c per channel, BF16-exact) agree to rounding. This is the reason
    # smooth_k is allowed to subtract the key mean.
    rng = np.random.default_rng(60)
    S = 64
    kf = (np.round(np.clip(rng.standard_normal((1, S, 1, 128)), -7, 7) * 16) / 16).astype(np.float32)
    c = np.round(rng.uniform(-3, 3, 128)).astype(np.float32)
    qf = rng.standard_normal((1, S, 1, 128)).astype(np.float32)
    vf = rng.standard_normal((1, S, 1, 128)).astype(np.float32)
    q, k, kc, v = (np.ascontiguousarray(bf16_of(a)) for a in (qf, kf, kf + c, vf))
    assert np.array_equal(synth.bf16_to_float(kc), kf + c)
    e0 = oracle.exact(q, k, v, 0.1)
    e1 = oracle.exact(q, kc, v, 0.1)
    assert np.max(np.abs(e0 - e1)) < 1e-11


# ---------------------------------------------------------------- method vs exact, derived bound
def error_bound(qf, kf, vf, prep, sm_scale, smooth_k, rows):
    """Worst-case |O - O*| per (row, channel) implied by the quantization steps.

    Score error (natural-log units) for query i and key j, with k~ the smoothed
    key actually quantized:  E_ij = sm * ((1/2 + 2^-15) q_s ||k~_j||_1
    + (1/2 + 2^-15) k_s ||q_i||_1 + D/4 q_s k_s) plus float slack; E_i = max_j.
    Then pi^_j / pi_j lies in [e^-2E, e^2E]; FP8 P has relative error 2^-4
    (absolute 2^-10 / 448 below the normal range, relative to the final max);
    FP8 V has |v - v~| <= 2^-4 |v| + 2^-10 v_scale; BF16 output adds 2^-8 |O|:
      B = (e^2E (17/16)^2 - 1) sum_j pi_j |v_j| + (17/16) 2^-10 v_scale
          + S (2^-10/448) ((17/16) max|v| + 2^-10 v_scale) + 2^-8 (|O*| + core)
          + S 2^-22 (17/16)^2 e^2E sum_j pi_j |v_j|        (float sums)
    """
    S, D = qf.shape
    ktil = kf - prep["k_mean"][None, :] if smooth_k else kf
    ktil = ktil.astype(np.float32).astype(np.float64)
    qs = np.repeat(prep["q_scale"].astype(np.float64), 32)[:S]
    ks = np.repeat(prep["k_scale"].astype(np.float64), 32)[:S]
    q1 = np.abs(qf).sum(axis=1)
    k1 = np.abs(ktil).sum(axis=1)
    vs = prep["v_scale"].astype(np.float64)
    out = []
    for i in rows:
        s = qf[i] @ kf.T * sm_scale
        Eij = sm_scale * ((0.5 + 2 ** -15) * qs[i] * k1 + (0.5 + 2 ** -15) * ks * q1[i] + D / 4 * qs[i] * ks)
        E = Eij.max() + 1e-5 * (1 + np.abs(s).max())
        pi = np.exp(s - s.max())
        pi /= pi.sum()
        spv = pi @ np.abs(vf)
        core = (math.exp(2 * E) * (17 / 16) ** 2 - 1) * spv + (17 / 16) * 2.0 ** -10 * vs \
            + S * (2.0 ** -10 / 448) * ((17 / 16) * np.abs(vf).max(axis=0) + 2.0 ** -10 * vs) \
            + S * 2.0 ** -22 * (17 / 16) ** 2 * math.exp(2 * E) * spv
        ostar = pi @ vf
        out.append(core + 2.0 ** -8 * (np.abs(ostar) + core) + 1e-30)
    return np.array(out)


@pytest.mark.parametrize("S,smooth_k,qk_scale,seed", [(32, False, 1.0, 70), (100, True, 1.0, 71), (256, False, 2.0, 72),
                                                      (256, True, 3.0, 73), (33, True, 0.5, 74)])
def test_method_within_derived_bound_of_exact(S, smooth_k, qk_scale, seed):
    w = synth.custom(1, S, 2, smooth_k=smooth_k, base_seed=seed)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    if qk_scale != 1.0:
        q = np.ascontiguousarray(bf16_of(synth.bf16_to_float(q) * qk_scale))
        k = np.ascontiguousarray(bf16_of(synth.bf16_to_float(k) * qk_scale))
    sm = w.sm_scale
    prep = oracle.prepare(q, k, v, smooth_k)
    O = oracle.bf16_bits_to_f64(oracle.attn(prep, sm))
    E = oracle.exact(q, k, v, sm)
    for h in range(2):
        qf, kf, vf = (synth.bf16_to_float(a[0, :, h]).astype(np.float64) for a in (q, k, v))
        bound = error_bound(qf, kf, vf, oracle.head_of(prep, 0, h), sm, smooth_k, range(S))
        err = np.abs(O[0, :, h] - E[0, :, h])
        assert np.all(err <= bound), (h, float((err / bound).max()))
        # the bound is loose; the typical error is far inside it
        assert np.median(err / bound) < 0.2


def test_c1_accuracy_against_exact():
    w = synth.WORKLOADS["C1"]
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    O = oracle.bf16_bits_to_f64(oracle.attn(oracle.prepare(q, k, v, w.smooth_k), w.sm_scale))
    E = oracle.exact(q, k, v, w.sm_scale)
    assert oracle.cosine(O, E) >= 0.999
