"""Pins for the oracle's causal rows. The pages reject causal attention; the
library offers it as an extension with the usual meaning for equal query and
key lengths: query i sees keys 0 .. i (torch's scaled_dot_product_attention
with is_causal=True draws the same line), over the same key tiles from key 0.

 - closed forms: row 0 is the dequantized V row 0 (one key, p = 1, and 448 is
   an E4M3 value); with every score equal, row i is the mean of the dequantized
   V rows 0 .. i and its log-sum-exp is s + ln(i + 1) (so one key too many or
   too few fails);
 - the last row sees every key, so it is the non-causal row bit for bit;
 - fp64 exact causal attention against torch's SDPA with is_causal in float64;
 - the method against fp64 exact causal attention within the bound derived
   from the quantization steps (the non-causal bound over keys 0 .. i), on rows
   on both sides of key-tile boundaries;
 - the log-sum-exp against an untiled fp64 log-sum-exp of the codes over keys
   0 .. i, within the rounding of the float score constant and of l.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from test_oracle_attention import bf16_of, error_bound


def _prep_head(S, seed, smooth_k=False, qscale=1.0):
    w = synth.custom(1, S, 1, smooth_k=smooth_k, base_seed=seed)
    q, k, v = (synth.tensor(w, x)[0, :, 0] for x in "qkv")
    if qscale != 1.0:
        q = bf16_of(synth.bf16_to_float(q) * qscale)
    return q, k, v, oracle.prepare_head(q, k, v, smooth_k)


def _dec_v(p, S):
    """Dequantized V [S, D] in fp64 from the codes and channel scales."""
    dec = oracle.e4m3_decode_table()[p["v8t"][:, :S]].astype(np.float64)      # [D, S]
    return (dec * p["v_scale"].astype(np.float64)[:, None]).T


def test_row0_is_the_dequantized_first_value_row():
    q, k, v, p = _prep_head(300, 80, qscale=2.0)
    _, of = oracle.attn_rows_head(p, [0], 0.088, want_f32=True, causal=True)
    assert np.allclose(of[0], _dec_v(p, 1)[0], rtol=3e-7, atol=0)


@pytest.mark.parametrize("S", [5, 200, 300])
def test_equal_scores_give_the_mean_of_the_first_i_plus_1_value_rows(S):
    q, k, v, p = _prep_head(S, 81, qscale=0.0)     # Q = 0: every score is 0
    assert not p["q8"].any()
    rows = np.unique(np.array([0, 1, 2, 31, 32, 127, 128, 129, 199, 255, 256, S - 1]).clip(0, S - 1))
    _, of, lse = oracle.attn_rows_head(p, rows, 0.088, want_f32=True, want_lse=True, causal=True)
    dv = _dec_v(p, S)
    for r, i in enumerate(rows):
        mean = dv[: i + 1].mean(axis=0)
        assert np.allclose(of[r], mean, rtol=(i + 1) * 2.0 ** -22, atol=1e-12), i
        # all scores 0: log-sum-exp = ln(i + 1)
        assert abs(lse[r] - math.log(i + 1)) <= (i + 1) * 2.0 ** -23 + 1e-7, i


def test_last_row_equals_the_non_causal_row():
    q, k, v, p = _prep_head(333, 82, qscale=2.0)
    rows = [332]
    a, fa, la = oracle.attn_rows_head(p, rows, 0.088, want_f32=True, want_lse=True, causal=True)
    b, fb, lb = oracle.attn_rows_head(p, rows, 0.088, want_f32=True, want_lse=True)
    assert np.array_equal(a, b) and np.array_equal(fa, fb) and np.array_equal(la, lb)
    # and an earlier row does not
    c = oracle.attn_rows_head(p, [200], 0.088, causal=True)
    d = oracle.attn_rows_head(p, [200], 0.088)
    assert not np.array_equal(c, d)


def test_exact_causal_rows_match_torch_sdpa_float64():
    import torch
    w = synth.custom(1, 77, 2, base_seed=83)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    ours = oracle.exact(q, k, v, 0.3, causal=True)
    tq, tk, tv = (torch.from_numpy(synth.bf16_to_float(a).astype(np.float64)).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3, is_causal=True)
    assert np.allclose(ours, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("S,smooth_k,qk_scale,seed", [(100, True, 1.0, 84), (300, False, 2.0, 85),
                                                      (260, True, 3.0, 86)])
def test_method_within_derived_bound_of_exact_causal(S, smooth_k, qk_scale, seed):
    w = synth.custom(1, S, 1, smooth_k=smooth_k, base_seed=seed)
    q, k, v = (synth.tensor(w, x) for x in "qkv")
    if qk_scale != 1.0:
        q = np.ascontiguousarray(bf16_of(synth.bf16_to_float(q) * qk_scale))
        k = np.ascontiguousarray(bf16_of(synth.bf16_to_float(k) * qk_scale))
    sm = w.sm_scale
    prep = oracle.prepare(q, k, v, smooth_k)
    O = oracle.bf16_bits_to_f64(oracle.attn(prep, sm, causal=True))[0, :, 0]
    E = oracle.exact(q, k, v, sm, causal=True)[0, :, 0]
    qf, kf, vf = (synth.bf16_to_float(a[0, :, 0]).astype(np.float64) for a in (q, k, v))
    ph = oracle.head_of(prep, 0, 0)
    ratios = []
    for i in sorted({min(r, S - 1) for r in (0, 1, 31, 32, 63, 127, 128, 129, S // 2, S - 2, S - 1)}):
        n = i + 1
        bound = error_bound(qf[:n], kf[:n], vf[:n], ph, sm, smooth_k, [i])[0]
        err = np.abs(O[i] - E[i])
        assert np.all(err <= bound), (i, float((err / bound).max()))
        ratios.append(np.median(err / bound))
    assert np.median(ratios) < 0.2


@pytest.mark.parametrize("S,qscale,seed", [(300, 1.0, 87), (260, 3.0, 88)])
def test_lse_matches_untiled_fp64_logsumexp_over_keys_up_to_i(S, qscale, seed):
    q, k, v, p = _prep_head(S, seed, qscale=qscale)
    rows = np.arange(S)
    _, lse = oracle.attn_rows_head(p, rows, 0.088, want_lse=True, causal=True)
    q8 = p["q8"].astype(np.int64)
    k8 = p["k8"].astype(np.int64)
    acc = q8 @ k8[:S].T
    qs = p["q_scale"].astype(np.float64)[rows // 32][:, None]
    ks = p["k_scale"].astype(np.float64)[np.arange(S) // 32][None, :]
    s = acc * qs * ks * 0.088
    s[np.arange(S)[None, :] > rows[:, None]] = -np.inf
    m = s.max(axis=1, keepdims=True)
    ref = (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]
    bound = 4 * 2.0 ** -23 * np.abs(np.where(np.isfinite(s), s, 0)).max(axis=1) + (rows + 1) * 2.0 ** -23 + 1e-7
    assert np.all(np.abs(lse - ref) <= bound)
