"""Pins for the oracle's log-sum-exp output (the natural-log normaliser of the
softmax over one query row's dequantized scores).

 - closed forms: one key (the score itself) and equal scores (score + ln S);
 - the log-sum-exp of the scores recomputed here in fp64 directly from the INT8
   codes and block scales, with no tiling: the tiled running-max form must
   agree within the rounding of the float score constant and of l;
 - the key-tile size does not change it beyond that rounding;
 - against fp64 exact attention's log-sum-exp on unquantized inputs, within
   max_j |s_quantized - s_exact| (the log-sum-exp is 1-Lipschitz in the
   maximum norm of its arguments), computed here from the data.
"""
import math

import numpy as np
import pytest

import oracle
import synth

LN2 = math.log(2.0)
LOG2E_F32 = np.float32(1.4426950408889634)


def _prep_head(S, seed, smooth_k=False, qscale=1.0):
    w = synth.custom(1, S, 1, smooth_k=smooth_k, base_seed=seed)
    q, k, v = (synth.tensor(w, x)[0, :, 0] for x in "qkv")
    if qscale != 1.0:
        import torch
        qf = torch.from_numpy(synth.bf16_to_float(q) * qscale).to(torch.bfloat16)
        q = qf.view(torch.int16).numpy().view(np.uint16)
    return q, k, v, oracle.prepare_head(q, k, v, smooth_k)


def _scores_fp64(p, rows, sm_scale):
    """Dequantized scores acc * q_scale * k_scale * sm_scale in fp64, from the codes."""
    q8 = p["q8"].astype(np.int64)
    k8 = p["k8"].astype(np.int64)
    S = q8.shape[0]
    acc = q8[rows] @ k8[:S].T                                              # exact integers
    qs = p["q_scale"].astype(np.float64)[np.asarray(rows) // 32][:, None]
    ks = p["k_scale"].astype(np.float64)[np.arange(S) // 32][None, :]
    return acc * qs * ks * sm_scale


def _logsumexp(s):
    m = s.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=1, keepdims=True)))[:, 0]


def _rounding_bound(s, S):
    # t = float(acc) * float(float(qs * ks) * float(sm * log2e)): a few float roundings of
    # each score (relative 2^-22 covers them) plus the float sum l over S terms
    return 4 * 2.0 ** -23 * np.abs(s).max(axis=1) + S * 2.0 ** -23 + 1e-7


def test_single_key_is_its_score():
    q, k, v, p = _prep_head(1, 11, qscale=2.0)
    _, lse = oracle.attn_rows_head(p, [0], 0.088, want_lse=True)
    s = _scores_fp64(p, [0], 0.088)
    assert abs(lse[0] - s[0, 0]) <= 4 * 2.0 ** -23 * abs(s[0, 0]) + 1e-7


@pytest.mark.parametrize("S", [7, 128, 300])
def test_equal_scores_add_ln_s(S):
    q, k, v, p = _prep_head(S, 12)
    p = dict(p)
    p["k8"] = np.ascontiguousarray(np.broadcast_to(p["k8"][0:1], p["k8"].shape))       # every key = key 0
    p["k_scale"] = np.full_like(p["k_scale"], p["k_scale"][0])
    rows = np.arange(0, S, max(1, S // 5))
    _, lse = oracle.attn_rows_head(p, rows, 0.088, want_lse=True)
    s = _scores_fp64(p, rows, 0.088)[:, 0]
    assert np.all(np.abs(lse - (s + math.log(S))) <= 4 * 2.0 ** -23 * np.abs(s) + S * 2.0 ** -23 + 1e-6)


@pytest.mark.parametrize("S,qscale,seed", [(300, 1.0, 13), (700, 3.0, 14), (129, 0.2, 15)])
def test_matches_untiled_fp64_logsumexp_of_the_codes(S, qscale, seed):
    q, k, v, p = _prep_head(S, seed, qscale=qscale)
    rows = np.arange(S)
    _, lse = oracle.attn_rows_head(p, rows, 0.088, want_lse=True)
    s = _scores_fp64(p, rows, 0.088)
    ref = _logsumexp(s)
    assert np.all(np.abs(lse - ref) <= _rounding_bound(s, S))


def test_tile_size_changes_only_rounding():
    S = 500
    q, k, v, p = _prep_head(S, 16, qscale=2.0)
    rows = np.arange(0, S, 3)
    s = _scores_fp64(p, rows, 0.088)
    a = oracle.attn_rows_head(p, rows, 0.088, T=128, want_lse=True)[1]
    b = oracle.attn_rows_head(p, rows, 0.088, T=16, want_lse=True)[1]
    c = oracle.attn_rows_head(p, rows, 0.088, T=S, want_lse=True)[1]
    bound = 2 * _rounding_bound(s, S)
    assert np.all(np.abs(a - b) <= bound) and np.all(np.abs(a - c) <= bound)


@pytest.mark.parametrize("S,smooth_k,seed", [(200, False, 17), (333, True, 18)])
def test_within_the_score_perturbation_of_exact(S, smooth_k, seed):
    q, k, v, p = _prep_head(S, seed, smooth_k=smooth_k, qscale=2.0)
    rows = np.arange(0, S, 7)
    sm = 1.0 / math.sqrt(128)
    _, lse = oracle.attn_rows_head(p, rows, sm, want_lse=True)
    _, lse_exact = oracle.exact_rows_head(q, k, v, rows, sm, want_lse=True)
    s_q = _scores_fp64(p, rows, sm)
    # exact scores; with smooth_k the subtracted mean shifts every score of a row
    # by q.mean, which softmax ignores but the log-sum-exp does not
    qf = synth.bf16_to_float(q).astype(np.float64)
    kf = synth.bf16_to_float(k).astype(np.float64)
    if smooth_k:
        kf = kf - p["k_mean"].astype(np.float64)[None, :]
    s_e = (qf[rows] @ kf.T) * sm
    shift = 0.0
    if smooth_k:
        shift = (qf[rows] @ p["k_mean"].astype(np.float64)) * sm
    perturb = np.abs(s_q - s_e).max(axis=1)
    assert np.all(np.abs((lse + shift) - lse_exact) <= perturb + _rounding_bound(s_q, S) + 1e-9)
