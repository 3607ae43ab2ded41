"""Head dim 64 in the oracle. The oracle is written for any D; these pins tie
D = 64 to D = 128 through an identity of the method: appending 64 zero
channels to Q, K and V changes nothing it computes on the first 64 channels
(block maxima and channel means over zeros add nothing, zero codes add 0 to
every integer score, zero V channels only add zero outputs), so the D = 128
results restricted to the first 64 channels must equal the D = 64 results bit
for bit: codes, scales, means, outputs and log-sum-exp. sm_scale is passed
explicitly (the same value to both)."""
import numpy as np
import pytest

import oracle
import synth


def _inputs(S, seed, smooth_k):
    w = synth.custom(1, S, 1, D=64, smooth_k=smooth_k, base_seed=seed)
    return [synth.tensor(w, x)[0, :, 0] for x in "qkv"]


def _pad(x):
    out = np.zeros((x.shape[0], 128), np.uint16)
    out[:, :64] = x
    return out


@pytest.mark.parametrize("S,smooth_k,seed", [(1, False, 91), (100, True, 92), (300, False, 93), (513, True, 94)])
def test_d64_equals_d128_with_zero_channels(S, smooth_k, seed):
    q, k, v = _inputs(S, seed, smooth_k)
    p64 = oracle.prepare_head(q, k, v, smooth_k)
    p128 = oracle.prepare_head(_pad(q), _pad(k), _pad(v), smooth_k)
    assert np.array_equal(p64["q8"], p128["q8"][:, :64]) and not p128["q8"][:, 64:].any()
    assert np.array_equal(p64["k8"], p128["k8"][:, :64]) and not p128["k8"][:, 64:].any()
    for key in ("q_scale", "k_scale"):
        assert np.array_equal(p64[key].view(np.uint32), p128[key].view(np.uint32)), key
    assert np.array_equal(p64["v8t"], p128["v8t"][:64]) and not p128["v8t"][64:].any()
    assert np.array_equal(p64["v_scale"].view(np.uint32), p128["v_scale"][:64].view(np.uint32))
    assert np.array_equal(p64["k_mean"].view(np.uint32), p128["k_mean"][:64].view(np.uint32))
    rows = np.arange(S)
    sm = 0.125
    b64, f64, l64 = oracle.attn_rows_head(p64, rows, sm, want_f32=True, want_lse=True)
    b128, f128, l128 = oracle.attn_rows_head(p128, rows, sm, want_f32=True, want_lse=True)
    assert np.array_equal(b64, b128[:, :64]) and not b128[:, 64:].any()
    assert np.array_equal(f64.view(np.uint32), f128[:, :64].view(np.uint32))
    assert np.array_equal(l64.view(np.uint32), l128.view(np.uint32))
    e64 = oracle.exact_rows_head(q, k, v, rows, sm)
    e128 = oracle.exact_rows_head(_pad(q), _pad(k), _pad(v), rows, sm)
    assert np.allclose(e64, e128[:, :64], rtol=1e-12, atol=1e-15)


def test_d64_within_its_error_bound_of_exact():
    # the method at D = 64 tracks exact attention as at D = 128 (cosine, as the GPU tests use it)
    S = 700
    q, k, v = _inputs(S, 95, True)
    p = oracle.prepare_head(q, k, v, True)
    rows = np.arange(0, S, 5)
    sm = 0.125
    _, f = oracle.attn_rows_head(p, rows, sm, want_f32=True)
    e = oracle.exact_rows_head(q, k, v, rows, sm)
    assert oracle.cosine(f.astype(np.float64), e) >= 0.999
