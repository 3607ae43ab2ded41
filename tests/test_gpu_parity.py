"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Prologue outputs (INT8 Q/K codes and scales, E4M3 V codes and scales, k_mean)
must match bit for bit. The attention output must satisfy, against the oracle
on the same inputs, max|O - O_oracle| <= 1e-2 max|O_oracle| and cosine >=
0.9995, and against fp64 exact attention cosine >= 0.999. Three named input
classes miss that last criterion with the oracle exactly as with the GPU, so
it is a property of the method there (METHOD_LIMITED below): for them the
GPU must not fall more than 2e-4 below the oracle's own cosine, the oracle
must indeed be below 0.999 (else the exception is stale), and the case is
recorded as a missed criterion.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

MAXABS_TOL = 1e-2
COS_ORACLE = 0.9995
COS_EXACT = 0.999
RESULTS = []
# Input classes on which the method itself (the oracle) stays below cosine
# 0.999 against fp64 exact attention, with the reason.
METHOD_LIMITED = {
    "C5": "1 % of K entries are N(0, 20^2) outliers, so per-32-row INT8 blocks quantize the ordinary keys "
          "to 2-3 levels",
    "qscale256": "Q scaled by 2^8: scores of hundreds of log2 units, rows close to one-hot, where the FP8 "
                 "rounding of the few non-negligible probabilities dominates",
    "causal_C3": "C3's per-head Q and K scales up to 3 make rows peaky (its non-causal rows reach only 0.99902); "
                 "causal rows, averaging fewer keys, fall just below",
}


@pytest.fixture(scope="module")
def sage():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import quantized_attention_prepare_amd as s
    s.lib()
    yield s
    # the per-case metrics go to SAGE_PARITY_OUT (a JSON-lines file) when it is set
    path = os.environ.get("SAGE_PARITY_OUT")
    if path:
        os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
        with open(path, "a") as f:
            for r in RESULTS:
                f.write(json.dumps(r) + "\n")


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def inputs(w):
    return [synth.tensor(w, x) for x in "qkv"]


def gpu_prepare(sage, q, k, v, smooth_k):
    import torch
    p = sage.prepare(to_dev(q), to_dev(k), to_dev(v), smooth_k)
    torch.cuda.synchronize()
    return {key: val.cpu().numpy() for key, val in p.items() if key not in ("S", "_ws")}


def check_prologue(g, o, S, heads=None, smooth_k=True):
    """Bit-exact comparison over the logical region and zero padding."""
    B, H, Sp, D = g["q8"].shape
    nb = -(-S // 32)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in todo:
        assert np.array_equal(g["q8"][b, h, :S], o["q8"][b, h]), ("q8", b, h)
        assert np.array_equal(g["k8"][b, h, :S], o["k8"][b, h]), ("k8", b, h)
        assert np.array_equal(g["q_scale"][b, h, :nb].view(np.uint32), o["q_scale"][b, h].view(np.uint32)), ("qs", b, h)
        assert np.array_equal(g["k_scale"][b, h, :nb].view(np.uint32), o["k_scale"][b, h].view(np.uint32)), ("ks", b, h)
        assert np.array_equal(g["v8t"][b, h, :, :S], o["v8t"][b, h, :, :S]), ("v8t", b, h)
        assert np.array_equal(g["v_scale"][b, h].view(np.uint32), o["v_scale"][b, h].view(np.uint32)), ("vs", b, h)
        assert np.array_equal(g["k_mean"][b, h].view(np.uint32), o["k_mean"][b, h].view(np.uint32)), ("km", b, h)
        assert not g["q8"][b, h, S:].any() and not g["k8"][b, h, S:].any() and not g["v8t"][b, h, :, S:].any()
        assert not g["q_scale"][b, h, nb:].any() and not g["k_scale"][b, h, nb:].any()


# ------------------------------------------------------------------ prologue
@pytest.mark.parametrize("name", ["C1", "C2", "C5", "C3"])
def test_prologue_bit_exact_workload(sage, name):
    w = synth.WORKLOADS[name]
    q, k, v = inputs(w)
    g = gpu_prepare(sage, q, k, v, w.smooth_k)
    o = oracle.prepare(q, k, v, w.smooth_k)
    check_prologue(g, o, w.S)


def test_prologue_bit_exact_c4_sampled_heads(sage):
    w = synth.WORKLOADS["C4"]
    q, k, v = inputs(w)
    g = gpu_prepare(sage, q, k, v, w.smooth_k)
    heads = [(0, 0), (0, 13), (0, 27)]
    o = oracle.prepare(q, k, v, w.smooth_k, heads=heads)
    check_prologue(g, o, w.S, heads=heads)


@pytest.mark.parametrize("B,S,H", [(1, 1, 1), (2, 33, 3), (1, 300, 2), (3, 1000, 2), (1, 4097, 1), (2, 127, 5)])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_prologue_bit_exact_ragged(sage, B, S, H, smooth_k):
    w = synth.custom(B, S, H, smooth_k=smooth_k, base_seed=1000 + S)
    q, k, v = inputs(w)
    check_prologue(gpu_prepare(sage, q, k, v, smooth_k), oracle.prepare(q, k, v, smooth_k), S)


@pytest.mark.parametrize("B,S,H,D", [(1, 512, 3, 128), (2, 385, 2, 64), (1, 128, 4, 128), (3, 129, 2, 64),
                                     (1, 513, 2, 128), (2, 512, 2, 64)])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_prologue_bit_exact_short_heads(sage, B, S, H, D, smooth_k):
    """Short heads (one to five 128-row chunks, full and ragged), both head
    dims: few statistics partials per head, a single chunk per head."""
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=8300 + S + D)
    q, k, v = inputs(w)
    check_prologue(gpu_prepare(sage, q, k, v, smooth_k), oracle.prepare(q, k, v, smooth_k), S)


def test_e4m3_conversion_of_every_in_range_bf16(sage):
    # channel 0 of V holds every BF16 value of magnitude <= 448 (both signs) and
    # the value 448 itself, so its scale is exactly 1 and the codes are
    # E4M3(v): the hardware conversion is compared with the oracle's encoder on
    # every such value, including ties and subnormal-range inputs.
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = synth.bf16_to_float(bits)
    bits = bits[vals <= 448.0]
    allb = np.concatenate([bits, bits | 0x8000, np.array([0x43E0], np.uint16)])   # 0x43E0 = 448
    S = allb.size
    w = synth.custom(1, S, 1, base_seed=77)
    q, k, v = inputs(w)
    v = v.copy()
    v[0, :, 0, 0] = allb
    g = gpu_prepare(sage, q, k, v, False)
    o = oracle.prepare(q, k, v, False)
    assert o["v_scale"][0, 0, 0] == 1.0
    check_prologue(g, o, S)


def test_prologue_is_deterministic(sage):
    w = synth.WORKLOADS["C2"]
    q, k, v = inputs(w)
    a = gpu_prepare(sage, q, k, v, True)
    b = gpu_prepare(sage, q, k, v, True)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def _scaled(bits, factor):
    """BF16 bits times a power of two, rounded back to BF16 by torch (values
    pushed among the BF16 subnormals lose low bits; both sides see the result)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).float() * factor
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("smooth_k", [False, True])
def test_tiny_blocks_and_channels(sage, D, smooth_k):
    """Blocks and channels whose absmax a makes 127/a or 448/a overflow a float
    (a below about 3.7e-37 and 1.3e-36; BF16 subnormals reach 9.2e-41): the
    prologue lifts them by 2^64 exactly as the oracle does, bit for bit; the
    output is finite and within tolerance of the oracle. A V channel of +-0
    only has scale 0 and codes 0 (its negative zeros too)."""
    import torch
    B, S, H = 2, 300, 3
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=8100 + D + int(smooth_k))
    q, k, v = (x.copy() for x in inputs(w))
    q[0, 32:64, 0] = _scaled(q[0, 32:64, 0], 2.0 ** -124)        # one tiny Q block
    q[1, :, 1] = _scaled(q[1, :, 1], 2.0 ** -130)                # a whole head of tiny Q (scores vanish)
    k[0, 64:96, 1] = _scaled(k[0, 64:96, 1], 2.0 ** -126)        # a tiny K block (smooth_k off)
    k[1, :, 2] = _scaled(k[1, :, 2], 2.0 ** -125)                # a tiny K head: K - mean stays tiny
    v[0, :, 0, 5] = _scaled(v[0, :, 0, 5], 2.0 ** -122)          # V channel with 448/a overflowing
    v[1, :, 2, 9] = _scaled(v[1, :, 2, 9], 2.0 ** -60)           # lifted, quotient finite either way
    v[0, :, 1, 3] = _scaled(v[0, :, 1, 3], 2.0 ** -140)          # all +-0: a zero channel with negative zeros
    v[0, :, 1, 4] = _scaled(v[0, :, 1, 4], 2.0 ** -128)          # BF16 subnormals with few bits
    o = oracle.prepare(q, k, v, smooth_k)
    assert o["q_scale"][0, 0, 1] < 3.7e-37 and o["v_scale"][0, 0, 5] < 1.3e-36 / 448
    assert o["v_scale"][0, 1, 3] == 0 and np.any(v[0, :, 1, 3] == 0x8000) and o["v_scale"][0, 1, 4] > 0
    g = gpu_prepare(sage, q, k, v, smooth_k)
    check_prologue(g, o, S, smooth_k=smooth_k)
    out = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, False, smooth_k)
    torch.cuda.synchronize()
    O = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(O)))
    compare_attention(f"tiny_{D}_{'sk' if smooth_k else 'nosk'}", O, oracle.attn(o, w.sm_scale),
                      oracle.exact(q, k, v, w.sm_scale))


def _adversarial_keys(k, rng):
    """Key channels whose fp64 running sums are not exact: 2^60, 1, -2^60, ...;
    2^70 and 2^-70 of both signs; subnormals beside 2^100; one channel of random
    exponents over the whole BF16 range."""
    import torch
    B, S, H, D = k.shape
    f = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).float()
    s = torch.arange(S)
    f[:, :, :, 0] = torch.tensor([2.0 ** 60, 1.0, -(2.0 ** 60)])[s % 3][None, :, None]
    f[:, :, :, 1] = (torch.where(s % 2 == 0, 2.0 ** 70, 2.0 ** -70) * torch.where(s % 4 < 2, 1.0, -1.0))[None, :, None]
    f[:, :, :, 2] = torch.where(s % 7 == 0, 2.0 ** 100, 2.0 ** -130)[None, :, None]
    e = torch.from_numpy(rng.integers(-130, 110, (B, S, H))).float()
    f[:, :, :, 3] = torch.from_numpy(rng.standard_normal((B, S, H))).float() * torch.pow(2.0, e)
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("B,S,H,D", [(1, 300, 2, 128), (2, 20000, 2, 128), (1, 4097, 3, 64)])
def test_k_mean_exact_on_adversarial_channels(sage, B, S, H, D):
    """smooth_k on key channels whose fp64 sums depend on the order of
    addition: the GPU's checked fp64 sums fall back to exact integer sums and
    k_mean (and with it every K code) matches the oracle's correctly rounded
    mean bit for bit. The attention output (rows made near one-hot by keys of
    magnitude 2^60 and more) is compared with the oracle only."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=True, base_seed=8200 + S)
    q, k, v = inputs(w)
    k = _adversarial_keys(k, np.random.default_rng(S))
    o = oracle.prepare(q, k, v, True)
    kd = synth.bf16_to_float(k[0, :, 0, 0]).astype(np.float64)
    assert o["k_mean"][0, 0, 0] == np.float32(math.fsum(kd.tolist()) / S)
    g = gpu_prepare(sage, q, k, v, True)
    check_prologue(g, o, S)
    if S <= 4097:
        out = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, False, True)
        torch.cuda.synchronize()
        compare_attention(f"adversarial_kmean_{B}x{S}x{H}x{D}", out.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.attn(o, w.sm_scale), None)


# ------------------------------------------------------------------ attention
def run_sageattn(sage, q, k, v, smooth_k, sm_scale):
    import torch
    out = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, sm_scale, False, smooth_k)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def compare_attention(name, O_gpu_bits, O_orc_bits, E, limited=None):
    """limited: a key of METHOD_LIMITED for the input classes where the method
    itself misses cosine 0.999 against exact attention; E None: no exact
    reference for this case (only the oracle bounds apply)."""
    G = oracle.bf16_bits_to_f64(O_gpu_bits)
    R = oracle.bf16_bits_to_f64(O_orc_bits)
    rec = dict(case=name, maxabs_vs_oracle=oracle.max_abs_rel(G, R), cos_vs_oracle=oracle.cosine(G, R),
               bits_equal_frac=float(np.mean(O_gpu_bits == O_orc_bits)))
    if E is not None:
        rec.update(cos_vs_exact=oracle.cosine(G, E), oracle_cos_vs_exact=oracle.cosine(R, E),
                   maxabs_vs_exact=oracle.max_abs_rel(G, E))
        if limited is not None:
            rec["criterion_missed"] = f"cosine vs exact {rec['cos_vs_exact']:.5f} < {COS_EXACT}: {METHOD_LIMITED[limited]}"
    RESULTS.append(rec)
    print(json.dumps(rec))
    assert rec["maxabs_vs_oracle"] <= MAXABS_TOL, rec
    assert rec["cos_vs_oracle"] >= COS_ORACLE, rec
    if E is None:
        return
    if limited is None:
        assert rec["cos_vs_exact"] >= COS_EXACT, rec
    else:
        assert rec["oracle_cos_vs_exact"] < COS_EXACT, ("stale exception", limited, rec)
        assert rec["cos_vs_exact"] >= rec["oracle_cos_vs_exact"] - 2e-4, rec


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_attention_workload(sage, name):
    """Every row against the oracle for C1, C2 and C5, seeded samples of 8192
    (C3) and 512 (C4) rows; fp64 exact attention on every row of C1 and C5 and
    on 8192 sampled rows of C2."""
    w = synth.WORKLOADS[name]
    q, k, v = inputs(w)
    O = run_sageattn(sage, q, k, v, w.smooth_k, w.sm_scale)
    if name in ("C1", "C2", "C5"):
        rows = None
    else:
        rows = synth.sample_rows(w, {"C3": 8192, "C4": 512}[name])
    heads = None if rows is None else sorted({(int(b), int(h)) for b, h, _ in rows})
    prep = oracle.prepare(q, k, v, w.smooth_k, heads=heads)
    R = oracle.attn(prep, w.sm_scale, rows=rows)
    if name == "C2":
        # all 114 688 rows against the oracle; fp64 exact on a seeded sample
        G, Rf = oracle.bf16_bits_to_f64(O), oracle.bf16_bits_to_f64(R)
        rec = dict(case="C2_all_rows", maxabs_vs_oracle=oracle.max_abs_rel(G, Rf), cos_vs_oracle=oracle.cosine(G, Rf),
                   bits_equal_frac=float(np.mean(O == R)))
        RESULTS.append(rec)
        print(json.dumps(rec))
        assert rec["maxabs_vs_oracle"] <= MAXABS_TOL and rec["cos_vs_oracle"] >= COS_ORACLE, rec
        rows = synth.sample_rows(w, 8192)
        E = oracle.exact(q, k, v, w.sm_scale, rows=rows)
        compare_attention(name, O[rows[:, 0], rows[:, 2], rows[:, 1]], R[rows[:, 0], rows[:, 2], rows[:, 1]], E)
        return
    E = oracle.exact(q, k, v, w.sm_scale, rows=rows)
    G = O if rows is None else O[rows[:, 0], rows[:, 2], rows[:, 1]]
    compare_attention(name, G, R, E, limited="C5" if name == "C5" else None)


@pytest.mark.parametrize("B,S,H,smooth_k", [(1, 1, 1, False), (2, 33, 3, True), (1, 129, 2, False),
                                             (2, 300, 3, True), (1, 1000, 2, True), (3, 127, 1, False)])
def test_attention_ragged(sage, B, S, H, smooth_k):
    w = synth.custom(B, S, H, smooth_k=smooth_k, base_seed=2000 + S)
    q, k, v = inputs(w)
    O = run_sageattn(sage, q, k, v, smooth_k, w.sm_scale)
    R = oracle.attn(oracle.prepare(q, k, v, smooth_k), w.sm_scale)
    E = oracle.exact(q, k, v, w.sm_scale)
    compare_attention(f"ragged{B}x{S}x{H}", O, R, E)


# ------------------------------------------------------------------ log-sum-exp
LSE_ABS, LSE_REL = 5e-5, 2e-6   # float sums of l in different orders, hardware exp2/log2


def check_lse(name, lse_gpu, lse_orc):
    d = np.abs(lse_gpu.astype(np.float64) - lse_orc.astype(np.float64))
    tol = LSE_ABS + LSE_REL * np.abs(lse_orc.astype(np.float64))
    rec = dict(case=name, lse_max_abs_diff=float(d.max()), lse_max_over_tol=float((d / tol).max()))
    RESULTS.append(rec)
    print(json.dumps(rec))
    assert np.all(d <= tol), rec


@pytest.mark.parametrize("B,S,H,smooth_k", [(1, 1, 1, False), (2, 33, 3, True), (1, 300, 2, False),
                                             (2, 1000, 3, True)])
def test_lse_ragged(sage, B, S, H, smooth_k):
    import torch
    w = synth.custom(B, S, H, smooth_k=smooth_k, base_seed=2500 + S)
    q, k, v = inputs(w)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    bits, lse_o = oracle.attn(oracle.prepare(q, k, v, smooth_k), w.sm_scale, want_lse=True)
    assert lse.shape == (B, H, S)
    check_lse(f"lse{B}x{S}x{H}", lse.cpu().numpy(), lse_o)
    # asking for the log-sum-exp leaves the output as it is
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), bits) or \
        oracle.max_abs_rel(oracle.bf16_bits_to_f64(out.view(torch.int16).cpu().numpy().view(np.uint16)),
                           oracle.bf16_bits_to_f64(bits)) <= MAXABS_TOL


@pytest.mark.parametrize("name", ["C2", "C3"])
def test_lse_workload_rows(sage, name):
    import torch
    w = synth.WORKLOADS[name]
    q, k, v = inputs(w)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, True, w.smooth_k)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w, 1024)
    heads = sorted({(int(b), int(h)) for b, h, _ in rows})
    prep = oracle.prepare(q, k, v, w.smooth_k, heads=heads)
    _, lse_o = oracle.attn(prep, w.sm_scale, rows=rows, want_lse=True)
    g = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    check_lse(f"lse_{name}", g, lse_o)


# ------------------------------------------------------------------ head dim 64
@pytest.mark.parametrize("B,S,H,smooth_k", [(1, 1, 1, False), (2, 33, 3, True), (1, 300, 2, False),
                                             (2, 1000, 3, True), (3, 127, 1, True)])
def test_d64_prologue_attention_and_lse(sage, B, S, H, smooth_k):
    import torch
    w = synth.custom(B, S, H, D=64, smooth_k=smooth_k, base_seed=4000 + S)
    q, k, v = inputs(w)
    g = gpu_prepare(sage, q, k, v, smooth_k)
    o = oracle.prepare(q, k, v, smooth_k)
    check_prologue(g, o, S, smooth_k=smooth_k)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    R, lse_o = oracle.attn(o, w.sm_scale, want_lse=True)
    E = oracle.exact(q, k, v, w.sm_scale)
    compare_attention(f"d64_{B}x{S}x{H}", out.view(torch.int16).cpu().numpy().view(np.uint16), R, E)
    check_lse(f"d64_lse{B}x{S}x{H}", lse.cpu().numpy(), lse_o)


def test_d64_equals_d128_with_zero_channels(sage):
    """Appending 64 zero channels changes nothing the method computes on the first
    64 (see the oracle's pin of the same identity): the two GPU paths agree bit
    for bit, outputs and log-sum-exp."""
    import torch
    w = synth.custom(2, 700, 3, D=64, smooth_k=True, base_seed=4100)
    q, k, v = (to_dev(a) for a in inputs(w))
    pad = [torch.nn.functional.pad(x, (0, 64)) for x in (q, k, v)]
    o64, l64 = sage.sageattn(q, k, v, sm_scale=0.125, return_lse=True)
    o128, l128 = sage.sageattn(*pad, sm_scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o64.view(torch.int16), o128[..., :64].contiguous().view(torch.int16))
    assert not o128[..., 64:].any()
    assert torch.equal(l64.view(torch.int32), l128.view(torch.int32))


def test_d64_workload_rows(sage):
    import torch
    w = synth.WORKLOADS["C6"]
    q, k, v = inputs(w)
    g = gpu_prepare(sage, q, k, v, w.smooth_k)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", False, w.sm_scale, True, w.smooth_k)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w, 1024)
    heads = sorted({(int(b), int(h)) for b, h, _ in rows})
    prep = oracle.prepare(q, k, v, w.smooth_k, heads=heads)
    check_prologue(g, prep, w.S, heads=heads[:6])
    R, lse_o = oracle.attn(prep, w.sm_scale, rows=rows, want_lse=True)
    E = oracle.exact(q, k, v, w.sm_scale, rows=rows)
    O = out.view(torch.int16).cpu().numpy().view(np.uint16)
    compare_attention("C6", O[rows[:, 0], rows[:, 2], rows[:, 1]], R, E)
    check_lse("lse_C6", lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]], lse_o)


# ------------------------------------------------------------------ causal
@pytest.mark.parametrize("B,S,H,D,smooth_k", [(1, 1, 1, 128, False), (2, 33, 3, 128, True), (1, 128, 2, 128, False),
                                               (1, 257, 2, 128, True), (2, 300, 3, 128, False),
                                               (1, 700, 2, 128, True), (1, 1000, 2, 64, True),
                                               (3, 127, 1, 64, False)])
def test_causal_attention_and_lse(sage, B, S, H, D, smooth_k):
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=6000 + S + D)
    q, k, v = inputs(w)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", True, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    R, lse_o = oracle.attn(oracle.prepare(q, k, v, smooth_k), w.sm_scale, want_lse=True, causal=True)
    E = oracle.exact(q, k, v, w.sm_scale, causal=True)
    compare_attention(f"causal{B}x{S}x{H}x{D}", out.view(torch.int16).cpu().numpy().view(np.uint16), R, E)
    check_lse(f"causal_lse{B}x{S}x{H}x{D}", lse.cpu().numpy(), lse_o)


@pytest.mark.parametrize("qscale", [0.0, 2.0 ** -40, 2.0 ** 8])
@pytest.mark.parametrize("B,S,H,D,causal", [(1, 300, 2, 128, False), (2, 333, 2, 128, True),
                                             (1, 1000, 2, 64, True), (1, 200, 3, 64, False)])
def test_extreme_score_scales_keep_masked_keys_out(sage, qscale, B, S, H, D, causal):
    """Q scaled to 0 or by 2^-40 makes every score (nearly) 0, and then a masked
    key's score, however low its integer stand-in, times the block's scale is
    no longer far below the row maximum. Only the infinite scale of blocks that
    no lane sees, the correction of l for the partly masked block and (causal)
    the cleared FP8 codes keep padded and masked keys out of the row. Every
    visible key has (nearly) the same weight there, so one leaked key moves the
    output and the log-sum-exp visibly. Q scaled by 2^8 is the other end:
    scores of hundreds (log2 units), rows close to one-hot, the running maximum
    jumping by more than the exponent range so that alpha underflows to 0."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=True, base_seed=6200 + S + D + int(causal))
    q, k, v = inputs(w)
    qt = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16) * qscale   # exact: a power of two or zero
    q = qt.contiguous().view(torch.int16).numpy().view(np.uint16)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", causal, w.sm_scale, True, True)
    torch.cuda.synchronize()
    R, lse_o = oracle.attn(oracle.prepare(q, k, v, True), w.sm_scale, want_lse=True, causal=causal)
    E = oracle.exact(q, k, v, w.sm_scale, causal=causal)
    name = f"qscale{qscale:g}_{B}x{S}x{H}x{D}{'_causal' if causal else ''}"
    compare_attention(name, out.view(torch.int16).cpu().numpy().view(np.uint16), R, E,
                      limited="qscale256" if qscale == 2.0 ** 8 else None)
    check_lse("lse_" + name, lse.cpu().numpy(), lse_o)


@pytest.mark.parametrize("B,S,H,D,causal,smooth_k", [(1, 700, 3, 128, False, False), (2, 333, 3, 128, True, True),
                                                      (1, 1000, 3, 64, True, False), (1, 300, 3, 64, False, True)])
def test_large_scores_take_the_exact_softmax_form(sage, B, S, H, D, causal, smooth_k):
    """Scores of 2^19 and more (log2 units), where the kernel's one-FMA
    exponent would no longer round the score first as the method does (and
    could exceed the FP8 range): the waves that may meet scores of 2^14 run the
    method's exact form. Head 0: Q and K times 2^8 (every wave exact); head 1:
    the queries of one wave times 2^10 (that wave exact, the other three of its
    workgroup fast, so the two loop copies run side by side); head 2: one
    32-key block times 2^12 (every wave exact). Output and log-sum-exp against
    the oracle; the rows are near one-hot, so exact attention is not compared."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=6300 + S + D)
    q, k, v = (x.copy() for x in inputs(w))
    q[:, :, 0] = _scaled(q[:, :, 0], 2.0 ** 8)
    k[:, :, 0] = _scaled(k[:, :, 0], 2.0 ** 8)
    q[:, 32:64, 1] = _scaled(q[:, 32:64, 1], 2.0 ** 10)
    k[:, 128:160, 2] = _scaled(k[:, 128:160, 2], 2.0 ** 12)
    o = oracle.prepare(q, k, v, smooth_k)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", causal, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    O = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.all(np.isfinite(oracle.bf16_bits_to_f64(O)))
    R, lse_o = oracle.attn(o, w.sm_scale, want_lse=True, causal=causal)
    name = f"large_scores_{B}x{S}x{H}x{D}{'_causal' if causal else ''}"
    compare_attention(name, O, R, None)
    check_lse("lse_" + name, lse.cpu().numpy(), lse_o)


def test_causal_last_row_is_the_non_causal_row(sage):
    """The last query sees every key, and on the diagonal tile the cleared
    codes of the padded keys multiplied V codes that are zero anyway: the
    causal and non-causal kernels agree on that row bit for bit (output and
    log-sum-exp). Through sage_attn_ex on prepare()'s output, the causal step
    is also the fused call's causal result."""
    import torch
    w = synth.custom(2, 1000, 3, smooth_k=True, base_seed=6100)
    q, k, v = (to_dev(a) for a in inputs(w))
    prep = sage.prepare(q, k, v, True)
    oc, lc = sage.attn(prep, w.sm_scale, return_lse=True, is_causal=True)
    on, ln = sage.attn(prep, w.sm_scale, return_lse=True)
    of = sage.sageattn(q, k, v, is_causal=True, sm_scale=w.sm_scale)
    oc2 = sage.attn(prep, w.sm_scale, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(oc[:, -1].view(torch.int16), on[:, -1].view(torch.int16))
    assert torch.equal(lc[:, :, -1].view(torch.int32), ln[:, :, -1].view(torch.int32))
    assert not torch.equal(oc[:, :-1].view(torch.int16), on[:, :-1].view(torch.int16))
    assert torch.equal(of.view(torch.int16), oc.view(torch.int16))
    assert torch.equal(oc2.view(torch.int16), oc.view(torch.int16))


@pytest.mark.parametrize("name,n", [("C2", 2048), ("C3", 768)])
def test_causal_workload_rows(sage, name, n):
    import torch
    w = synth.WORKLOADS[name]
    q, k, v = inputs(w)
    out, lse = sage.sageattn(to_dev(q), to_dev(k), to_dev(v), "NHD", True, w.sm_scale, True, w.smooth_k)
    torch.cuda.synchronize()
    rows = synth.sample_rows(w, n)
    # plus the rows on either side of two key-tile boundaries and the first and last row of head 0
    extra = np.array([[0, 0, s] for s in (0, 1, 127, 128, 129, 255, 256, w.S - 1)], dtype=np.int64)
    rows = np.unique(np.concatenate([rows, extra]), axis=0)
    heads = sorted({(int(b), int(h)) for b, h, _ in rows})
    prep = oracle.prepare(q, k, v, w.smooth_k, heads=heads)
    R, lse_o = oracle.attn(prep, w.sm_scale, rows=rows, want_lse=True, causal=True)
    E = oracle.exact(q, k, v, w.sm_scale, rows=rows, causal=True)
    O = out.view(torch.int16).cpu().numpy().view(np.uint16)
    compare_attention(f"causal_{name}", O[rows[:, 0], rows[:, 2], rows[:, 1]], R, E,
                      limited="causal_C3" if name == "C3" else None)
    check_lse(f"causal_lse_{name}", lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]], lse_o)


# ------------------------------------------------------------------ randomized sweep
def _random_cases(n=None, seed=None):
    # 24 cases from a fixed seed by default; SAGE_RANDOM_CASES and SAGE_RANDOM_SEED
    # run a longer or different sweep
    n = int(os.environ.get("SAGE_RANDOM_CASES", "24")) if n is None else n
    seed = int(os.environ.get("SAGE_RANDOM_SEED", "20261202")) if seed is None else seed
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        S = int(rng.choice([int(rng.integers(1, 40)), int(rng.integers(40, 300)), int(rng.integers(300, 700))]))
        cases.append((i, int(rng.integers(1, 4)), S, int(rng.integers(1, 5)), int(rng.choice([64, 128])),
                      bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), str(rng.choice(["NHD", "HND"]))))
    return cases


@pytest.mark.parametrize("i,B,S,H,D,smooth_k,causal,layout", _random_cases())
def test_random_configurations_against_the_oracle(sage, i, B, S, H, D, smooth_k, causal, layout):
    """Seeded random shapes (B <= 3, S < 700, H <= 4), head dims, smooth_k,
    causal and layouts: prologue bit for bit, output and log-sum-exp within
    tolerance, against the oracle on every row."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=7100 + i)
    q, k, v = inputs(w)
    o = oracle.prepare(q, k, v, smooth_k)
    check_prologue(gpu_prepare(sage, q, k, v, smooth_k), o, S, smooth_k=smooth_k)
    tq, tk, tv = (to_dev(x) for x in (q, k, v))
    if layout == "HND":
        tq, tk, tv = (x.permute(0, 2, 1, 3).contiguous() for x in (tq, tk, tv))
    out, lse = sage.sageattn(tq, tk, tv, layout, causal, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    if layout == "HND":
        out = out.permute(0, 2, 1, 3).contiguous()
    R, lse_o = oracle.attn(o, w.sm_scale, want_lse=True, causal=causal)
    E = oracle.exact(q, k, v, w.sm_scale, causal=causal)
    compare_attention(f"random{i}_{B}x{S}x{H}x{D}_{'sk' if smooth_k else 'nosk'}_{'c' if causal else 'nc'}_{layout}",
                      out.view(torch.int16).cpu().numpy().view(np.uint16), R, E)
    check_lse(f"random{i}_lse", lse.cpu().numpy(), lse_o)


def _larger_cases(n=6, seed=4242):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B, H, S = int(rng.integers(1, 3)), int(rng.integers(1, 7)), int(rng.integers(2000, 20000))
        cases.append((i, B, S, H, int(rng.choice([64, 128])), bool(rng.integers(0, 2)), bool(rng.integers(0, 2)),
                      str(rng.choice(["NHD", "HND"]))))
    return cases


@pytest.mark.parametrize("i,B,S,H,D,smooth_k,causal,layout", _larger_cases())
def test_random_larger_configurations_on_sampled_rows(sage, i, B, S, H, D, smooth_k, causal, layout):
    """Seeded random shapes with S between 2 000 and 20 000 (many key tiles, a
    ragged last one): output and log-sum-exp on about 200 sampled rows plus the
    rows at the first and last tile edges of the last head, the last head's
    prologue bit for bit."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=9000 + i)
    q, k, v = inputs(w)
    tq, tk, tv = (to_dev(x) for x in (q, k, v))
    if layout == "HND":
        tq, tk, tv = (x.permute(0, 2, 1, 3).contiguous() for x in (tq, tk, tv))
    out, lse = sage.sageattn(tq, tk, tv, layout, causal, w.sm_scale, True, smooth_k)
    torch.cuda.synchronize()
    if layout == "HND":
        out = out.permute(0, 2, 1, 3).contiguous()
    edge = np.array([[B - 1, H - 1, s] for s in (0, 127, 128, S - 129, S - 128, S - 1)], dtype=np.int64)
    rows = np.unique(np.concatenate([synth.sample_rows(w, 192), edge]), axis=0)
    heads = sorted({(int(b), int(h)) for b, h, _ in rows})
    prep = oracle.prepare(q, k, v, smooth_k, heads=heads)
    R, lse_o = oracle.attn(prep, w.sm_scale, rows=rows, want_lse=True, causal=causal)
    E = oracle.exact(q, k, v, w.sm_scale, rows=rows, causal=causal)
    O = out.view(torch.int16).cpu().numpy().view(np.uint16)
    name = f"larger{i}_{B}x{S}x{H}x{D}_{'sk' if smooth_k else 'nosk'}_{'c' if causal else 'nc'}_{layout}"
    compare_attention(name, O[rows[:, 0], rows[:, 2], rows[:, 1]], R, E)
    check_lse(name + "_lse", lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]], lse_o)
    g = gpu_prepare(sage, q, k, v, smooth_k)
    b, h = B - 1, H - 1
    o = oracle.prepare_head(q[b, :, h].copy(), k[b, :, h].copy(), v[b, :, h].copy(), smooth_k)
    check_prologue({key: val[b:b + 1, h:h + 1] for key, val in g.items()}, {key: val[None, None] for key, val in o.items()},
                   S)


# ------------------------------------------------------------------ 64-bit offsets, graph capture
def test_tensors_past_2_31_elements(sage):
    """B*S*H*D = 3*65536*96*128 > 2^31 elements (4.8 GB per BF16 tensor): the
    prologue's codes of the first, a middle and the last head are bit-exact and
    the last head's attention rows (element offsets past 2^31) match the oracle.
    Inputs are seeded normal draws made on the device."""
    import torch
    B, S, H, D = 3, 65536, 96, 128
    assert B * S * H * D > 2 ** 31
    gen = torch.Generator(device="cuda").manual_seed(7000)
    q = torch.randn((B, S, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((B, S, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    k.add_(0.5)
    v = torch.randn((B, S, H, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    sm = 1.0 / math.sqrt(D)
    prep = sage.prepare(q, k, v, True)
    out = sage.attn(prep, sm)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 127, 128, 40000, S - 129, S - 2, S - 1], dtype=np.int64)
    for b, h in ((0, 0), (1, 47), (B - 1, H - 1)):
        host = [x[b, :, h, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for x in (q, k, v)]
        o = oracle.prepare_head(*host, True)
        g = {key: prep[key][b, h].cpu().numpy() for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale",
                                                            "k_mean")}
        check_prologue({key: val[None, None] for key, val in g.items()},
                       {key: val[None, None] for key, val in o.items()}, S)
        if (b, h) == (B - 1, H - 1):
            R = oracle.attn_rows_head(o, rows, sm)
            E = oracle.exact_rows_head(*host, rows, sm)
            G = out[b, :, h, :].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[rows]
            compare_attention("past_2^31_last_head", G, R, E)
    del q, k, v, prep, out
    torch.cuda.empty_cache()


def test_tensors_past_2_31_elements_hnd(sage):
    """The same size in the HND layout ([B, H, S, D] inputs, output written
    through an HND view): here the head stride S*D carries the offsets past
    2^31 (the last head starts at element 2.4e9), in the prologue's loads and
    in the attention epilogue's stores."""
    import torch
    B, S, H, D = 3, 65536, 96, 128
    gen = torch.Generator(device="cuda").manual_seed(7100)
    q = torch.randn((B, H, S, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    k = torch.randn((B, H, S, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    k.add_(0.5)
    v = torch.randn((B, H, S, D), generator=gen, device="cuda", dtype=torch.bfloat16)
    assert q[B - 1, H - 1].storage_offset() > 2 ** 31
    sm = 1.0 / math.sqrt(D)
    prep = sage.prepare(q, k, v, True, layout="HND")
    out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    sage.attn(prep, sm, out=out.permute(0, 2, 1, 3))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 31, 32, 127, 128, 40000, S - 129, S - 2, S - 1], dtype=np.int64)
    for b, h in ((0, 0), (1, 47), (B - 1, H - 1)):
        host = [x[b, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for x in (q, k, v)]
        o = oracle.prepare_head(*host, True)
        g = {key: prep[key][b, h].cpu().numpy() for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale",
                                                            "k_mean")}
        check_prologue({key: val[None, None] for key, val in g.items()},
                       {key: val[None, None] for key, val in o.items()}, S)
        if (b, h) == (B - 1, H - 1):
            R = oracle.attn_rows_head(o, rows, sm)
            E = oracle.exact_rows_head(*host, rows, sm)
            G = out[b, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)[rows]
            compare_attention("past_2^31_last_head_hnd", G, R, E)
    del q, k, v, prep, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("S", [700, 300])
def test_fused_calls_replay_from_a_hip_graph(sage, S):
    """sageattn, causal and not, captured in one HIP graph (the library launches
    kernels only: no allocation, memset or synchronisation inside) and replayed
    three times with eager work in between: every replay equals the eager result
    bit for bit. 700 tokens take the separate launches, 300 the one-launch form."""
    import torch
    w = synth.custom(2, S, 3, smooth_k=True, base_seed=6200 + S)
    q, k, v = (to_dev(a) for a in inputs(w))
    ref = [sage.sageattn(q, k, v, is_causal=c, sm_scale=w.sm_scale, return_lse=True) for c in (False, True)]
    torch.cuda.synchronize()
    nws = sage.fused_workspace_bytes(2, S, 3, 128)
    ws = [torch.empty(nws, dtype=torch.uint8, device="cuda") for _ in range(2)]
    outs = [torch.empty_like(q) for _ in range(2)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm up on the capture stream
        for c in (False, True):
            sage.sageattn(q, k, v, is_causal=c, sm_scale=w.sm_scale, out=outs[c], workspace=ws[c])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        lses = [sage.sageattn(q, k, v, is_causal=c, sm_scale=w.sm_scale, return_lse=True, out=outs[c],
                              workspace=ws[c])[1] for c in (False, True)]
    torch.cuda.synchronize()
    for _ in range(3):
        for t in outs + lses:
            t.zero_()
        ws[0].fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for c in (0, 1):
            assert torch.equal(outs[c].view(torch.int16), ref[c][0].view(torch.int16)), c
            assert torch.equal(lses[c].view(torch.int32), ref[c][1].view(torch.int32)), c


def test_fused_equals_prepare_then_attn_and_is_deterministic(sage):
    import torch
    w = synth.custom(2, 700, 3, smooth_k=True, base_seed=3000)
    q, k, v = (to_dev(a) for a in inputs(w))
    f1 = sage.sageattn(q, k, v, smooth_k=True)
    f2 = sage.sageattn(q, k, v, smooth_k=True)
    p = sage.prepare(q, k, v, True)
    t = sage.attn(p, w.sm_scale)
    f3, l3 = sage.sageattn(q, k, v, smooth_k=True, return_lse=True)
    t2, l2 = sage.attn(p, w.sm_scale, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(f1.view(torch.int16), f2.view(torch.int16))
    assert torch.equal(f1.view(torch.int16), t.view(torch.int16))
    assert torch.equal(f1.view(torch.int16), f3.view(torch.int16))
    assert torch.equal(f1.view(torch.int16), t2.view(torch.int16))
    assert torch.equal(l3.view(torch.int32), l2.view(torch.int32))


@pytest.mark.parametrize("B,S,H,D,causal,smooth_k", [(2, 384, 3, 128, False, True), (1, 300, 2, 128, True, False),
                                                      (3, 129, 2, 128, False, False), (1, 1, 1, 128, False, True),
                                                      (2, 700, 2, 64, True, True), (1, 257, 3, 64, False, False),
                                                      (2, 768, 1, 64, False, True), (2, 385, 2, 128, False, True),
                                                      (1, 769, 2, 64, True, False), (6, 128, 50, 128, True, True)])
def test_fused_short_heads_equal_prepare_then_attn(sage, B, S, H, D, causal, smooth_k):
    """Heads of up to three key tiles (six at head dim 64) run the whole fused
    call in one workgroup per head with the codes kept in LDS: outputs and
    log-sum-exp bit for bit those of prepare then attn (longer heads, here
    2x385x2 and 1x769x2 at head dim 64, take the separate launches)."""
    import torch
    w = synth.custom(B, S, H, D=D, smooth_k=smooth_k, base_seed=3100 + S + D)
    q, k, v = (to_dev(a) for a in inputs(w))
    f, lf = sage.sageattn(q, k, v, is_causal=causal, smooth_k=smooth_k, return_lse=True)
    p = sage.prepare(q, k, v, smooth_k)
    t, lt = sage.attn(p, w.sm_scale, is_causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(f.view(torch.int16), t.view(torch.int16))
    assert torch.equal(lf.view(torch.int32), lt.view(torch.int32))


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_fused_short_heads_hnd_equal_prepare_then_attn(sage, D, causal):
    """The one-launch form on HND inputs ([B, H, S, D]) into an HND output: the
    same bits as prepare then attn on the same layout."""
    import torch
    w = synth.custom(2, 333, 3, D=D, smooth_k=True, base_seed=3400 + D)
    q, k, v = (to_dev(a).permute(0, 2, 1, 3).contiguous() for a in inputs(w))
    f, lf = sage.sageattn(q, k, v, tensor_layout="HND", is_causal=causal, return_lse=True)
    p = sage.prepare(q, k, v, True, layout="HND")
    t, lt = sage.attn(p, w.sm_scale, is_causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(f.permute(0, 2, 1, 3).contiguous().view(torch.int16), t.view(torch.int16))
    assert torch.equal(lf.view(torch.int32), lt.view(torch.int32))


def test_prepare_reuse_rewrites_the_same_buffers(sage):
    """prepare(reuse=...) writes a previous result's tensors again: same
    storage, same bits as a fresh call, on other inputs of the same shape;
    another shape is refused before any launch."""
    import torch
    w1 = synth.custom(2, 300, 3, smooth_k=True, base_seed=6300)
    w2 = synth.custom(2, 300, 3, smooth_k=True, base_seed=6301)
    a = [to_dev(x) for x in inputs(w1)]
    b = [to_dev(x) for x in inputs(w2)]
    p = sage.prepare(*a, True)
    ptrs = {key: val.data_ptr() for key, val in p.items() if torch.is_tensor(val)}
    p2 = sage.prepare(*b, True, reuse=p)
    fresh = sage.prepare(*b, True)
    torch.cuda.synchronize()
    assert p2 is p and all(p[key].data_ptr() == ptr for key, ptr in ptrs.items())
    for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale", "k_mean"):
        assert torch.equal(p2[key], fresh[key]), key
    c = [to_dev(x) for x in inputs(synth.custom(2, 400, 3, smooth_k=True, base_seed=6302))]
    with pytest.raises(ValueError):
        sage.prepare(*c, True, reuse=p)


def test_calls_on_two_streams_at_once_match_serial_results(sage):
    """The library keeps no state between calls: fused calls with their own
    workspaces, issued alternately on two streams so that they overlap, give
    the results of the same calls made one after another."""
    import torch
    ws_ = [synth.custom(1, 1000 + 37 * i, 4, smooth_k=bool(i % 2), base_seed=6400 + i) for i in range(4)]
    data = [[to_dev(x) for x in inputs(w)] for w in ws_]
    ref = [sage.sageattn(*d, is_causal=bool(i % 2), sm_scale=0.1, smooth_k=bool(i % 2)) for i, d in enumerate(data)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(d[0]) for d in data]
    wss = [torch.empty(sage.fused_workspace_bytes(w.B, w.S, w.H, w.D), dtype=torch.uint8, device="cuda") for w in ws_]
    for s_ in streams:
        s_.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for i, d in enumerate(data):
            sage.sageattn(*d, is_causal=bool(i % 2), sm_scale=0.1, smooth_k=bool(i % 2), out=outs[i],
                          workspace=wss[i], stream=streams[i % 2])
        torch.cuda.synchronize()
        for i in range(4):
            assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16)), (rep, i)


def test_call_on_another_stream_keeps_its_workspace_from_the_current_stream(sage):
    """A fused call on a side stream without a workspace: the temporary the
    binding allocates must not be handed to the current stream's allocations
    while the side stream still works on it. The current stream fills fresh
    buffers of the workspace's size right after the call; the result is that
    of a call on the current stream."""
    import torch
    w = synth.custom(2, 3000, 6, smooth_k=True, base_seed=6450)
    q, k, v = (to_dev(x) for x in inputs(w))
    ref = sage.sageattn(q, k, v, sm_scale=0.1)
    torch.cuda.synchronize()
    nws = sage.fused_workspace_bytes(w.B, w.S, w.H, w.D)
    side = torch.cuda.Stream()
    for rep in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            out = torch.empty_like(q)
        out2 = sage.sageattn(q, k, v, sm_scale=0.1, out=out, stream=side)
        junk = [torch.full((nws,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(3)]
        torch.cuda.synchronize()
        assert out2 is out
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        del junk


def test_outputs_leave_guard_bands_untouched(sage):
    """Every output buffer sits inside a larger allocation filled with a
    canary byte: after prepare, attn (with the log-sum-exp) and the fused call,
    causal and not, on ragged shapes at both head dims, the canary bytes on
    either side are unchanged (and the outputs are those of ordinary calls)."""
    import ctypes
    import torch
    G = 4096   # guard bytes on each side
    for (B, S, H, D) in ((2, 300, 3, 128), (1, 129, 2, 64), (3, 33, 1, 128)):
        w = synth.custom(B, S, H, D=D, smooth_k=True, base_seed=6500 + S)
        q, k, v = (to_dev(x) for x in inputs(w))
        Sp = sage.padded_len(S)
        L = sage.lib()
        shapes = dict(q8=(B * H * Sp * D, 1), q_scale=(B * H * Sp // 32, 4), k8=(B * H * Sp * D, 1),
                      k_scale=(B * H * Sp // 32, 4), v8t=(B * H * D * Sp, 1), v_scale=(B * H * D, 4),
                      k_mean=(B * H * D, 4), out=(B * S * H * D, 2), lse=(B * H * S, 4))
        bufs = {}
        for name, (n, item) in shapes.items():
            raw = torch.full((n * item + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
            bufs[name] = raw
        def inner(name):
            n, item = shapes[name]
            return bufs[name][G:G + n * item]
        nws = L.sage_prepare_workspace_bytes(B, S, H, D, 1)
        wsraw = torch.full((nws + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
        tq, tk, tv = sage.describe(q), sage.describe(k), sage.describe(v)
        P = sage._ptr
        sage.check(L.sage_prepare(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), 1, P(inner("q8")),
                                  P(inner("q_scale")), P(inner("k8")), P(inner("k_scale")), P(inner("v8t")),
                                  P(inner("v_scale")), P(inner("k_mean")), P(wsraw[G:G + nws]), nws, sage._stream(None)))
        out = inner("out").view(torch.bfloat16).view(B, S, H, D)
        to = sage.describe(out)
        for causal in (0, 1):
            sage.check(L.sage_attn_ex(P(inner("q8")), P(inner("q_scale")), P(inner("k8")), P(inner("k_scale")),
                                      P(inner("v8t")), P(inner("v_scale")), B, S, H, D, 0.1, causal, ctypes.byref(to),
                                      P(inner("lse")), sage._stream(None)))
            torch.cuda.synchronize()
            ref = sage.sageattn(q, k, v, is_causal=bool(causal), sm_scale=0.1, return_lse=True)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16))
            assert torch.equal(inner("lse").view(torch.float32).view(B, H, S), ref[1])
        # the fused call into a guarded output, with a guarded workspace
        nf = sage.fused_workspace_bytes(B, S, H, D)
        fws = torch.full((nf + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
        oraw = torch.full((B * S * H * D * 2 + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
        fo = oraw[G:G + B * S * H * D * 2].view(torch.bfloat16).view(B, S, H, D)
        sage.sageattn(q, k, v, sm_scale=0.1, out=fo, workspace=fws[G:G + nf])
        torch.cuda.synchronize()
        for name, raw in list(bufs.items()) + [("ws", wsraw), ("fused_ws", fws), ("fused_out", oraw)]:
            head, tail = raw[:G], raw[-G:]
            assert bool((head == 0xA5).all()) and bool((tail == 0xA5).all()), (B, S, H, D, name)


def test_v_times_a_power_of_two_scales_the_output_exactly(sage):
    """V * 2^k scales each channel's amax, hence v_scale, by 2^k and leaves the
    FP8 codes as they are, so the output is multiplied by 2^k bit for bit."""
    import torch
    w = synth.custom(2, 500, 3, smooth_k=True, base_seed=6600)
    q, k, v = (to_dev(x) for x in inputs(w))
    for causal in (False, True):
        o1 = sage.sageattn(q, k, v, is_causal=causal, sm_scale=w.sm_scale)
        for e in (-3, 2, 5):
            o2 = sage.sageattn(q, k, v * (2.0 ** e), is_causal=causal, sm_scale=w.sm_scale)
            torch.cuda.synchronize()
            assert torch.equal((o1.float() * 2.0 ** e).to(torch.bfloat16).view(torch.int16), o2.view(torch.int16)), e


def test_hnd_layout_and_strided_output_match_nhd(sage):
    import torch
    w = synth.custom(2, 200, 3, smooth_k=True, base_seed=3100)
    q, k, v = (to_dev(a) for a in inputs(w))
    ref = sage.sageattn(q, k, v)
    qh, kh, vh = (x.permute(0, 2, 1, 3).contiguous() for x in (q, k, v))
    hnd = sage.sageattn(qh, kh, vh, tensor_layout="HND")
    big = torch.zeros((2, 200, 3, 256), dtype=torch.bfloat16, device=q.device)
    out = big[..., 64:192]
    sage.sageattn(q, k, v, out=out)
    torch.cuda.synchronize()
    assert torch.equal(hnd.permute(0, 2, 1, 3).contiguous().view(torch.int16), ref.view(torch.int16))
    assert torch.equal(out.contiguous().view(torch.int16), ref.view(torch.int16))
    assert not big[..., :64].any() and not big[..., 192:].any()


def test_empty_problem_is_a_no_op(sage):
    import torch
    q = torch.zeros((2, 0, 3, 128), dtype=torch.bfloat16, device="cuda")
    out = sage.sageattn(q, q, q)
    torch.cuda.synchronize()
    assert out.shape == q.shape


def test_unsupported_inputs_raise(sage):
    import torch
    q = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        sage.sageattn(q.half(), q.half(), q.half())
    q96 = torch.zeros((1, 64, 2, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        sage.sageattn(q96, q96, q96)
    k = torch.zeros((1, 65, 2, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(NotImplementedError):
        sage.sageattn(q, k, k)
    with pytest.raises(ValueError):
        sage.sageattn(q, q, q, sm_scale=-1.0)
