"""The C ABI on the CPU: the library loads without a GPU, exports every
function include/sage.h declares, and validates arguments on the host in the
documented order before any device call. No compute call is made here; the
pointers passed are host addresses that the library never dereferences."""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_attention_prepare_amd as sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WS_SMALL, DEVICE = range(5)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "sage.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = sage.lib()
    names = declared_functions()
    assert {"sage_prepare", "sage_attn", "sage_attn_fused", "sage_kv_tile"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_constants_and_sizes():
    assert sage.kv_tile() == 128
    assert [sage.padded_len(s) for s in (0, 1, 128, 129, 300)] == [0, 128, 128, 256, 384]
    assert sage.padded_len(2 ** 63 - 1) == -1 and sage.padded_len(2 ** 63 - 128) == 2 ** 63 - 128
    assert sage.padded_len(-5) == 0
    L = sage.lib()
    assert L.sage_fused_workspace_bytes(0, 10, 2, 128) == 0
    small = L.sage_fused_workspace_bytes(1, 256, 2, 128)
    big = L.sage_fused_workspace_bytes(1, 32768, 28, 128)
    assert 0 < small < big
    # the quantized tensors alone: 3 * B*H*S_pad*128 bytes
    assert big >= 3 * 28 * 32768 * 128
    assert L.sage_prepare_workspace_bytes(1, 4096, 28, 128, 1) > 0
    # head dim 64: half the quantized bytes; other head dims are not supported (0 bytes)
    assert 0 < L.sage_fused_workspace_bytes(1, 32768, 28, 64) < big
    assert L.sage_fused_workspace_bytes(1, 32768, 28, 64) >= 3 * 28 * 32768 * 64
    assert L.sage_fused_workspace_bytes(1, 256, 2, 96) == 0
    for s in range(5):
        assert L.sage_status_string(s).decode().startswith("SAGE_")


class Host:
    """16-byte aligned host buffers that stand in for device pointers."""

    def __init__(self):
        self.keep = []

    def buf(self, nbytes=4096, misalign=0):
        a = np.zeros(nbytes + 64, np.uint8)
        self.keep.append(a)
        base = (a.ctypes.data + 15) & ~15
        return ctypes.c_void_p(base + misalign)

    def tensor(self, size=(1, 64, 2, 128), dtype=1, stride=None, misalign=0):
        if stride is None:
            B, S, H, D = size
            stride = (S * H * D, H * D, D, 1)
        return sage.SageTensor(self.buf(misalign=misalign).value, dtype, (ctypes.c_int64 * 4)(*size),
                               (ctypes.c_int64 * 4)(*stride))


def fused(h, q=None, k=None, v=None, o=None, causal=0, sm=0.088, lse_flag=0, lse=None, ws=None, ws_bytes=None):
    q = q or h.tensor()
    k = k or h.tensor()
    v = v or h.tensor()
    o = o or h.tensor()
    B, S, H, D = q.size
    need = sage.lib().sage_fused_workspace_bytes(B, S, H, D)
    ws = h.buf() if ws is None else ws
    ws_bytes = need if ws_bytes is None else ws_bytes
    return sage.lib().sage_attn_fused(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(o), causal, sm,
                                      lse_flag, lse, 1, ws, ws_bytes, None)


def last_error():
    return sage.lib().sage_last_error().decode()


def test_fused_validation_order_on_host():
    h = Host()
    # 1. invalid arguments
    assert sage.lib().sage_attn_fused(None, None, None, None, 0, 0.1, 0, None, 1, None, 0, None) == INVALID
    assert fused(h, sm=float("nan")) == INVALID
    assert fused(h, sm=0.0) == INVALID
    assert fused(h, sm=-1.0) == INVALID
    bad = h.tensor()
    bad.size[1] = -1
    assert fused(h, q=bad) == INVALID
    assert fused(h, ws=ctypes.c_void_p(0)) == INVALID
    # log-sum-exp: the flag and the pointer must agree
    assert fused(h, lse_flag=1) == INVALID and "lse" in last_error()
    assert fused(h, lse=ctypes.c_void_p(h.buf().value)) == INVALID and "lse" in last_error()
    # invalid beats unsupported
    assert fused(h, causal=1, sm=float("inf")) == INVALID
    # 2. unsupported contract
    assert fused(h, lse_flag=1, lse=ctypes.c_void_p(h.buf().value + 2)) == UNSUPPORTED and "lse" in last_error()
    assert fused(h, q=h.tensor(dtype=2), k=h.tensor(dtype=2), v=h.tensor(dtype=2), o=h.tensor(dtype=2)) == UNSUPPORTED
    d96 = (1, 64, 2, 96)
    assert fused(h, q=h.tensor(d96), k=h.tensor(d96), v=h.tensor(d96), o=h.tensor(d96)) == UNSUPPORTED
    assert "64 or 128" in last_error()
    assert fused(h, k=h.tensor((1, 65, 2, 128))) == UNSUPPORTED and "shape" in last_error()
    assert fused(h, v=h.tensor(stride=(64 * 256, 256, 128, 2))) == UNSUPPORTED
    assert fused(h, o=h.tensor(stride=(64 * 256, 260, 128, 1))) == UNSUPPORTED
    assert fused(h, q=h.tensor(misalign=2)) == UNSUPPORTED and "aligned" in last_error()
    # 3. workspace
    assert fused(h, ws_bytes=10) == WS_SMALL
    # unsupported beats a small workspace
    assert fused(h, q=h.tensor(dtype=2), k=h.tensor(dtype=2), v=h.tensor(dtype=2), o=h.tensor(dtype=2),
                 ws_bytes=10) == UNSUPPORTED
    # 4. with everything valid, the device check is last: no GPU here
    rc = fused(h)
    assert rc == UNSUPPORTED and ("device" in last_error().lower())
    d64 = (1, 64, 2, 64)   # the other head dim: valid up to the device check
    assert fused(h, q=h.tensor(d64), k=h.tensor(d64), v=h.tensor(d64), o=h.tensor(d64)) == UNSUPPORTED
    assert "device" in last_error().lower()
    assert fused(h, lse_flag=1, lse=ctypes.c_void_p(h.buf().value)) == UNSUPPORTED and "device" in last_error().lower()
    # causal (an extension) is valid up to the device check as well
    assert fused(h, causal=1) == UNSUPPORTED and "device" in last_error().lower()
    assert fused(h, causal=1, ws_bytes=10) == WS_SMALL


def test_oversized_problems_are_refused_on_the_host():
    """Sizes whose products overflow, problems with more workgroups than a
    32-bit grid, and strides reaching past 2^60 elements are refused before any
    device call (the workspace figure of such a problem is 0)."""
    h = Host()
    L = sage.lib()
    huge = (1 << 40, 1 << 25, 1 << 40, 128)          # element count overflows int64
    big = (1 << 20, 1 << 24, 1 << 10, 128)           # B*H*S/128 = 2^47 workgroups
    t = h.tensor(big, stride=(8, 8, 8, 1))
    for size, want in ((huge, INVALID), (big, UNSUPPORTED)):
        q = h.tensor(size, stride=(8, 8, 8, 1))
        assert fused(h, q=q, k=q, v=q, o=q, ws_bytes=1 << 62) == want, size
        assert L.sage_fused_workspace_bytes(*size) == 0
        assert L.sage_prepare_workspace_bytes(*size, 1) == 0
    assert "too large" in (fused(h, q=t, k=t, v=t, o=t, ws_bytes=1 << 62) and last_error())
    # sage_attn with the same sizes: o describes them, the extent check refuses
    ptrs = [h.buf() for _ in range(6)]
    o = h.tensor(big, stride=(8, 8, 8, 1))
    assert L.sage_attn(*ptrs, *big[:3], 128, 0.1, ctypes.byref(o), None) == UNSUPPORTED
    assert "too large" in last_error()
    # the largest accepted grid is fine up to the device check
    smax = (1 << 25) - 128                           # longest sequence: S_pad * 128 bytes < 4 GiB
    edge = (1, smax, (1 << 13) + 1, 128)             # (2^13 + 1) heads x (2^18 - 1) tiles > 2^31 - 1 workgroups
    ok_edge = (1, smax, 1 << 13, 128)                # 2^31 - 2^13 workgroups
    assert L.sage_fused_workspace_bytes(*edge) == 0 and L.sage_fused_workspace_bytes(*ok_edge) > 0
    # S = 2^25 would give a 2^32-byte head, past the kernel's 32-bit buffer extent
    for D in (64, 128):
        assert L.sage_fused_workspace_bytes(1, smax, 1, D) > 0 and L.sage_fused_workspace_bytes(1, smax + 1, 1, D) == 0
        o_max = h.tensor((1, smax + 1, 1, D), stride=(8, 8, 8, 1))
        assert L.sage_attn(*ptrs, 1, smax + 1, 1, D, 0.1, ctypes.byref(o_max), None) == UNSUPPORTED
        o_ok = h.tensor((1, smax, 1, D), stride=(8, 8, 8, 1))
        assert L.sage_attn(*ptrs, 1, smax, 1, D, 0.1, ctypes.byref(o_ok), None) == UNSUPPORTED
        assert "device" in last_error().lower()
    # strides that reach past 2^60 elements
    far = h.tensor((4, 64, 2, 128), stride=(1 << 59, 256, 128, 1))
    assert fused(h, q=far) == UNSUPPORTED and "2^60" in last_error()


def test_random_descriptors_never_reach_the_device():
    """Random descriptors (sizes, strides, dtypes, alignments, flags) on host
    buffers: every call returns a documented status and none reaches a launch
    (there is no GPU here, so success is only possible for an empty problem)."""
    import random
    rng = random.Random(20261202)
    h = Host()
    statuses = set()
    for _ in range(3000):
        size = [rng.choice([0, 1, 2, 3, 31, 64, 96, 128, 129, 1 << 20, (1 << 25) - 128, (1 << 25) - 127, 1 << 25,
                            1 << 40, -1])
                for _ in range(4)]
        if rng.random() < 0.6:
            size[3] = rng.choice([64, 128])
        stride = [rng.choice([0, 1, 8, 16, 128, 256, 1 << 20, 1 << 59, 7, -8]) for _ in range(3)] + \
                 [rng.choice([1, 1, 1, 2])]
        q = sage.SageTensor(h.buf(misalign=rng.choice([0, 0, 0, 2])).value, rng.choice([1, 1, 1, 2]),
                            (ctypes.c_int64 * 4)(*size), (ctypes.c_int64 * 4)(*stride))
        other = q if rng.random() < 0.7 else h.tensor()
        rc = fused(h, q=q, k=other, v=q, o=q, causal=rng.choice([0, 1]), sm=rng.choice([0.1, 0.0, float("nan")]),
                   lse_flag=0, ws_bytes=rng.choice([0, 1 << 20, 1 << 62]))
        statuses.add(rc)
        assert rc in (OK, INVALID, UNSUPPORTED, WS_SMALL), rc
        if rc == OK:
            assert 0 in size[:3]
        if rc == UNSUPPORTED and "device" in last_error().lower():
            # everything up to the device check passed: the problem is within the limits
            B, S, H, D = size
            assert 0 < S <= (1 << 25) - 128 and D in (64, 128) and B * H * (-(-S // 128)) < (1 << 31) - 1
    assert {INVALID, UNSUPPORTED} <= statuses


def test_empty_problem_returns_ok_without_device():
    h = Host()
    z = (2, 0, 3, 128)
    assert fused(h, q=h.tensor(z), k=h.tensor(z), v=h.tensor(z), o=h.tensor(z), ws=ctypes.c_void_p(0), ws_bytes=0) == OK


def test_prepare_and_attn_validation_on_host():
    h = Host()
    L = sage.lib()
    q, k, v = h.tensor(), h.tensor(), h.tensor()
    outs = [h.buf() for _ in range(7)]
    need = L.sage_prepare_workspace_bytes(1, 64, 2, 128, 1)

    def prep(q=q, k=k, v=v, outs=outs, ws=None, ws_bytes=need):
        return L.sage_prepare(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1, *outs, ws or h.buf(), ws_bytes, None)

    assert prep(outs=[ctypes.c_void_p(0)] + outs[1:]) == INVALID
    assert prep(k=h.tensor(dtype=3)) == UNSUPPORTED
    assert prep(ws_bytes=need - 1) == WS_SMALL
    assert prep() == UNSUPPORTED and "device" in last_error().lower()

    o = h.tensor()
    ptrs = [h.buf() for _ in range(6)]

    def at(B=1, S=64, H=2, D=128, sm=0.1, o=o, ptrs=ptrs):
        return L.sage_attn(*ptrs, B, S, H, D, sm, ctypes.byref(o), None)

    assert at(S=-1) == INVALID
    assert at(ptrs=[ctypes.c_void_p(0)] + ptrs[1:]) == INVALID
    assert at(sm=float("nan")) == INVALID
    assert at(D=96) == UNSUPPORTED and "64 or 128" in last_error()
    assert at(D=64) == UNSUPPORTED          # o is (1, 64, 2, 128): shape mismatch
    o64 = h.tensor((1, 64, 2, 64))
    assert at(D=64, o=o64) == UNSUPPORTED and "device" in last_error().lower()
    assert at(S=65) == UNSUPPORTED          # o's shape differs from (B, S, H, D)
    assert at() == UNSUPPORTED and "device" in last_error().lower()

    def at_lse(lse, S=64, sm=0.1):
        return L.sage_attn_lse(*ptrs, 1, S, 2, 128, sm, ctypes.byref(o), lse, None)

    assert at_lse(None) == INVALID and "lse" in last_error()
    assert at_lse(None, sm=-1.0) == INVALID
    assert at_lse(ctypes.c_void_p(h.buf().value + 1)) == UNSUPPORTED and "aligned" in last_error()
    assert at_lse(h.buf()) == UNSUPPORTED and "device" in last_error().lower()
    z = (1, 0, 2, 128)
    oz = h.tensor(z)
    assert L.sage_attn_lse(*ptrs, 1, 0, 2, 128, 0.1, ctypes.byref(oz), None, None) == OK   # empty: nothing to write

    def at_ex(causal, lse, S=64, D=128, sm=0.1, o=o):
        return L.sage_attn_ex(*ptrs, 1, S, 2, D, sm, causal, ctypes.byref(o), lse, None)

    # lse is optional here; causal and non-causal both reach the device check
    for causal in (0, 1):
        assert at_ex(causal, None) == UNSUPPORTED and "device" in last_error().lower()
        assert at_ex(causal, h.buf()) == UNSUPPORTED and "device" in last_error().lower()
        assert at_ex(causal, None, sm=0.0) == INVALID
        assert at_ex(causal, ctypes.c_void_p(h.buf().value + 2)) == UNSUPPORTED and "aligned" in last_error()
        assert at_ex(causal, None, D=96) == UNSUPPORTED and "64 or 128" in last_error()
    assert L.sage_attn_ex(*ptrs, 1, 0, 2, 128, 0.1, 1, ctypes.byref(oz), None, None) == OK


def test_python_binding_raises_typed_errors():
    with pytest.raises(sage.SageUnsupported):
        sage.check(UNSUPPORTED)
    with pytest.raises(ValueError):
        sage.check(INVALID)
    with pytest.raises(ValueError):
        sage.check(WS_SMALL)
    with pytest.raises(RuntimeError):
        sage.check(DEVICE)


def test_binding_refuses_host_tensors_before_any_library_call():
    """The library takes device pointers; the binding turns host tensors into an
    error (a host pointer reaching a kernel would fault the GPU)."""
    import torch
    q = torch.zeros((1, 64, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        sage.sageattn(q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        sage.prepare(q, q, q)
    prep = {key: torch.zeros(4) for key in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale")}
    with pytest.raises(ValueError, match="GPU"):
        sage.attn(prep, 0.1)


def test_prepare_noalloc_validates_and_rejects_problems_beyond_its_scratch():
    """The allocation-free prologue checks its arguments like sage_prepare and
    refuses a problem whose statistics do not fit its static scratch, all
    before any device call."""
    h = Host()
    L = sage.lib()
    outs = [h.buf() for _ in range(7)]
    q, k, v = h.tensor(), h.tensor(), h.tensor()
    assert L.sage_prepare_noalloc(None, ctypes.byref(k), ctypes.byref(v), 1, *outs, None) == INVALID
    assert L.sage_prepare_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1, None, *outs[1:], None) == INVALID
    bad = h.tensor(dtype=2)
    assert L.sage_prepare_noalloc(ctypes.byref(q), ctypes.byref(bad), ctypes.byref(v), 1, *outs, None) == UNSUPPORTED
    big = (512, 4096, 32, 128)
    assert L.sage_prepare_workspace_bytes(*big, 1) > (16 << 20)
    qb, kb, vb = h.tensor(size=big), h.tensor(size=big), h.tensor(size=big)
    assert L.sage_prepare_noalloc(ctypes.byref(qb), ctypes.byref(kb), ctypes.byref(vb), 1, *outs, None) == WS_SMALL
    assert "static scratch" in L.sage_last_error().decode()
    empty = h.tensor(size=(0, 64, 2, 128))
    assert L.sage_prepare_noalloc(ctypes.byref(empty), ctypes.byref(empty), ctypes.byref(empty), 1, *outs, None) == OK
