"""The allocation-free prologue, sage_prepare_noalloc, through the C ABI:
its outputs equal sage_prepare's bit for bit on two calls in a row (the
second on a smaller problem, so the static scratch holds the first call's
statistics when it starts), and a problem beyond the static scratch is
rejected before any device work."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

WS_SMALL = 3


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _outputs(B, S, H, D, Sp):
    import torch
    return dict(q8=torch.empty((B, H, Sp, D), dtype=torch.int8, device="cuda"),
                q_scale=torch.empty((B, H, Sp // 32), dtype=torch.float32, device="cuda"),
                k8=torch.empty((B, H, Sp, D), dtype=torch.int8, device="cuda"),
                k_scale=torch.empty((B, H, Sp // 32), dtype=torch.float32, device="cuda"),
                v8t=torch.empty((B, H, D, Sp), dtype=torch.uint8, device="cuda"),
                v_scale=torch.empty((B, H, D), dtype=torch.float32, device="cuda"),
                k_mean=torch.empty((B, H, D), dtype=torch.float32, device="cuda"))


KEYS = ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale", "k_mean")


def test_prepare_noalloc_equals_prepare_on_two_calls():
    import torch
    import quantized_attention_prepare_amd as sage
    L = sage.lib()
    stream = torch.cuda.current_stream()
    # the second call is smaller than the first; both have smooth_k on, and the
    # first has key channels whose fp64 sums are not exact (the exact path)
    for i, (B, S, H, D) in enumerate([(2, 5000, 6, 128), (1, 700, 3, 64)]):
        w = synth.custom(B, S, H, D=D, smooth_k=True, base_seed=9500 + i)
        q, k, v = (synth.tensor(w, x) for x in "qkv")
        if i == 0:
            kf = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).float()
            kf[:, :, :, 0] = torch.tensor([2.0 ** 60, 1.0, -(2.0 ** 60)])[torch.arange(S) % 3][None, :, None]
            k = kf.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        tq, tk, tv = _dev(q), _dev(k), _dev(v)
        ref = sage.prepare(tq, tk, tv, True)
        Sp = sage.padded_len(S)
        need = L.sage_prepare_workspace_bytes(B, S, H, D, 1)
        assert 0 < need <= (16 << 20)
        out = _outputs(B, S, H, D, Sp)
        for t in out.values():
            t.fill_(0x5A if t.dtype in (torch.int8, torch.uint8) else 7.0)
        d = [sage.describe(x) for x in (tq, tk, tv)]
        st = L.sage_prepare_noalloc(ctypes.byref(d[0]), ctypes.byref(d[1]), ctypes.byref(d[2]), 1,
                                    *[ctypes.c_void_p(out[key].data_ptr()) for key in KEYS],
                                    ctypes.c_void_p(stream.cuda_stream))
        assert st == 0, L.sage_last_error().decode()
        torch.cuda.synchronize()
        for key in KEYS:
            a, b = out[key], ref[key]
            if a.dtype == torch.float32:
                a, b = a.view(torch.int32), b.view(torch.int32)
            assert torch.equal(a, b), (i, key)


def test_prepare_noalloc_rejects_problems_beyond_its_scratch():
    import quantized_attention_prepare_amd as sage
    L = sage.lib()
    B, S, H, D = 512, 4096, 32, 128   # 16 384 heads: their per-channel statistics alone pass 16 MiB
    assert L.sage_prepare_workspace_bytes(B, S, H, D, 1) > (16 << 20)
    keep = []

    def desc():
        a = np.zeros(64, np.uint8)
        keep.append(a)
        base = (a.ctypes.data + 15) & ~15
        return sage.SageTensor(base, 1, (ctypes.c_int64 * 4)(B, S, H, D),
                               (ctypes.c_int64 * 4)(S * H * D, H * D, D, 1))

    q, k, v = desc(), desc(), desc()
    bufs = []
    for _ in KEYS:
        a = np.zeros(64, np.uint8)
        bufs.append(a)
    ptrs = [ctypes.c_void_p((a.ctypes.data + 15) & ~15) for a in bufs]
    st = L.sage_prepare_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1, *ptrs, None)
    assert st == WS_SMALL
    assert "static scratch" in L.sage_last_error().decode()
