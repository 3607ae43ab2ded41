"""Host-side checks of the Python binding's argument marshalling (no GPU)."""
import ctypes

import numpy as np
import pytest

import quantized_attention_prepare_amd as sage


def _fresh_buf():
    arr = (sage.SageTensor * 4)()
    elems = [arr[i] for i in range(4)]
    return arr, elems, [ctypes.byref(e) for e in elems]


@pytest.mark.parametrize("layout", ["NHD", "HND"])
def test_in_place_descriptors_equal_describe(layout):
    """The fused call's in-place descriptors hold the bytes describe() builds,
    for contiguous tensors, strided views and every dtype code, in each of the
    four slots."""
    import torch
    rng = np.random.default_rng(5)
    buf = _fresh_buf()
    for case in range(40):
        shape = [int(x) for x in rng.integers(1, 6, 4)]
        dtype = [torch.bfloat16, torch.float16, torch.float32, torch.int8][case % 4]
        base = torch.zeros([s * 2 for s in shape], dtype=torch.float32).to(dtype)
        t = base[::2, ::2, ::2, ::2] if case % 3 == 0 else base[: shape[0], : shape[1], : shape[2], : shape[3]]
        if case % 5 == 0:
            t = t.contiguous()
        slot = case % 4
        sage._fill(buf, slot, t, layout)
        assert bytes(buf[1][slot]) == bytes(sage.describe(t, layout)), (case, shape, dtype)


def test_in_place_descriptors_reject_what_describe_rejects():
    import torch
    buf = _fresh_buf()
    with pytest.raises(ValueError):
        sage._fill(buf, 0, torch.zeros((2, 3, 4)), "NHD")
    with pytest.raises(ValueError):
        sage._fill(buf, 0, torch.zeros((2, 3, 4, 5)), "HSD")


def test_host_tensors_are_refused_before_the_library():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        sage._gpu_of(torch.zeros(2))
