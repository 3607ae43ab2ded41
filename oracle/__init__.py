"""CPU oracle for the quantized attention forward (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports, links or
calls it.  The arithmetic lives in ``oracle.c`` (plain C, one step at a time,
no fast-math, no contraction); this module only marshals numpy arrays and
spreads independent heads / rows over threads (each C call is single-threaded
and releases the GIL).

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against things other than itself (brute-force nearest-code search, the
correctly rounded sum ``math.fsum``, torch's float8 and round routines,
hand-worked blocks, exactly representable attention cases worked by hand in
rational arithmetic, fp64 exact attention within a derived error bound, and
invariants).  The exact output bits of the quantized attention are not pinned
by anything but the oracle's own definition; only closed-form cases and the
error bound against exact attention pin them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_TILE = 128  # keys per online-softmax tile (part of the result's definition)


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-o", tmp, os.path.join(_HERE, "oracle.c"), "-lm"], check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = ctypes.c_float
        L.oracle_bf16_encode.argtypes = [ctypes.c_float]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_float
        L.oracle_quant_block_int8.argtypes = [_P, _I, _I, _P]
        L.oracle_quant_block_int8.restype = ctypes.c_float
        L.oracle_bf16_exact_sum.argtypes = [_P, _I, _I]
        L.oracle_bf16_exact_sum.restype = ctypes.c_double
        L.oracle_prepare_head.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_int, _I, _P, _P, _P, _P, _P, _P, _P]
        L.oracle_prepare_head.restype = ctypes.c_int
        L.oracle_attn_rows.argtypes = [_P, _P, _P, _P, _P, _I, _P, _I, _I, ctypes.c_float, _I, ctypes.c_int, _P, _I,
                                       _P, _P, _P]
        L.oracle_attn_rows.restype = ctypes.c_int
        L.oracle_exact_rows.argtypes = [_P, _P, _P, _I, _I, _I, ctypes.c_double, ctypes.c_int, _P, _I, _P, _P]
        L.oracle_exact_rows.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def threads() -> int:
    """Worker threads: the host's CPUs, at most 16 (the CPU share a one-GPU
    job is given on the machines this runs on, whatever the host shows)."""
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------ scalar codecs
def e4m3_encode(x: float) -> int:
    return int(lib().oracle_e4m3_encode(float(x)))


def e4m3_decode(c: int) -> float:
    return float(lib().oracle_e4m3_decode(int(c)))


def e4m3_encode_array(x: np.ndarray) -> np.ndarray:
    f = lib().oracle_e4m3_encode
    return np.array([f(float(v)) for v in np.asarray(x, np.float32).ravel()], dtype=np.uint8).reshape(np.shape(x))


def e4m3_decode_table() -> np.ndarray:
    """Decoded value of every one of the 256 codes (NaN for 0x7F / 0xFF)."""
    return np.array([lib().oracle_e4m3_decode(c) for c in range(256)], dtype=np.float32)


def bf16_encode_array(x: np.ndarray) -> np.ndarray:
    f = lib().oracle_bf16_encode
    return np.array([f(float(v)) for v in np.asarray(x, np.float32).ravel()], dtype=np.uint16).reshape(np.shape(x))


def quant_block_int8(x: np.ndarray) -> tuple[np.ndarray, float]:
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, D = x.shape
    q = np.empty((rows, D), dtype=np.int8)
    s = lib().oracle_quant_block_int8(_ptr(x), rows, D, _ptr(q))
    return q, float(s)


def bf16_exact_sum(x: np.ndarray) -> float:
    """Exact sum of BF16 values (uint16 bits) rounded once to double."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.uint16).ravel())
    return float(lib().oracle_bf16_exact_sum(_ptr(x), x.size, 1))


# ------------------------------------------------------------ prologue
def s_pad(S: int, T: int = KV_TILE) -> int:
    return -(-S // T) * T


def prepare_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, smooth_k: bool, S_pad: int | None = None) -> dict:
    """Prologue of one head from dense [S, D] BF16 (uint16) arrays."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    S, D = q.shape
    S_pad = s_pad(S) if S_pad is None else S_pad
    nb = -(-S // 32)
    out = dict(q8=np.empty((S, D), np.int8), q_scale=np.empty(nb, np.float32), k8=np.empty((S, D), np.int8),
               k_scale=np.empty(nb, np.float32), v8t=np.empty((D, S_pad), np.uint8),
               v_scale=np.empty(D, np.float32), k_mean=np.empty(D, np.float32))
    rc = lib().oracle_prepare_head(_ptr(q), _ptr(k), _ptr(v), S, D, D, int(bool(smooth_k)), S_pad, _ptr(out["q8"]),
                                   _ptr(out["q_scale"]), _ptr(out["k8"]), _ptr(out["k_scale"]), _ptr(out["v8t"]),
                                   _ptr(out["v_scale"]), _ptr(out["k_mean"]))
    if rc != 0:
        raise ValueError("oracle_prepare_head rejected its arguments")
    return out


def prepare(q: np.ndarray, k: np.ndarray, v: np.ndarray, smooth_k: bool, heads=None, nthreads=None) -> dict:
    """Prologue of whole [B, S, H, D] BF16 tensors.

    Returns arrays in the library's layouts: q8/k8 [B,H,S,D], q_scale/k_scale
    [B,H,ceil(S/32)], v8t [B,H,D,S_pad], v_scale/k_mean [B,H,D].  With
    ``heads`` (a list of (b, h)) only those heads are computed; the others
    are left uninitialised.
    """
    B, S, H, D = q.shape
    for a in (q, k, v):
        assert a.shape == (B, S, H, D) and a.dtype == np.uint16 and a.flags.c_contiguous
    Sp = s_pad(S)
    nb = -(-S // 32)
    out = dict(q8=np.empty((B, H, S, D), np.int8), q_scale=np.empty((B, H, nb), np.float32),
               k8=np.empty((B, H, S, D), np.int8), k_scale=np.empty((B, H, nb), np.float32),
               v8t=np.empty((B, H, D, Sp), np.uint8), v_scale=np.empty((B, H, D), np.float32),
               k_mean=np.empty((B, H, D), np.float32))
    L = lib()
    rs = H * D

    def job(bh):
        b, h = bh
        off = (b * S * H + h) * D * 2  # bytes to element (b, 0, h, 0)
        rc = L.oracle_prepare_head(ctypes.c_void_p(q.ctypes.data + off), ctypes.c_void_p(k.ctypes.data + off),
                                   ctypes.c_void_p(v.ctypes.data + off), S, D, rs, int(bool(smooth_k)), Sp,
                                   _ptr(out["q8"][b, h]), _ptr(out["q_scale"][b, h]), _ptr(out["k8"][b, h]),
                                   _ptr(out["k_scale"][b, h]), _ptr(out["v8t"][b, h]), _ptr(out["v_scale"][b, h]),
                                   _ptr(out["k_mean"][b, h]))
        if rc != 0:
            raise ValueError("oracle_prepare_head rejected its arguments")

    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    with ThreadPoolExecutor(nthreads or threads()) as ex:
        list(ex.map(job, todo))
    return out


# ------------------------------------------------------------ attention
def attn_rows_head(prep_head: dict, rows, sm_scale: float, T: int = KV_TILE, want_f32: bool = False,
                   want_lse: bool = False, causal: bool = False):
    """Quantized attention for the given query rows of one head.

    prep_head holds that head's q8 [S,D], q_scale, k8, k_scale, v8t [D,S_pad],
    v_scale.  Returns BF16 bits [n, D], then (if asked) the pre-rounding float
    values and the rows' log-sum-exp of the dequantized scores (float [n]).
    causal: row i sees keys 0 .. i only.
    """
    q8 = np.ascontiguousarray(prep_head["q8"])
    S, D = q8.shape
    v8t = np.ascontiguousarray(prep_head["v8t"])
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.size
    ob = np.empty((n, D), np.uint16)
    of = np.empty((n, D), np.float32) if want_f32 else None
    ks = np.ascontiguousarray(prep_head["k_scale"], dtype=np.float32)
    qs = np.ascontiguousarray(prep_head["q_scale"], dtype=np.float32)
    vs = np.ascontiguousarray(prep_head["v_scale"], dtype=np.float32)
    k8 = np.ascontiguousarray(prep_head["k8"])
    lse = np.empty(n, np.float32) if want_lse else None
    rc = lib().oracle_attn_rows(_ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(v8t), v8t.shape[1], _ptr(vs), S, D,
                                float(sm_scale), int(T), int(bool(causal)), _ptr(rows), n, _ptr(of), _ptr(ob),
                                _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attn_rows rejected its arguments")
    extra = ([of] if want_f32 else []) + ([lse] if want_lse else [])
    return tuple([ob] + extra) if extra else ob


def head_of(prep: dict, b: int, h: int) -> dict:
    return {k: prep[k][b, h] for k in ("q8", "q_scale", "k8", "k_scale", "v8t", "v_scale", "k_mean")}


def attn(prep: dict, sm_scale: float, rows=None, T: int = KV_TILE, nthreads=None, chunk: int = 64,
         want_lse: bool = False, causal: bool = False):
    """Quantized attention over full-tensor prologue outputs.

    rows=None computes every row and returns BF16 bits [B, S, H, D] (and, with
    want_lse, the log-sum-exp float [B, H, S]).
    rows = int array [n, 3] of (b, h, s) returns BF16 bits [n, D] (and float [n]).
    """
    B, H, S, D = prep["q8"].shape
    if rows is None:
        out = np.empty((B, S, H, D), np.uint16)
        lse_all = np.empty((B, H, S), np.float32) if want_lse else None
        jobs = [(b, h, s0) for b in range(B) for h in range(H) for s0 in range(0, S, chunk)]

        def job(j):
            b, h, s0 = j
            r = np.arange(s0, min(S, s0 + chunk), dtype=np.int64)
            res = attn_rows_head(head_of(prep, b, h), r, sm_scale, T, want_lse=want_lse, causal=causal)
            if want_lse:
                out[b, s0:s0 + r.size, h, :], lse_all[b, h, s0:s0 + r.size] = res
            else:
                out[b, s0:s0 + r.size, h, :] = res

        with ThreadPoolExecutor(nthreads or threads()) as ex:
            list(ex.map(job, jobs))
        return (out, lse_all) if want_lse else out
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.uint16)
    lse_rows = np.empty(rows.shape[0], np.float32) if want_lse else None
    groups = {}
    for idx, (b, h, s) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(idx)
    jobs = []
    for (b, h), idxs in groups.items():
        for c in range(0, len(idxs), chunk):
            jobs.append((b, h, idxs[c:c + chunk]))

    def job2(j):
        b, h, idxs = j
        res = attn_rows_head(head_of(prep, b, h), rows[idxs, 2], sm_scale, T, want_lse=want_lse, causal=causal)
        if want_lse:
            out[idxs], lse_rows[idxs] = res
        else:
            out[idxs] = res

    with ThreadPoolExecutor(nthreads or threads()) as ex:
        list(ex.map(job2, jobs))
    return (out, lse_rows) if want_lse else out


def exact_rows_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows, sm_scale: float, want_lse: bool = False,
                    causal: bool = False):
    """fp64 exact attention rows of one head from dense [S, D] BF16 arrays
    (and, if asked, each row's ln sum_j exp(q.k_j * sm_scale)); causal: keys j <= i."""
    q, k, v = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q, k, v))
    S, D = q.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.empty((rows.size, D), np.float64)
    lse = np.empty(rows.size, np.float64) if want_lse else None
    rc = lib().oracle_exact_rows(_ptr(q), _ptr(k), _ptr(v), S, D, D, float(sm_scale), int(bool(causal)), _ptr(rows),
                                 rows.size, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_exact_rows rejected its arguments")
    return (out, lse) if want_lse else out


def exact(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float, rows=None, nthreads=None, chunk: int = 32,
          causal: bool = False):
    """fp64 exact attention over [B, S, H, D] BF16 tensors (all rows, or (b,h,s) rows); causal: keys j <= i."""
    B, S, H, D = q.shape
    L = lib()
    rs = H * D

    def run(b, h, rr):
        off = (b * S * H + h) * D * 2
        rr = np.ascontiguousarray(rr, dtype=np.int64)
        o = np.empty((rr.size, D), np.float64)
        rc = L.oracle_exact_rows(ctypes.c_void_p(q.ctypes.data + off), ctypes.c_void_p(k.ctypes.data + off),
                                 ctypes.c_void_p(v.ctypes.data + off), S, D, rs, float(sm_scale), int(bool(causal)),
                                 _ptr(rr), rr.size, _ptr(o), None)
        if rc != 0:
            raise ValueError("oracle_exact_rows rejected its arguments")
        return o

    if rows is None:
        out = np.empty((B, S, H, D), np.float64)
        jobs = [(b, h, s0) for b in range(B) for h in range(H) for s0 in range(0, S, chunk)]

        def job(j):
            b, h, s0 = j
            r = np.arange(s0, min(S, s0 + chunk))
            out[b, s0:s0 + r.size, h, :] = run(b, h, r)

        with ThreadPoolExecutor(nthreads or threads()) as ex:
            list(ex.map(job, jobs))
        return out
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], D), np.float64)
    groups = {}
    for idx, (b, h, s) in enumerate(rows):
        groups.setdefault((int(b), int(h)), []).append(idx)
    jobs = []
    for (b, h), idxs in groups.items():
        for c in range(0, len(idxs), chunk):
            jobs.append((b, h, idxs[c:c + chunk]))

    def job2(j):
        b, h, idxs = j
        out[idxs] = run(b, h, rows[idxs, 2])

    with ThreadPoolExecutor(nthreads or threads()) as ex:
        list(ex.map(job2, jobs))
    return out


# ------------------------------------------------------------ metrics
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cosine(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(np.dot(a, b) / (np.linalg.norm(a) * np.linalg.norm(b)))


def max_abs_rel(a: np.ndarray, ref: np.ndarray) -> float:
    """max|a - ref| / max|ref| over the compared elements."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(a - ref)) / np.max(np.abs(ref)))
