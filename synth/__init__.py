"""Seeded synthetic inputs shared by the CPU oracle side and the GPU side.

The generator itself is ``synth.c`` (counter-based SplitMix64, Box-Muller in
double, then float, then BF16 round-to-nearest-even).  This module names the
five workloads and builds their BF16 tensors as numpy ``uint16`` bit patterns
in [B, S, H, D] order.  It contains none of the quantized attention method's
arithmetic.

Workloads (the pages measure on MiniMax-H3 text-to-video attention, BF16,
28 heads, head dim 128, with no token counts; these synthetic tensors stand in
for it):

  C1  B=1  H=2  S=256     Q,K,V ~ N(0,1)                                     smooth_k off
  C2  B=1  H=28 S=4096    Q,V ~ N(0,1); K = N(0,1) + bias[h,d], bias~N(0,2^2) smooth_k on
  C3  B=1  H=28 S=32768   Q = a_q[h] N(0,1), K = a_k[h] N(0,1), a ~ U[0.5,3]
                          (independent draws for Q and K); V ~ N(0,1)         smooth_k on
  C4  B=1  H=28 S=131072  Q,K,V ~ N(0,1)                                     smooth_k on
  C5  B=8  H=28 S=384     Q,V ~ N(0,1); K: each entry replaced with
                          probability 0.01 by N(0,20^2)                      smooth_k off

Seeds: 20261200 + 10*config + tensor id (Q=0, K=1, V=2, per-head scale /
bias / outlier values=3, outlier mask=4, sampled rows=5).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

NORMAL, HEAD_SCALE, CHANNEL_BIAS, OUTLIERS = 0, 1, 2, 3


class _Spec(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("seed", ctypes.c_uint64), ("aux_seed", ctypes.c_uint64),
                ("mask_seed", ctypes.c_uint64), ("p0", ctypes.c_double), ("p1", ctypes.c_double)]


def build() -> str:
    """Compile synth.c into libsynth.so next to it (always recompiles)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _LIB_PATH + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", tmp, src, "-lm"],
                   check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.synth_fill.argtypes = [ctypes.POINTER(_Spec), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_fill_head.argtypes = [ctypes.POINTER(_Spec), ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p]
        lib.synth_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_uniform.restype = ctypes.c_double
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_normal.restype = ctypes.c_double
        lib.synth_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.synth_splitmix64.restype = ctypes.c_uint64
        _lib = lib
    return _lib


@dataclass(frozen=True)
class TensorSpec:
    kind: int = NORMAL
    seed: int = 0
    aux_seed: int = 0
    mask_seed: int = 0
    p0: float = 0.0
    p1: float = 0.0

    def c(self) -> _Spec:
        return _Spec(self.kind, self.seed, self.aux_seed, self.mask_seed, self.p0, self.p1)


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    H: int
    S: int
    D: int
    smooth_k: bool
    q: TensorSpec
    k: TensorSpec
    v: TensorSpec
    oracle_rows: int | None  # None: every query row; else a seeded sample of this many rows
    note: str = ""

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.D))

    def spec(self, which: str) -> TensorSpec:
        return {"q": self.q, "k": self.k, "v": self.v}[which]

    def seed(self, tensor_id: int) -> int:
        return seed(self.index, tensor_id)


def seed(config_index: int, tensor_id: int) -> int:
    return 20261200 + 10 * config_index + tensor_id


def _normal(ci, tid):
    return TensorSpec(NORMAL, seed(ci, tid))


def _workloads():
    w = {}
    w["C1"] = Workload("C1", 1, 1, 2, 256, 128, False, _normal(1, 0), _normal(1, 1), _normal(1, 2), None,
                       "B=1 H=2 S=256, N(0,1)")
    w["C2"] = Workload("C2", 2, 1, 28, 4096, 128, True, _normal(2, 0),
                       TensorSpec(CHANNEL_BIAS, seed(2, 1), seed(2, 3), 0, 2.0), _normal(2, 2), None,
                       "B=1 H=28 S=4096, K with per-channel bias N(0,2^2)")
    w["C3"] = Workload("C3", 3, 1, 28, 32768, 128, True,
                       TensorSpec(HEAD_SCALE, seed(3, 0), seed(3, 3), 0, 0.5, 3.0),
                       TensorSpec(HEAD_SCALE, seed(3, 1), seed(3, 3) + 1_000_000, 0, 0.5, 3.0),
                       _normal(3, 2), 8192, "video-DiT-like B=1 H=28 S=32768, per-head scales U[0.5,3]")
    w["C4"] = Workload("C4", 4, 1, 28, 131072, 128, True, _normal(4, 0), _normal(4, 1), _normal(4, 2), 512,
                       "long sequence B=1 H=28 S=131072")
    w["C5"] = Workload("C5", 5, 8, 28, 384, 128, False, _normal(5, 0),
                       TensorSpec(OUTLIERS, seed(5, 1), seed(5, 3), seed(5, 4), 0.01, 20.0), _normal(5, 2), None,
                       "many short calls B=8 H=28 S=384, 1% K outliers N(0,20^2)")
    # head dim 64 (an extension beyond the pages' D = 128): the video-DiT-like
    # token count with the same H * D as C3
    w["C6"] = Workload("C6", 6, 1, 56, 32768, 64, True,
                       TensorSpec(HEAD_SCALE, seed(6, 0), seed(6, 3), 0, 0.5, 3.0),
                       TensorSpec(HEAD_SCALE, seed(6, 1), seed(6, 3) + 1_000_000, 0, 0.5, 3.0),
                       _normal(6, 2), 8192, "head dim 64: B=1 H=56 S=32768 D=64, per-head scales U[0.5,3]")
    return w


WORKLOADS = _workloads()


def custom(B, S, H, D=128, smooth_k=False, base_seed=777, kinds=None) -> Workload:
    """A workload of any shape with N(0,1) inputs (or the given TensorSpecs), for tests."""
    kinds = kinds or {}
    q = kinds.get("q", TensorSpec(NORMAL, base_seed))
    k = kinds.get("k", TensorSpec(NORMAL, base_seed + 1))
    v = kinds.get("v", TensorSpec(NORMAL, base_seed + 2))
    return Workload(f"custom{B}x{S}x{H}x{D}", 0, B, H, S, D, smooth_k, q, k, v, None, "custom")


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def tensor(w: Workload, which: str, threads: int | None = None) -> np.ndarray:
    """BF16 bit patterns of Q, K or V for the whole workload, shape [B, S, H, D], dtype uint16."""
    lib = _load()
    n = w.B * w.S * w.H * w.D
    out = np.empty(n, dtype=np.uint16)
    sp = w.spec(which).c()
    nt = threads or _threads()
    step = max(1, -(-n // (nt * 8)))
    ptr = out.ctypes.data

    def job(s0):
        lib.synth_fill(ctypes.byref(sp), w.S, w.H, w.D, s0, min(n, s0 + step), ctypes.c_void_p(ptr))

    if n:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(job, range(0, n, step)))
    return out.reshape(w.B, w.S, w.H, w.D)


def head(w: Workload, which: str, b: int, h: int, s0: int = 0, s1: int | None = None) -> np.ndarray:
    """Rows [s0, s1) of head (b, h) as a dense [rows, D] uint16 array (same bits as tensor())."""
    lib = _load()
    s1 = w.S if s1 is None else s1
    out = np.empty((s1 - s0, w.D), dtype=np.uint16)
    sp = w.spec(which).c()
    lib.synth_fill_head(ctypes.byref(sp), w.S, w.H, w.D, b, h, s0, s1, ctypes.c_void_p(out.ctypes.data))
    return out


def sample_rows(w: Workload, n: int) -> np.ndarray:
    """n distinct seeded query rows as an int64 array of (b, h, s) triples, sorted."""
    lib = _load()
    total = w.B * w.H * w.S
    n = min(n, total)
    chosen: set[int] = set()
    ctr = 0
    sd = w.seed(5)
    while len(chosen) < n:
        chosen.add(int(lib.synth_splitmix64(sd, ctr) % total))
        ctr += 1
    flat = np.array(sorted(chosen), dtype=np.int64)
    s = flat % w.S
    bh = flat // w.S
    return np.stack([bh // w.H, bh % w.H, s], axis=1)


def uniform(seed_: int, n: int) -> float:
    return float(_load().synth_uniform(seed_, n))


def normal(seed_: int, n: int) -> float:
    return float(_load().synth_normal(seed_, n))


def bf16_to_float(bits: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32 (a bit shift)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)
