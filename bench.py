"""Benchmark of the quantized attention forward on one MI355X.

One step = the whole hot path (prologue + attention: sage_attn_fused) over
one batch of synthetic input already resident in HBM. Default workload: the
video-DiT-like shape B=1, H=28, S=32768, D=128 with smooth_k on (the first
configuration at S >= 16k, where the attention throughput target is stated).

Prints ONE JSON line with the step throughput (attention TFLOPS,
4*B*H*S^2*D per second of whole step), the roofline of the dominant kernel
(the attention kernel, timed alone with HIP events on its stream, against the
dense INT8/FP8 MFMA peak of 5.0 POP/s), the prologue's HBM bandwidth against
8 TB/s, the other workloads' figures, and the CPU oracle timed on a bounded
sample on this host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense INT8 (POP/s) and FP8 (PFLOP/s): 5.0 P
HBM_PEAK_GBS = 8000.0       # MI355X HBM3E: 8 TB/s


def attn_flops(w, causal: bool = False) -> float:
    """4*D ops per query-key pair the rows see: S^2 pairs per head, S(S+1)/2 when causal."""
    pairs = w.S * (w.S + 1) / 2 if causal else float(w.S) * w.S
    return 4.0 * w.B * w.H * pairs * w.D


def prologue_compulsory_bytes(w) -> int:
    """Read Q, K, V once as BF16 and write the INT8/FP8 codes once (9 B per element), plus scales."""
    n = w.B * w.S * w.H * w.D
    blocks = w.B * w.H * (-(-w.S // 32))
    return 9 * n + 2 * 4 * blocks + 4 * w.B * w.H * w.D * (2 if w.smooth_k else 1)


def kernel_source_hash(main: str = "attention.hip") -> str:
    """First 16 hex digits of sha256 over the code of a kernel source and the shared
    headers it includes, with comments removed and every run of whitespace made one
    space: a comment edit or a re-indent keeps the hash."""
    h = hashlib.sha256()
    for f in (main, "sage_internal.hpp", "prologue_ops.hpp"):
        with open(os.path.join(ROOT, "quantized_attention_prepare_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_prologue_traffic(workload: str):
    """HBM bytes of one prologue call (its three kernels) from committed counters, if taken on this source."""
    path = os.path.join(ROOT, "profiles", f"prologue_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("prologue_source_sha") != kernel_source_hash("prologue.hip"):
        return None
    return rec.get("traffic_bytes_per_call")


def load_traffic(workload: str):
    """HBM bytes per attention launch from committed rocprofv3 counters, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"attn_kernel_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def to_dev(bits):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def time_events(fn, iters: int, stream) -> float:
    """Average milliseconds of fn() over iters launches, HIP events on `stream`."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def measure(w, steps: int, warmup: int, causal: bool = False, keep_head: bool = False):
    import torch
    import quantized_attention_prepare_amd as sage
    import synth

    q, k, v = (to_dev(synth.tensor(w, x)) for x in "qkv")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(q)
    ws = torch.empty(sage.fused_workspace_bytes(w.B, w.S, w.H, w.D), dtype=torch.uint8, device=q.device)

    def step():
        sage.sageattn(q, k, v, "NHD", causal, w.sm_scale, False, w.smooth_k, out=out, workspace=ws, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms_ev = time_events(step, steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps

    # the two parts alone, each timed with events on the same stream
    prep = sage.prepare(q, k, v, w.smooth_k, stream=stream)
    o2 = torch.empty_like(q)
    for _ in range(max(1, warmup)):
        sage.attn(prep, w.sm_scale, out=o2, stream=stream, is_causal=causal)
    attn_ms = time_events(lambda: sage.attn(prep, w.sm_scale, out=o2, stream=stream, is_causal=causal), steps, stream)
    prep_ms = time_events(lambda: sage.prepare(q, k, v, w.smooth_k, stream=stream, reuse=prep), steps, stream)
    torch.cuda.synchronize()
    # the output rows of head (0, 0) from the last timed step, for the CPU leg's accuracy check
    head = out[0, :, 0, :].contiguous().view(torch.int16).cpu().numpy() if keep_head else None
    del q, k, v, out, ws, prep, o2
    torch.cuda.empty_cache()
    return dict(step_ms=step_ms_ev, step_wall_ms=wall_ms, attn_ms=attn_ms, prologue_ms=prep_ms, head=head)


def one_call_at_a_time(w, calls: int, causal: bool = False):
    """Each fused call timed alone: events around the call, synchronised before
    the next one starts (no overlap with other calls). Median and minimum, ms."""
    import torch
    import quantized_attention_prepare_amd as sage
    import synth

    q, k, v = (to_dev(synth.tensor(w, x)) for x in "qkv")
    stream = torch.cuda.current_stream()
    out = torch.empty_like(q)
    ws = torch.empty(sage.fused_workspace_bytes(w.B, w.S, w.H, w.D), dtype=torch.uint8, device=q.device)
    ts = []
    for i in range(calls + 20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sage.sageattn(q, k, v, "NHD", causal, w.sm_scale, False, w.smooth_k, out=out, workspace=ws, stream=stream)
        e1.record(stream)
        e1.synchronize()
        if i >= 20:   # warm-up calls
            ts.append(e0.elapsed_time(e1))
    ts.sort()
    return {"median_ms": round(ts[len(ts) // 2], 4), "min_ms": round(ts[0], 4), "calls": calls}


def cold_prologue(w, calls: int = 10):
    """The prologue timed with the memory-side cache flushed before each call
    (a 512 MiB buffer is written first, twice the cache): median and minimum, ms."""
    import torch
    import quantized_attention_prepare_amd as sage
    import synth

    q, k, v = (to_dev(synth.tensor(w, x)) for x in "qkv")
    stream = torch.cuda.current_stream()
    prep = sage.prepare(q, k, v, w.smooth_k, stream=stream)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=q.device)
    ts = []
    for _ in range(calls):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sage.prepare(q, k, v, w.smooth_k, stream=stream, reuse=prep)
        e1.record(stream)
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    del q, k, v, prep, flush
    torch.cuda.empty_cache()
    return {"median_ms": round(ts[len(ts) // 2], 4), "min_ms": round(ts[0], 4), "calls": calls}


def in_step_prologue(w, steps: int = 10):
    """The prologue as it runs inside a step: each step is the prologue then the
    attention launch on one stream (the kernels of the fused call), events around
    the prologue alone, read after the last step. Median and minimum, ms."""
    import torch
    import quantized_attention_prepare_amd as sage
    import synth

    q, k, v = (to_dev(synth.tensor(w, x)) for x in "qkv")
    stream = torch.cuda.current_stream()
    prep = sage.prepare(q, k, v, w.smooth_k, stream=stream)
    o = torch.empty_like(q)
    evs = []
    for i in range(steps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        sage.prepare(q, k, v, w.smooth_k, stream=stream, reuse=prep)
        e1.record(stream)
        sage.attn(prep, w.sm_scale, out=o, stream=stream)
        if i >= 2:   # the first two steps warm up
            evs.append((e0, e1))
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    del q, k, v, prep, o
    torch.cuda.empty_cache()
    return {"median_ms": round(ts[len(ts) // 2], 4), "min_ms": round(ts[0], 4), "steps": steps}


def _prologue_figures(t, pro_bytes, pro_traffic, cache):
    ms = t["median_ms"]
    rec = {"ms": ms, "cache": cache, "compulsory_bytes": pro_bytes,
           "gbs": round(pro_bytes / (ms * 1e-3) / 1e9, 1),
           "frac_of_hbm_peak": round(pro_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "counted_bytes": pro_traffic,
           "counted_gbs": round(pro_traffic / (ms * 1e-3) / 1e9, 1) if pro_traffic else None,
           "counted_frac_of_hbm_peak": (round(pro_traffic / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                        if pro_traffic else None)}
    for key in ("min_ms", "calls", "steps"):
        if key in t:
            rec[key] = t[key]
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(w, budget_s: float = 12.0, gpu_head=None):
    """The CPU oracle on a bounded sample of the workload: the prologue of one
    head plus as many of that head's query rows as fit the time budget. With
    gpu_head (the GPU's BF16 output bits of head (0, 0), [S, D]) it also
    returns the GPU's error on the rows the oracle computed."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    nthreads = oracle.threads()
    qh, kh, vh = (synth.head(w, x, 0, 0) for x in "qkv")
    t0 = time.perf_counter()
    prep = oracle.prepare_head(qh, kh, vh, w.smooth_k)
    t_prep = time.perf_counter() - t0
    rows_done = 0
    t_attn = 0.0
    start = int(synth.sample_rows(w, 1)[0, 2])
    rows, bits = [], []
    with ThreadPoolExecutor(nthreads) as ex:
        while t_attn < budget_s and rows_done < w.S:
            batch = [(start + rows_done + i) % w.S for i in range(nthreads)]
            t1 = time.perf_counter()
            res = list(ex.map(lambda r: oracle.attn_rows_head(prep, [r], w.sm_scale), batch))
            t_attn += time.perf_counter() - t1
            rows_done += len(batch)
            rows += batch
            bits += res
    ops = 4.0 * rows_done * w.S * w.D
    t_share = t_prep * rows_done / w.S
    accuracy = None
    if gpu_head is not None:
        ref = oracle.bf16_bits_to_f64(np.concatenate(bits).astype(np.uint16))
        got = oracle.bf16_bits_to_f64(gpu_head.view(np.uint16)[np.array(rows)])
        accuracy = {"rows": len(rows), "head": "(0, 0)", "maxabs_vs_oracle": round(oracle.max_abs_rel(got, ref), 6),
                    "cos_vs_oracle": round(oracle.cosine(got, ref), 8),
                    "bits_equal_frac": round(float(np.mean(got == ref)), 4)}
    return accuracy, {"value": ops / (t_attn + t_share) / 1e12, "unit": "TFLOPS", "cores": nthreads, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"{w.name}: oracle prologue of head (0,0) ({w.S} rows, {t_prep:.2f} s, charged pro rata) + "
                      f"quantized attention of {rows_done} consecutive query rows of that head from a seeded start "
                      f"({t_attn:.2f} s); "
                      f"{nthreads} threads (the CPU share one GPU's job is given; the host shows "
                      f"{os.cpu_count()} CPUs) on {cpu_model()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="C3")
    ap.add_argument("--others", default="C1,C2,C4,C5,C6,C3:causal",
                    help="comma list of further workloads to report, NAME or NAME:causal ('' for none)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 512 MiB five times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 4
        # also the practical streaming rate the prologue's passes are held against
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n, "launches": 5,
                          "copy_ms": round(ms, 4), "copy_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}))
        return

    w = synth.WORKLOADS[args.workload]
    r = measure(w, args.steps, args.warmup, keep_head=not args.no_cpu)
    fl = attn_flops(w)
    value = fl / (r["step_ms"] * 1e-3) / 1e12
    achieved = fl / (r["attn_ms"] * 1e-3) / 1e12
    pro_bytes = prologue_compulsory_bytes(w)
    pro_traffic = load_prologue_traffic(w.name)
    cold = cold_prologue(w)
    in_step = in_step_prologue(w)
    others = {}
    for name in [x for x in args.others.split(",") if x and x != args.workload]:
        base, _, mode = name.partition(":")
        causal = mode == "causal"
        wo = synth.WORKLOADS[base]
        ro = measure(wo, max(5, args.steps // 2), max(2, args.warmup // 2), causal=causal)
        fo = attn_flops(wo, causal)
        others[name] = {"step_ms": round(ro["step_ms"], 4),
                        "step_tflops": round(fo / (ro["step_ms"] * 1e-3) / 1e12, 1),
                        "attn_ms": round(ro["attn_ms"], 4),
                        "attn_tflops": round(fo / (ro["attn_ms"] * 1e-3) / 1e12, 1),
                        "prologue_ms": round(ro["prologue_ms"], 4),
                        "prologue_gbs": round(prologue_compulsory_bytes(wo) / (ro["prologue_ms"] * 1e-3) / 1e9, 1)}
        # attention roofline: min(MFMA peak, arithmetic intensity x HBM peak) on 5 algorithmic bytes per element
        ai = fo / (5.0 * wo.B * wo.S * wo.H * wo.D)
        bound = min(MFMA_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
        others[name]["attn_roofline_tflops"] = round(bound, 1)
        others[name]["attn_roofline_frac"] = round(fo / (ro["attn_ms"] * 1e-3) / 1e12 / bound, 4)
        if base in ("C1", "C5") and not causal:
            # short calls, each timed alone and synchronised before the next one
            others[name]["one_call_at_a_time"] = one_call_at_a_time(wo, 200)
        if base != "C4" and not causal:
            # the inputs of C1, C2 and C5 fit in the 256 MB memory-side cache: the warm
            # prologue time above reads them from there, the flushed one from HBM
            co = cold_prologue(wo)
            others[name]["prologue_cold_ms"] = co["median_ms"]
            others[name]["prologue_cold_gbs"] = round(prologue_compulsory_bytes(wo) / (co["median_ms"] * 1e-3) / 1e9, 1)
    line = {
        "metric": "attention TFLOPS (4*B*H*S^2*D/s) at H=28 D=128; prologue HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+fp8",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.note}, D=128, smooth_k {'on' if w.smooth_k else 'off'}, "
                               f"non-causal, sm_scale 1/sqrt(128)",
                   "B": w.B, "H": w.H, "S": w.S, "D": w.D, "smooth_k": w.smooth_k},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS, 4), "traffic": load_traffic(w.name),
                     "kernel": "attn_kernel", "kernel_ms": round(r["attn_ms"], 4),
                     "algorithmic_per_launch": f"{fl:.4e} ops (4*D ops per query-key pair)"},
        # the prologue's headline is a call with the 256 MB memory-side cache flushed first (512 MiB
        # written before each call, so the inputs come from HBM); beside it the prologue as the step
        # runs it (each call right after an attention launch on the same stream) and back-to-back
        # calls on the same inputs, which find part of them in that cache. "gbs" and
        # "frac_of_hbm_peak" count the compulsory bytes (read Q, K, V once, write the codes once);
        # "counted_gbs" counts the rocprofv3 bytes (FETCH_SIZE x 2 + WRITE_SIZE, calibrated on a copy),
        # which are what the L2 fetches and writes, memory-side cache hits included: an upper bound
        # of the bytes that cross the HBM interface
        "prologue": _prologue_figures(cold, pro_bytes, pro_traffic, "512 MiB written before each call") | {
                     "in_step": _prologue_figures(in_step, pro_bytes, pro_traffic,
                                                  "each call follows an attention launch on the same stream"),
                     "warm": _prologue_figures({"median_ms": round(r["prologue_ms"], 4)}, pro_bytes, pro_traffic,
                                               "back-to-back calls on the same inputs")},
        "step_wall_ms": round(r["step_wall_ms"], 4),
        "one_call_at_a_time": one_call_at_a_time(w, 10),
        "other_workloads": others,
    }
    if not args.no_cpu:
        accuracy, line["cpu_baseline"] = cpu_baseline(w, gpu_head=r["head"])
        line["accuracy_vs_oracle"] = accuracy
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
