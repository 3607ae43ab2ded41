"""CPU tests of bench.py's host-side accounting: the algorithmic work and bytes
it divides by, the code-only source hash that keys the committed counter
figures, and the single-GPU guard."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


# Attention work 4*B*H*S^2*D and prologue compulsory bytes (9 per element, plus
# 8 per 32-row block pair of scales and 4 or 8 per (b, h, d) for v_scale and
# k_mean), as tabulated for the five workloads before any code was written.
@pytest.mark.parametrize("name,ops,nbytes", [("C1", 6.711e7, 590_976), ("C2", 2.405e11, 132_177_920),
                                             ("C3", 1.539e13, 1_057_222_656), ("C4", 2.463e14, 4_228_804_608),
                                             ("C5", 1.691e10, 99_226_624)])
def test_work_and_compulsory_bytes_match_the_tabulated_values(name, ops, nbytes):
    w = synth.WORKLOADS[name]
    assert abs(bench.attn_flops(w) - ops) <= 5e-4 * ops
    assert bench.prologue_compulsory_bytes(w) == nbytes


def test_causal_work_counts_the_pairs_a_causal_row_sees():
    w = synth.WORKLOADS["C3"]
    pairs = w.B * w.H * w.S * (w.S + 1) // 2
    assert bench.attn_flops(w, causal=True) == 4.0 * w.D * pairs
    # a bit over half of the non-causal work
    assert 0.5 < bench.attn_flops(w, causal=True) / bench.attn_flops(w) < 0.5001


def _copy_tree(tmp_path):
    for sub in ("quantized_attention_prepare_amd/csrc", "profiles"):
        shutil.copytree(os.path.join(ROOT, sub), tmp_path / sub)


def test_source_hash_ignores_comments_and_whitespace_runs_not_code(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    src = tmp_path / "quantized_attention_prepare_amd/csrc/attention.hip"
    text = src.read_text()
    src.write_text("// a new comment line\n" + text.replace("\n", "\n\n", 5) + "\n/* and a block */\n")
    assert bench.kernel_source_hash() == h0
    src.write_text(text.replace("constexpr int kWaves = 4;", "constexpr   int\n  kWaves =\t4;"))
    assert bench.kernel_source_hash() == h0
    src.write_text(text.replace("constexpr int kWaves = 4;", "constexpr int kWaves = 8;"))
    assert bench.kernel_source_hash() != h0


def test_traffic_figures_are_used_only_for_the_sources_they_were_taken_on(tmp_path, monkeypatch):
    _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    attn, pro = bench.load_traffic("C3"), bench.load_prologue_traffic("C3")
    if attn is None or pro is None:
        pytest.skip("the committed counter figures were taken on other sources")
    for f, loader in (("attention.hip", bench.load_traffic), ("prologue.hip", bench.load_prologue_traffic)):
        src = tmp_path / "quantized_attention_prepare_amd/csrc" / f
        text = src.read_text()
        src.write_text(text + "\nstatic int changed_code;\n")
        assert loader("C3") is None, f
        src.write_text(text)
        assert loader("C3") is not None, f


def test_more_than_one_gpu_is_refused_before_any_device_call():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
