"""Host-side measurement logic of bench.py (no GPU): the algorithmic bytes it
assigns to each kernel the library's timing can report for the attention
workloads, the step roofline of the headline workload against figures
derived by hand from the workload's shape, the traffic field's lookup in the
committed counter summaries (dropped once a kernel source changes), and the
refusal of more than one GPU."""
import os
import re

import pytest

import bench
import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_transformers_amd", "csrc")
ATTN_SOURCES = ("la_generic.hip", "la_mfma_fwd.hip", "la_mfma_bwd.hip", "la_mfma_bwd_cos.hip")


def _timed_names():
    """Every kernel name the attention sources give their timed launches."""
    names = set()
    for f in ATTN_SOURCES:
        text = open(os.path.join(CSRC, f)).read()
        for call in re.findall(r"TimedLaunch tl\(([^;]*)\)", text):
            names.update(re.findall(r'"(k_\w+)"', call))
    return names


def test_every_attention_kernel_has_its_bytes():
    names = _timed_names()
    assert {"k_fwd_mfma", "k_fwd_split_mfma", "k_bwd_q_mfma", "k_bwd_kv_mfma",
            "k_bwd_q_cos_mfma", "k_bwd_kv_cos_mfma", "k_state_mfma"} <= names
    w = si.WORKLOADS["causal_gqa_cos_b1h32kv8n65536d128"]
    for n in names:
        got = bench.kernel_bytes(n, w, 2)
        if n.startswith("k_scan_"):
            assert got is None, n   # state records only: not the method's bytes
        else:
            assert got is not None and got > 0, n


def test_kernel_bytes_by_hand():
    # B=2, H=H_kv=32, N=16384, D=128, bf16: one q-sized tensor is 2^28 bytes
    w = si.WORKLOADS[si.HEADLINE]
    t, rows = 2 ** 28, 2 * 32 * 16384 * 4
    assert bench.kernel_bytes("k_state_mfma", w, 2) == 2 * t              # k, v
    assert bench.kernel_bytes("k_fwd_mfma", w, 2) == 4 * t                # q, k, v -> out
    assert bench.kernel_bytes("k_bwd_q_mfma", w, 2) == 5 * t + 2 * rows   # q, k, v, g -> dq; den, c
    assert bench.kernel_bytes("k_bwd_kv_mfma", w, 2) == 6 * t + 2 * rows  # q, g, k, v -> dk, dv
    # the split forward computes the same part of the method as k_fwd_mfma
    w5 = si.WORKLOADS["causal_gqa_cos_b1h32kv8n65536d128"]
    assert bench.kernel_bytes("k_fwd_split_mfma", w5, 2) == bench.kernel_bytes("k_fwd_mfma", w5, 2)


def test_headline_step_roofline():
    # fwd reads q, k, v and writes out (4 tensors), bwd reads q, k, v, g and
    # writes dq, dk, dv (7): 11 tensors of 2^28 bytes; flops 2 D^2 per token
    # for each of the four state products (fwd: update, read; bwd: 3 + 3 at
    # H = H_kv) -> 2 * 128^2 * 32768 * (2*32 + 6*32)
    w = si.WORKLOADS[si.HEADLINE]
    t_roof, nbytes, flops = bench.step_roofline(w, 2, True)
    assert nbytes == 11 * 2 ** 28
    assert flops == 2 * 128 * 128 * 32768 * (2 * 32 + 6 * 32)
    assert t_roof == pytest.approx(11 * 2 ** 28 / 8.0e12)   # HBM-bound: 0.369 ms
    assert t_roof * 1e3 == pytest.approx(0.369, abs=1e-3)


# --------------------------------------------------------------------------
# traffic field: read from the committed counter summaries, and dropped as
# soon as a kernel source differs from the one the counters were taken on
# --------------------------------------------------------------------------
LOWRANK = "lowrank_m32768_in4096_r1024_out4096"


def _copy_tree(tmp_path):
    import shutil
    shutil.copytree(os.path.join(ROOT, "profiles"), str(tmp_path / "profiles"))
    shutil.copytree(CSRC, str(tmp_path / "linear_attention_transformers_amd" / "csrc"))
    return tmp_path


def test_traffic_from_committed_summary():
    t = bench.measured_traffic(LOWRANK, "k_lowrank_gemm_xVt")
    if t is None:
        pytest.skip("the low-rank counter summary predates the current la_lowrank.hip")
    # x V^T moves at least its algorithmic bytes: x and V read, t written
    M, n_in, rank = 32768, 4096, 1024
    algorithmic = 2 * (M * n_in + rank * n_in + M * rank)
    assert algorithmic <= t <= 3 * algorithmic


def test_traffic_dropped_when_a_source_changes(tmp_path, monkeypatch):
    root = _copy_tree(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(root))
    before = bench.measured_traffic(LOWRANK, "k_lowrank_gemm_xVt")
    src = root / "linear_attention_transformers_amd" / "csrc" / "la_lowrank.hip"
    src.write_text(src.read_text() + "\n// edited\n")
    assert bench.measured_traffic(LOWRANK, "k_lowrank_gemm_xVt") is None
    if before is None:
        pytest.skip("the committed summary was already stale")


def test_traffic_none_without_summary_or_kernel():
    assert bench.measured_traffic("no_such_workload", "k_lowrank_gemm_xVt") is None
    assert bench.measured_traffic(LOWRANK, "k_no_such_kernel") is None


def test_more_than_one_gpu_refused():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr or "1 GPU" in r.stderr, r.stderr[-400:]
