"""Host logic of bench.py (no GPU): the algorithmic work model behind the
roofline figures, the counter summaries, the source hashes that decide
whether committed counters still apply, and the single-GPU scope."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from positive_random_feature_amd.workloads import WORKLOADS  # noqa: E402


def test_alg_work_by_hand():
    # bidirectional 4 x 8 x 4096, d = 64, m = 256, bf16, one projection for
    # all heads: per token 8md + 4m FLOPs; q, k, v read and out written (4d
    # bf16 elements); the fp32 projection read once
    flops, nbytes = bench.alg_work(WORKLOADS["bidir_bf16_4k"])
    tokens = 4 * 8 * 4096
    assert flops == tokens * (8 * 256 * 64 + 4 * 256)
    assert nbytes == tokens * 4 * 64 * 2 + 256 * 64 * 4
    # per-head projections (causal 2 x 8 x 8192): eight of them
    flops, nbytes = bench.alg_work(WORKLOADS["causal_bf16_8k"])
    tokens = 2 * 8 * 8192
    assert nbytes == tokens * 4 * 64 * 2 + 8 * 256 * 64 * 4
    # fp32 elements are four bytes
    _, nbytes = bench.alg_work(WORKLOADS["bidir_f32_tiny"])
    w = WORKLOADS["bidir_f32_tiny"]
    assert nbytes == w.tokens * 4 * w.d * 4 + (w.H if w.omega_per_head else 1) * w.m * w.d * 4


def _write_pass(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for kname, counter, value in rows:
            f.write(f'"{kname}",{counter},{value}\n')


def test_summarise_sq_per_wave(tmp_path, capsys):
    k = "void favor::kv_partial_kernel<bf16, 64, 2, false>(...)"
    other = "some_library_kernel"
    p1 = [(k, "SQ_WAVES", 8), (k, "SQ_WAVE_CYCLES", 800), (k, "SQ_ACTIVE_INST_VALU", 160), (other, "SQ_WAVES", 99)]
    p2 = [(k, "SQ_WAVES", 4), (k, "SQ_INSTS_VALU", 400), (k, "SQ_INSTS_MFMA", 40), (k, "SQ_INSTS_VALU_TRANS_F32", 12),
          (k, "SQ_INSTS_LDS", 20), (k, "SQ_INSTS_SALU", 8), (k, "SQ_WAIT_INST_LDS", 44), (k, "SQ_LDS_BANK_CONFLICT", 4)]
    # two dispatches of the kernel in the third pass: their counters add up
    p3 = [(k, "SQ_WAVES", 2), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 100), (k, "SQ_WAVES", 2), (k, "SQ_VALU_MFMA_BUSY_CYCLES", 60)]
    dirs = [str(tmp_path / f"pmc{i}") for i in (1, 2, 3)]
    for d, rows in zip(dirs, (p1, p2, p3)):
        _write_pass(d, rows)
    bench.summarise_sq(dirs)
    out = capsys.readouterr().out.strip().splitlines()
    assert len(out) == 3  # header, rule, one kernel (the other kernel is not ours)
    # VALU 400/4, MFMA 40/4, trans 12/4, LDS 20/4, SALU 8/4, VALU busy 160/8,
    # MFMA busy 160/4, LDS wait 44/4, wave life 800/8, conflicts 4/4
    assert out[2] == "| kv_partial_kernel | 100 | 10 | 3 | 5 | 2 | 20 | 40 | 11 | 100 | 1 |"


def test_kernel_source_hash():
    a = bench.kernel_source_hash("causal_tile")
    assert a == bench.kernel_source_hash("causal_tile")
    assert a != bench.kernel_source_hash("kv_partial")
    assert a != bench.kernel_source_hash()
    with pytest.raises(ValueError):
        bench.kernel_source_hash("no_such")


def test_strip_comments_ignores_comment_edits():
    code = "int a; // one\n/* two\nlines */ int b;\n"
    assert bench._strip_comments(code) == bench._strip_comments("int a; // other\n/* x */ int b;")


def test_traffic_for_unknown_stage():
    assert bench.traffic_for("bidir_bf16_4k:no_such") is None
    assert bench.traffic_for("no_such_workload:causal_tile") is None


def test_single_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
