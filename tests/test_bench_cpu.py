"""Host-side checks of bench.py: the one-GPU guard and the FLOP / byte counts behind its roofline
figures, against closed forms. No GPU is needed."""

import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from io_aware_exact_23_amd import configs, inputs  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("flags", [["--steps", "0"], ["--warmup", "-1"]])
def test_step_counts_are_checked(flags):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *flags],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--steps must be >= 1" in r.stderr and r.stdout == ""


def test_counted_flops_of_the_workloads():
    # 4*B*H*Nq*Nk*d, halved when causal.
    assert configs.LONG_CAUSAL_16K.counted_flops() == 2 * 16 * 16384 * 16384 * 128 * 2
    assert configs.GPT2_SMALL_CAUSAL.counted_flops() == 12_884_901_888
    assert configs.SINGLE_HEAD_FP32.counted_flops() == 4 * 128 * 128 * 64


@pytest.mark.parametrize("N", [1, 5, 64, 1000])
def test_allowed_pairs_causal_closed_form(N):
    w = configs.Workload("t", "bf16", 3, 2, N, N, 64, True, 1.0, None, 0)
    assert bench.allowed_scores(w, None) == 3 * 2 * N * (N + 1) // 2


def test_allowed_pairs_with_lengths():
    # Non-causal: Nq * L_b per (b, h). Causal: query i sees min(L_b, i + 1) keys. Lengths outside
    # [0, Nk] are clamped as the library clamps them.
    w = configs.Workload("t", "bf16", 3, 2, 7, 9, 64, False, 1.0, None, 0)
    assert bench.allowed_scores(w, [9, 4, 0]) == 2 * 7 * (9 + 4 + 0)
    assert bench.allowed_scores(w, [12, -3, 1]) == 2 * 7 * (9 + 0 + 1)
    wc = configs.Workload("t", "bf16", 2, 1, 6, 6, 64, True, 1.0, None, 0)
    brute = sum(min(L, i + 1) for L in (6, 2) for i in range(6))
    assert bench.allowed_scores(wc, [6, 2]) == brute


def test_decode_algorithmic_bytes_of_the_workload():
    # K and V rows of the valid keys (2 * d * 2 bytes each) plus Q, O (bf16) and lse per (b, h).
    w = configs.DECODE_SPLIT_KV
    lens = inputs.lengths(w.B, w.lengths[0], w.lengths[1], w.seed + 3).numpy()
    assert bench.decode_bytes(w, lens) == w.H * (512 * int(lens.sum()) + 516 * w.B)
    assert bench.decode_bytes(w, lens) == 4_973_060_096


def test_standard_bytes_small_case():
    # S written in full (fp32), read where allowed, P written and read over rows padded to 128.
    w = configs.Workload("t", "bf16", 1, 1, 4, 4, 64, True, 1.0, None, 0)
    qo = 2 * 4 * 64 * 2 + 4 * 4
    kv = 2 * 4 * 64 * 2
    expect = qo + kv + 4 * 4 * 4 + 10 * 4 + 2 * 4 * 128 * 2
    assert bench.standard_bytes(w, None) == expect


def test_counter_traffic_is_used_only_for_the_sources_it_was_taken_on(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k__w__hbm_counters.txt").write_text(
        '# header\nRESULT {"source_sha": "abc", "hbm_bytes_per_launch": 1234}\n')
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k", "w", "abc") == 1234
    assert bench.traffic_from_profile("k", "w", "def") is None
    assert bench.traffic_from_profile("k", "other", "abc") is None

