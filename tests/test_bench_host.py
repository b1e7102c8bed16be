"""Host logic of bench.py (no GPU): the algorithmic-byte accounting the
roofline divides by, the reading of committed counter summaries (and its
guard against a changed kernel source), the phase summary of the debug
timestamps, and the refusal of more than one GPU."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_of_the_qwen3_layer():
    """Per (request, layer, head) unit at T = 2048, d = 128, bf16: K once
    (2048 rows of 256 bytes), the 16 window rows of the 4 query heads, the
    16 evicted slots as int32; moved rows x 256 bytes x (K, V) x (read,
    write); decode K and V over the tokens plus the queries."""
    R, H, Hq, d, b, n_max, w = 64, 8, 32, 128, 16, 128, 16
    moved, tokens = 957_000, 64 * 2033
    alg, flops = bench._alg_bytes(R, R, 1, H, Hq, d, b, n_max, w, moved, tokens)
    per_unit_k, per_unit_q, per_unit_e = 2048 * 256, 16 * 4 * 256, 16 * 4
    assert alg["score"] == R * H * (per_unit_k + per_unit_q + per_unit_e)
    assert per_unit_k == 524_288 and R * H * per_unit_k == 268_435_456
    assert alg["compact"] == moved * 256 * 2 * 2
    assert alg["score_compact"] == alg["score"] + alg["compact"]
    assert alg["decode"] == tokens * H * 256 * 2 + R * Hq * 256
    # window logits 2*Hq*w*T*d per request plus the in-block Gram 2*H*T*b*d
    assert flops["score"] == R * (2 * Hq * w * 2048 * d + 2 * H * n_max * b * b * d)


def test_algorithmic_bytes_past_the_cap():
    """n_src = 160 blocks compressed to N_max = 128: E = (160 - 128 + 1) * 16
    = 528 evicted slots per head, K read over all 2560 slots."""
    alg, _ = bench._alg_bytes(64, 64, 1, 8, 32, 128, 16, 160, 16, 0, 0, n_max_keep=128)
    T = 160 * 16
    assert alg["score"] == 64 * 8 * (T * 256 + 16 * 4 * 256 + 528 * 4)


def _profile(tmp_path, kernel_src_sha):
    text = ("# header\n"
            f"phase score_compact: fetch_bytes=1000 write_bytes=500 source_sha={kernel_src_sha} "
            "(raw ...)\n"
            f"phase score_compact: dram_read_bytes=900 dram_write_bytes=400 source_sha={kernel_src_sha}\n")
    (tmp_path / "hot_path_kernels_wl.txt").write_text(text)


def test_counters_are_read_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    sha = bench.source_sha(bench.KERNEL_SOURCES["score_compact"])
    _profile(tmp_path, sha)
    assert bench.read_counters("score_compact", "wl") == 1500
    assert bench.read_counters("score_compact", "wl", "dram") == 1300
    assert bench.read_counters("score_compact", "other_workload") is None
    _profile(tmp_path, "0" * 16)               # taken on another kernel source
    assert bench.read_counters("score_compact", "wl") is None
    assert bench.read_counters("score_compact", "wl", "dram") is None


def test_phase_summary_of_known_stamps():
    # two units on a 100 MHz clock (100 ticks = 1 us): phases 10, 20, 5, 40 us
    # and 12, 18, 6, 44 us, the second starting 3 us later
    t = np.array([[0, 1000, 3000, 3500, 7500],
                  [300, 1500, 3300, 3900, 8300]], dtype=np.int64)
    s = bench.phase_summary(t, 100_000)
    assert s["units"] == 2 and s["start_spread_us"] == 3.0 and s["span_us"] == 83.0
    assert s["pass1_us"]["mean"] == 11.0 and s["pass2_us"]["mean"] == 19.0
    assert s["select_us"]["max"] == 6.0 and s["compact_us"]["mean"] == 42.0
    assert bench.phase_summary(t, 0) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in (r.stdout + r.stderr)
