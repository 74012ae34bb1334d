"""The bench's algorithmic byte and FLOP formulas, checked against counts written out by hand for
the workloads (CPU), and the bench harness contract (N > 1 refused)."""
import os
import subprocess
import sys

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_scan_bytes_headline_layer():
    cfg = workloads.CONFIGS[1]
    tc = 8 * 2048 * 1536
    # x, delta, z read and y written in bf16 (8 B per token*channel); B and C bf16 per token and state;
    # A (1536 x 16 fp32) and the two per-channel fp32 vectors (Dskip, delta bias)
    by_hand = tc * 8 + 2 * 8 * 2048 * 16 * 2 + 1536 * 16 * 4 + 2 * 1536 * 4
    assert bench.scan_bytes(cfg) == by_hand == 202485760


def test_scan_bytes_long_sequence_has_no_gate_and_returns_the_state():
    cfg = workloads.CONFIGS[3]
    tc = 131072 * 2048
    # x, delta read and y written (6 B per token*channel), B, C, A, Dskip (delta given directly: no bias),
    # and the fp32 final state
    by_hand = tc * 6 + 2 * 131072 * 16 * 2 + 2048 * 16 * 4 + 2048 * 4 + 2048 * 16 * 4
    assert bench.scan_bytes(cfg) == by_hand


def test_ssd_flops_causal_triangle():
    cfg = workloads.CONFIGS[4]
    b, L, H, P, N, Q = 2, 8192, 64, 64, 128, 256
    chunks = L // Q
    cb = b * chunks * Q * Q * N                 # C B^T once per group (G = 1), lower triangle: 2 Q^2 N / 2
    diag = b * H * chunks * Q * Q * P           # (C B^T o L) X, lower triangle
    states = 2 * b * H * chunks * Q * N * P     # chunk states
    off = 2 * b * H * chunks * Q * N * P        # C H^T
    assert bench.ssd_flops(cfg) == cb + diag + states + off
    # 776 FLOP per token*channel: Q + 4N + Q N / (H P)
    assert abs(bench.ssd_flops(cfg) / (b * L * H * P) - (Q + 4 * N + Q * N / (H * P))) < 1e-9


def test_ssd_flops_of_the_64_token_blocks_the_kernel_runs():
    # the kernel passes the state every 64 tokens: its own algorithmic FLOPs are those of 64-token blocks,
    # 612 FLOP per token*channel (Q + 4N + Q N / (H P) with Q = 64), against 776 for 256-token chunks
    cfg = workloads.CONFIGS[4]
    b, L, H, P, N, Q = 2, 8192, 64, 64, 128, 64
    per_tc = Q + 4 * N + Q * N / (H * P)
    assert abs(bench.ssd_flops(cfg, bench.SSD_BLOCK) / (b * L * H * P) - per_tc) < 1e-9
    assert bench.ssd_flops(cfg, 64) < bench.ssd_flops(cfg)


def test_headline_is_the_largest_single_gpu_workload():
    # by token*channel work and by algorithmic bytes
    scans = [c for c in workloads.CONFIGS if c["kind"] == "scan"]
    big = max(range(len(workloads.CONFIGS)), key=lambda i: bench.scan_bytes(workloads.CONFIGS[i])
              if workloads.CONFIGS[i]["kind"] == "scan" else bench.ssd_bytes(workloads.CONFIGS[i]))
    assert big == bench.HEADLINE and workloads.CONFIGS[big] in scans


def test_valu_peak_from_unit_counts():
    # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz
    assert abs(bench.VALU_PEAK_TSLOTS - 39.3216) < 1e-9


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0 and "one GPU" in r.stderr
