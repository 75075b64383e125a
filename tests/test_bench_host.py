"""bench.py's host side: the algorithmic byte and flop counts behind the roofline figures
(the per-token-head formulas written out for three workloads), and the one-GPU limit."""
import os
import subprocess
import sys

import pytest

import bench
from workloads import config_lengths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_forward_counts_varlen():
    # T = 4096, H = 16, K = V = 128: q, k, v, o in bf16 (4 x 256 B) and g, beta in fp32
    # (8 B) per token-head, 1032 B, plus the 48 final states of 64 KiB; flops
    # 2 (3 K V + C (K + 2 V)) per v-head token and 2 * 2 C K per q/k-head token
    by, fl = bench.algorithmic_counts(config_lengths(2), 16, 16, 128, 128, False, False, True)
    assert by == 4096 * 16 * 1032 + 48 * 128 * 128 * 4
    assert fl == 4096 * 16 * (2 * (3 * 128 * 128 + 64 * (128 + 256)) + 4 * 64 * 128)
    assert round(by / 1e6, 2) == 70.78 and round(fl / 1e10, 3) == 1.181


def test_forward_counts_grouped_heads_with_initial_state():
    # HK = 4, HV = 16: q and k per q/k head; initial and final states read and written
    by, fl = bench.algorithmic_counts(config_lengths(3), 4, 16, 128, 128, False, True, True)
    T = 32768
    assert by == T * (2 * 4 * 128 * 2 + 2 * 16 * 128 * 2 + 2 * 16 * 4) + 2 * 8 * 16 * 128 * 128 * 4
    assert round(by / 1e6, 1) == 356.5
    assert fl == T * (4 * 2 * 2 * 64 * 128 + 16 * 2 * (3 * 128 * 128 + 64 * (128 + 256)))


def test_summary_counts():
    # no q or o; start, end and transition states; the state widened to [S | P]
    by, fl = bench.algorithmic_counts(config_lengths(5), 16, 16, 128, 128, True, True, True)
    T = 262144
    assert by == T * (16 * 128 * 2 + 16 * 128 * 2 + 2 * 16 * 4) + 32 * 16 * 4 * (128 * 128 * 2 + 128 * 128)
    assert round(by / 1e9, 3) == 2.282
    assert fl == T * (16 * 2 * 64 * 128 + 16 * 2 * (64 * 256 + 2 * 128 * 256))
    assert round(fl / 1e11, 2) == 7.56


def test_option_counts():
    lens = config_lengths(2)
    plain = bench.algorithmic_counts(lens, 16, 16, 128, 128, False, False, True)
    fused = bench.algorithmic_counts(lens, 16, 16, 128, 128, False, False, True, beta_bytes=2)
    assert plain[0] - fused[0] == 4096 * 16 * 2 and plain[1] == fused[1]
    gdp = bench.algorithmic_counts(lens, 16, 16, 128, 128, False, False, True, nh=2)
    # k, v and beta twice per token; flops of the chunked method over 2 T update rows
    assert gdp[0] - plain[0] == 4096 * 16 * (128 * 2 + 128 * 2 + 4) and gdp[1] == 2 * plain[1]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_backward_counts_varlen():
    # per token-head at H = 16, K = V = 128: q, k, v, dO in bf16 (4 x 256 B), g, beta (8 B)
    # read; dq, dk, dv in fp32 (3 x 512 B), dg, dbeta (8 B) written: 2576 B; plus per (sequence,
    # head) the final-state gradient read and the initial-state gradient written.  Flops: the
    # forward (180,224), the reverse chunk pass (114,688) and the intra pass (327,680)
    by, fl = bench.backward_counts(config_lengths(2), 16, 16, 128, 128, False)
    assert by == 4096 * 16 * 2576 + 48 * 2 * 128 * 128 * 4
    assert fl == 4096 * 16 * (180224 + 114688 + 327680)
