"""Host-side parts of bench.py (no GPU): the algorithmic work it divides by, the roofline's
choice of bound, the per-stage reporting, and the refusal of several GPUs."""
import importlib.util
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _inp(lens, H=128, d_n=128, d_c=512, d_R=64, d_v=128, mp=64):
    return dict(B=len(lens), H=H, d_n=d_n, d_c=d_c, d_R=d_R, d_v=d_v, max_pages=mp,
                seq_lens=torch.tensor(lens, dtype=torch.int32))


def test_headline_work_per_token(bench):
    # 278,528 FLOP and 1,152 cache bytes per KV token at the DeepSeek widths, at T = 1
    a = bench.algorithmic(_inp([4096] * 16))
    assert a["sumS"] == 65536
    assert a["attn_flops"] == 278528 * 65536
    assert a["attn_bytes"] == 1152 * 65536
    # plus the absorb and the up-projection, and the weights, queries, output and tables
    assert a["flops"] == a["attn_flops"] + 2 * 16 * 128 * 128 * 512 * 2
    assert a["bytes"] == (a["attn_bytes"] + 2 * 128 * 512 * 256 + 2 * 16 * 128 * 192
                          + 2 * 16 * 128 * 128 + 4 * (16 * 64 + 16))


def test_query_token_pairs(bench):
    # query token i of a sequence of S tokens attends to S - T + 1 + i of them
    a = bench.algorithmic(_inp([10, 3]), T=4)
    pairs = sum(max(0, s - 4 + 1 + i) for s in (10, 3) for i in range(4))
    assert pairs == (7 + 8 + 9 + 10) + (0 + 1 + 2 + 3)
    assert a["sumS"] == pairs
    assert a["attn_bytes"] == 13 * 1152  # the cache is read once


def test_bound_follows_the_ridge(bench):
    ridge = bench.RIDGE_FLOP_PER_BYTE
    assert 314 < ridge < 315  # 2516.6 TFLOP/s over 8 TB/s
    one = bench.algorithmic(_inp([4096] * 16), T=1)
    two = bench.algorithmic(_inp([4096] * 16), T=2)
    assert one["attn_flops"] / one["attn_bytes"] < ridge < two["attn_flops"] / two["attn_bytes"]


def test_decompressed_branch_arithmetic(bench):
    # decompression 2 S H (d_n + d_v) d_c, then 2 H (d_n + d_R + d_v) per (query, token) pair
    a = bench.algorithmic(_inp([300, 256]), T=256)
    pairs = sum(max(0, s - 256 + 1 + i) for s in (300, 256) for i in range(256))
    assert a["decomp_flops"] == 2 * 556 * 128 * 256 * 512 + 2 * 128 * 320 * pairs


def test_quantised_cache_bytes_per_token(bench):
    m2 = _inp([32768] * 32, H=32, d_n=120, d_c=64, d_R=8)
    assert bench.algorithmic(m2)["attn_bytes"] == 144 * 32768 * 32
    assert bench.algorithmic(m2, 1, 64 + 16 + 4)["attn_bytes"] == 84 * 32768 * 32  # FP8
    assert bench.algorithmic(m2, 1, 32 + 16 + 2)["attn_bytes"] == 50 * 32768 * 32  # MXFP4


def test_stage_reporting(bench):
    assert bench.stage_us([0.0056, 0.026, 0.0071], False) == {"absorb": 5.6, "attention": 26.0,
                                                             "combine": 7.1}
    assert bench.stage_us([0.001, 4.9, 0.002], True) == {"decompressed_branch": 4900.0}


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
