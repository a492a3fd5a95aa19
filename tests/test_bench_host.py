"""Host logic of bench.py, on the CPU: the algorithmic byte counts the
roofline divides by (pinned to the per-configuration figures worked out from
the definitions of the two operations: the norm-quant reads 2 (Nq + Nkv)
bytes per row plus both gammas once and writes Nq code bytes, 4 bytes per
128-group and 2 Nkv kv bytes; the GEMM moves the weight, its 128x128 block
scales, the activation pair and the bf16 output once), the parity summary
it prints, the committed counter lookup, and the one-GPU refusal."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("M,want", [(1, 10_800), (16, 111_360), (64, 433_152), (256, 1_720_320),
                                    (8192, 54_923_264)])
def test_normquant_bytes(M, want):
    # 6704 bytes per row (3072 + 1024 read, 1536 + 48 + 1024 written) + 4096 of gammas
    assert bench.algorithmic_bytes_normquant(M) == want == 6704 * M + 4096


@pytest.mark.parametrize("M,N,want", [(1, 24576, 37_808_688), (16, 24576, 38_569_728), (64, 24576, 41_005_056),
                                      (256, 24576, 50_746_368), (1, 8192, 12_603_952), (16, 8192, 12_873_472),
                                      (64, 8192, 13_735_936), (256, 8192, 17_185_792)])
def test_gemm_bytes(M, N, want):
    assert bench.algorithmic_bytes_gemm(M, N, 1536) == want


@pytest.mark.parametrize("M", [1, 16, 64, 256])
def test_pair_bytes_share_the_activation_once(M):
    a = bench.algorithmic_bytes_gemm(M, 24576, 1536)
    b = bench.algorithmic_bytes_gemm(M, 8192, 1536)
    activation = M * 1536 + 4 * M * 12
    assert bench.algorithmic_bytes_gemm_pair(M, 24576, 8192, 1536) == a + b - activation


def test_gemm_flops():
    assert bench.gemm_flops(256, 24576, 1536) == 2 * 256 * 24576 * 1536


def test_sign_magnitude_order():
    # e4m3: +0, -0, the smallest subnormals of each sign, 448 and -448
    codes = np.array([0x00, 0x80, 0x01, 0x81, 0x7E, 0xFE], np.uint8)
    assert bench.sign_magnitude_ord(codes, np, 0x80).tolist() == [0, 0, 1, -1, 126, -126]
    # bf16: 1.0 (0x3F80) and its neighbours
    bits = np.array([0x3F7F, 0x3F80, 0x3F81, 0xBF80], np.uint16)
    assert bench.sign_magnitude_ord(bits, np, 0x8000).tolist() == [0x3F7F, 0x3F80, 0x3F81, -0x3F80]


def test_parity_stats_reports_planted_differences():
    r = np.random.default_rng(3)
    q = r.integers(0, 0x7E, size=(4, 1536), dtype=np.uint8)
    s = (r.random(48) + 0.5).astype(np.float32)
    kv = r.integers(0x3000, 0x4000, size=(4, 512), dtype=np.uint16)
    o1 = r.standard_normal((4, 256))
    o2 = r.standard_normal((4, 128))
    ref = (q, s, kv, o1, o2)
    same = bench.parity_stats(np, ref, ref)
    assert same["q_codes_exact"] == 1.0 and same["q_codes_max_ulp"] == 0 and same["kv_max_ulp"] == 0
    assert same["scale_max_rel"] == 0.0 and same["gemm_W_a_rel_fro"] == 0.0 and same["gemm_W_b_rel_max"] == 0.0
    q2, kv2, s2 = q.copy(), kv.copy(), s.copy()
    q2[0, 0] += 1                 # one code one step up
    kv2[1, 2] += 2                # one kv value two bf16 steps up
    s2[5] = np.nextafter(s[5], np.float32(np.inf))  # one fp32 step up
    got = bench.parity_stats(np, (q2, s2, kv2, o1 * (1 + 1e-3), o2), ref)
    assert got["q_codes_max_ulp"] == 1 and got["q_codes_exact"] == pytest.approx(1 - 1 / q.size)
    assert got["kv_max_ulp"] == 2 and got["kv_exact"] == pytest.approx(1 - 1 / kv.size)
    assert got["scale_max_rel"] == float(s2[5]) / float(s[5]) - 1.0
    assert got["gemm_W_a_rel_fro"] == pytest.approx(1e-3, rel=1e-2)
    assert got["gemm_W_a_rel_max"] == pytest.approx(1e-3, rel=1e-2)
    assert got["gemm_W_b_rel_fro"] == 0.0


def test_committed_traffic_is_keyed_by_source_and_batch():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    e = t["block_scaled_fp8_gemm_pair"]
    assert bench.measured_traffic("block_scaled_fp8_gemm_pair", e["source_sha"], e["M"]) == e["bytes_per_launch"]
    assert bench.measured_traffic("block_scaled_fp8_gemm_pair", "0" * 16, e["M"]) is None
    assert bench.measured_traffic("block_scaled_fp8_gemm_pair", e["source_sha"], e["M"] + 1) is None
    # the figures read every byte the kernel must move, and not far more
    assert 1.0 <= e["bytes_per_launch"] / bench.algorithmic_bytes_gemm_pair(e["M"], 24576, 8192, 1536) < 1.2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
