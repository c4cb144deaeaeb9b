"""Host logic of the benchmark (no GPU): the one-GPU guard, the decoding of
kernel-kind codes into the names the profiler reports, and the synthetic
attention inputs' shapes and value ranges."""

import os
import subprocess
import sys

import numpy as np

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kind_names_and_symbols():
    # 10000*(10*mi + ni) + 1000 + 100*epilogue + 10*loader_A + loader_B
    assert bench.kind_symbol(220000 + 1000 + 100 * 1 + 0) == "gemm_i8_kernel<0, 0, 2, 2, false, false, 0, 0>"
    assert bench.kind_symbol(bench.ROW_KIND + 220000 + 1000 + 100 * 1 + 0) == "gemm_i8_kernel<0, 0, 2, 2, false, false, 1, 0>"
    assert bench.kind_symbol(110000 + 1000 + 100 * 2 + 10 * 1 + 4) == "gemm_i8_kernel<1, 4, 1, 1, true, false, 0, 0>"
    one_row = bench.ROW_KIND + bench.ONE_KIND + 220000 + 1000 + 100 * 8
    assert bench.is_one(one_row) and bench.is_row(one_row)
    assert bench.kind_symbol(one_row) == "gemm_max_kernel<0, 0, 2, 2, true, 1>"
    assert bench.kind_symbol(bench.ONE_KIND + 220000 + 1000 + 100 * 9) == "gemm_i8_kernel<0, 0, 2, 2, false, true, 0, 1>"
    assert bench.kind_symbol(220000 + 1000 + 100 * 0) == "gemm_i8_kernel<0, 0, 2, 2, false, false, 0, 1>"
    assert bench.kind_name(one_row) == bench.kind_name(one_row - bench.ROW_KIND) + "_rows"
    assert bench.kind_symbol(140000 + 1000 + 100 * 6) == "gemm_batched_kernel<0, 0, 1, 4, true>"
    assert bench.kind_symbol(210000 + 1000 + 100 * 4 + 1) == "gemm_batched_kernel<0, 1, 2, 1, false>"
    assert bench.kind_name(210000 + 1000 + 100 * 4 + 11) == "gemm_T_T_bmm_direct_128x64"
    pair = 1000000 * 11 + 10000 * 21 + 1000 + 300 + 10 * 3 + 5
    assert bench.is_pair(pair) and bench.kind_symbol(pair) == "gemm_pair_kernel<3, 5, 2, 1, 1, 4, 1, 1>"
    assert bench.kind_symbol(3210) == "pad_rows_z_kernel" and bench.kind_name(3000) == "rto_finalize"
    assert not bench.is_gemm(3400) and not bench.is_gemm(2001)


def test_roofline_bound_follows_arithmetic_intensity():
    # 5.0 POP/s over 8 TB/s: the roofs meet at 625 ops per byte
    assert bench.RIDGE_OPS_PER_BYTE == 625.0
    # 128x128x128 product at 1000 ops/byte, 1 ms: MFMA roof
    r = bench.roofline(1e12, 1e9, 1.0)
    assert r["bound"] == "mfma" and r["unit"] == "TOPS" and r["achieved"] == 1000.0 and r["frac"] == 0.2
    # a contraction of 64 (attention scores, ~80 ops/byte): HBM roof, bytes / time
    r = bench.roofline(8e10, 1e9, 0.5)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["achieved"] == 2000.0 and r["frac"] == 0.25
    # exactly at the ridge: MFMA; no ops (a pointwise pass): HBM
    assert bench.roofline(625e9, 1e9, 1.0)["bound"] == "mfma"
    assert bench.roofline(0.0, 4e9, 1.0)["achieved"] == 4000.0


def test_attention_inputs():
    a = wl.vit_attention_inputs(2, 3, 197, 64, seed=1)
    assert a.z == 6 and a.Q.mant.shape == (6 * 197, 64) and a.P.mant.shape == (6 * 197, 197)
    for c in (a.Q, a.K, a.V, a.dO, a.P, a.dS):
        assert c.group == wl.ROW and c.exp.shape == (c.mant.shape[0],)
        assert np.abs(c.mant.astype(int)).max() == 127  # the max-127 rule per row
    assert a.P.mant.min() >= 0  # probabilities
    b = wl.vit_attention_inputs(2, 3, 197, 64, seed=1, slices=2)
    assert b.z == 2 and b.P.mant.shape == (2 * 197, 197)
