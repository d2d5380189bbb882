"""Host-side logic of bench.py (no GPU): the algorithmic byte and flop counts against the
figures worked out by hand from the layouts, the counter post-processing on synthetic
rocprofv3 databases, and the one-GPU guard."""
from __future__ import annotations

import os
import sqlite3
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from speculative_decode_amd import synth  # noqa: E402


def test_verify_bytes_single_sequence():
    # 32 heads of a 128 x 128 fp32 state read and written (2 MiB each way), 2 pending and 4
    # draft rows of x, B, dt (bf16), C for the drafts, and 4 x 32 x 128 fp32 y
    w = synth.WORKLOADS["llama8b_single"]
    byt, fl = bench.verify_work(w, 1, 4, 2.0, 1.0)
    want = 2 * 2 ** 21 + 6 * (4096 + 1024 + 32) * 2 + 4 * 1024 * 2 + 4 * 4096 * 4
    assert byt == want and abs(byt - 4.33e6) < 0.01e6
    assert fl == 32 * 128 * 128 * (3 * 2 + 5 * 4)


def test_verify_bytes_batched_and_hybrid():
    w = synth.WORKLOADS["llama8b_batched"]
    byt, _ = bench.verify_work(w, 16, 8, 4.0, 1.0)
    assert abs(byt - 71.45e6) < 0.01e6          # 67.1 MB of state, 2.2 MB of tokens, 2.1 MB of y
    h = synth.WORKLOADS["hybrid_decode"]
    byt, _ = bench.verify_work(h, 32, 4, 1.773, 1.0)
    state = 32 * 32 * 256 * 128 * 4
    assert byt > 2 * state and byt - 2 * state < 5e6


def test_prefill_work_long_prompt():
    # 8192 tokens: x, B, C, dt in (101.2 MB), fp32 y out (134.2 MB), final state (2.1 MB);
    # flops per chunk-head: causal C B^T once per group, causal M X, C h_in and the state
    w = synth.WORKLOADS["llama8b_long_prefill"]
    pw = bench.prefill_work(w, 8192)
    byt, fl = pw["all"]
    assert byt == 8192 * (4096 + 2048 + 32) * 2 + 8192 * 4096 * 4 + 32 * 128 * 128 * 4
    per_chunk_head = 256 * 256 * 128 / 4 + 256 * 256 * 128 + 2 * 256 * 128 * 128 + 2 * 256 * 128 * 128
    assert fl == pytest.approx(32 * 32 * per_chunk_head)
    assert abs(fl - 27.92e9) < 0.01e9  # 106.5 kFLOP per token-head


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _db(path, rows):
    con = sqlite3.connect(path)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con.close()


def test_traffic_is_scaled_by_the_copy(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> > >"
    ver = "void mil::ssm_verify_kernel<unsigned short, 8>"
    mib = 256
    # counters in KiB per dispatch: the copy reads mib MiB but its fetch counter says a third
    other = "void at::native::vectorized_elementwise_kernel<4, at::native::bfloat16_copy_kernel_cuda>"
    _db(tmp_path / "f.db", [(copy, "FETCH_SIZE", mib * 1024 / 3), (ver, "FETCH_SIZE", 1000.0),
                            (ver, "FETCH_SIZE", 1200.0), (other, "FETCH_SIZE", 5.0), (other, "FETCH_SIZE", 5.0)])
    _db(tmp_path / "w.db", [(copy, "WRITE_SIZE", mib * 1024), (ver, "WRITE_SIZE", 500.0)])
    t = bench.traffic(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "wl", mib)
    assert t["_calibration"]["fetch_scale"] == pytest.approx(3.0)  # other elementwise kernels do not count
    assert t["_calibration"]["write_scale"] == pytest.approx(1.0)
    e = t["verify/wl"]
    assert e["fetch_bytes"] == pytest.approx(1100.0 * 1024 * 3)
    assert e["write_bytes"] == pytest.approx(500.0 * 1024)
    assert e["source_sha"] == bench.source_hash("verify")


def test_traffic_sums_the_kernels_of_a_family(tmp_path):
    # a projection launches its product and its reduction once each: their bytes add up
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, float, float, at::native::binary_internal::MulFunctor<float> > >"
    gemm = "void mil::(anonymous namespace)::project_gemm<64, true>(mil::ProjParams)"
    red = "mil::(anonymous namespace)::project_reduce(mil::ProjParams)"
    setup = "void mil::(anonymous namespace)::ssm_verify_kernel<unsigned short, 4>(mil::VerifyParams)"
    step = "void mil::(anonymous namespace)::ssm_verify_kernel<unsigned short, 8>(mil::VerifyParams)"
    _db(tmp_path / "f.db", [(copy, "FETCH_SIZE", 1024.0), (gemm, "FETCH_SIZE", 100.0), (gemm, "FETCH_SIZE", 300.0),
                            (red, "FETCH_SIZE", 10.0), (red, "FETCH_SIZE", 30.0),
                            (setup, "FETCH_SIZE", 7.0)] + [(step, "FETCH_SIZE", 50.0)] * 8)
    _db(tmp_path / "w.db", [(copy, "WRITE_SIZE", 1024.0), (gemm, "WRITE_SIZE", 4.0), (red, "WRITE_SIZE", 2.0),
                            (step, "WRITE_SIZE", 5.0)])
    t = bench.traffic(str(tmp_path / "f.db"), str(tmp_path / "w.db"), "wl", 1)
    assert t["project/wl"]["fetch_bytes"] == pytest.approx((200.0 + 20.0) * 1024)
    assert t["project/wl"]["write_bytes"] == pytest.approx((4.0 + 2.0) * 1024)
    # a kernel launched once while setting up, beside eight launches in the steps, counts zero times
    assert t["verify/wl"]["fetch_bytes"] == pytest.approx(50.0 * 1024)


def test_mfma_counters(tmp_path):
    k = "void mil::(anonymous namespace)::chunk_scan_mfma<128, 64>(mil::MParams)"
    _db(tmp_path / "m.db", [(k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0), (k, "MfmaUtil", 10.0),
                            (k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 3000.0), (k, "MfmaUtil", 20.0),
                            ("void at::native::vectorized_elementwise_kernel<4>", "MfmaUtil", 0.0)])
    t = bench.mfma_counters(str(tmp_path / "m.db"), "wl")
    assert set(t) == {"prefill_scan/wl"}
    assert t["prefill_scan/wl"]["issued_bf16_flops"] == pytest.approx(2000.0 * 512)
    assert t["prefill_scan/wl"]["mfma_busy_frac"] == pytest.approx(0.15)


def test_summarize_kernel_trace(tmp_path):
    con = sqlite3.connect(tmp_path / "t.db")
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", [("a", 1000), ("a", 3000), ("b", 500)])
    con.commit()
    con.close()
    lines = bench.summarize([str(tmp_path / "t.db")]).splitlines()
    assert lines[1].split()[:2] == ["2", "2.000"] and lines[1].endswith("a")
    assert lines[2].split()[:2] == ["1", "0.500"] and lines[2].endswith("b")


def test_source_hash_is_per_family():
    fams = {f: bench.source_hash(f) for f in bench.FAMILY_SOURCES}
    assert fams["prefill_state"] == fams["prefill_out"]      # one source file
    assert fams["verify"] != fams["prefill_scan"] != fams["project"]
    assert len(bench.source_hash()) == 16
    assert np.all([len(h) == 16 for h in fams.values()])
