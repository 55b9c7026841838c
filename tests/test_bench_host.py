"""Host logic of bench.py (no GPU): the algorithmic work per stage against figures derived
independently from the workload shapes, the roofline classification, and the one-GPU
guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _ffn(wl, N, E_hit):
    alg = bench.algorithmic(wl, N, E_hit)
    return alg, alg["gate_up"]["flops"] + alg["down"]["flops"]


def test_ffn_flops_and_weight_bytes():
    # 6 H I N flops for the three projections; 3 H I b weight bytes per expert hit
    wl = synth.WORKLOADS["dsv3_prefill"]
    alg, flops = _ffn(wl, N=16384 * 8, E_hit=256)
    assert flops == pytest.approx(11.54e12, rel=1e-3)
    wbytes = 256 * 3 * 7168 * 2048 * 2
    assert wbytes == pytest.approx(22.55e9, rel=1e-3)
    assert alg["gate_up"]["bytes"] + alg["down"]["bytes"] > wbytes
    wl = synth.WORKLOADS["qwen3_30b_a3b"]
    alg, flops = _ffn(wl, N=4096 * 8, E_hit=128)
    assert flops == pytest.approx(309.2e9, rel=1e-3)


def test_combine_bytes():
    # yp rows in, the slot weights and rows, y out: 2.114 GB on the DSV3 prefill shape
    wl = synth.WORKLOADS["dsv3_prefill"]
    alg = bench.algorithmic(wl, N=16384 * 8, E_hit=256)
    assert alg["combine"]["bytes"] == pytest.approx(2.114e9, rel=1e-3)
    assert alg["combine"]["flops"] == 0


def test_fp8_bytes_are_one_byte_plus_scales():
    bf = synth.WORKLOADS["dsv3_decode"]
    f8 = synth.WORKLOADS["dsv3_decode_fp8"]
    N, E_hit = 1024, 250
    a16 = bench.algorithmic(bf, N, E_hit)["down"]["bytes"]
    a8 = bench.algorithmic(f8, N, E_hit)["down"]["bytes"]
    w16 = E_hit * bf.I * bf.H * 2
    w8 = E_hit * bf.I * bf.H * (1 + 1 / 32)
    assert a16 - a8 == pytest.approx((w16 - w8) + N * bf.I * (2 - (1 + 1 / 32)), rel=1e-9)


@pytest.mark.parametrize("name,stage,bound", [
    ("dsv3_prefill", "gate_up", "mfma"),   # N/E = 512 flops per weight byte > the ridge
    ("qwen3_30b_a3b", "gate_up", "hbm"),   # N/E = 256 < the ridge: weight streaming
    ("dsv3_decode", "down", "hbm"),
    ("dsv3_prefill", "combine", "hbm"),
    ("tiny_f32", "gate_up", "alu"),        # fp32 on the vector ALUs, 2 KiB of weights per expert
])
def test_roofline_bound(name, stage, bound):
    wl = synth.WORKLOADS[name]
    N = wl.T * wl.k
    alg = bench.algorithmic(wl, N, min(wl.E, N))
    r = bench.roofline_of(stage, alg, 1e-3, wl.dtype)
    assert r["bound"] == bound
    peak = bench.PEAK_HBM_GBS if bound == "hbm" else bench.PEAK_TFLOPS[wl.dtype]
    assert r["frac"] == pytest.approx(r["achieved"] / peak, rel=1e-3, abs=6e-5)  # 4 decimals


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_source_hash_ignores_comments_only(tmp_path):
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k(int* p) {\n  p[0] = 1;\n}\n")
    h0 = bench.kernel_source_hash(str(tmp_path))
    src.write_text("// a kernel\n__global__ void k(int* p) {  /* one store */\n\n  p[0] = 1;  // x\n}\n")
    assert bench.kernel_source_hash(str(tmp_path)) == h0
    src.write_text("__global__ void k(int* p) {\n  p[0] = 2;\n}\n")
    assert bench.kernel_source_hash(str(tmp_path)) != h0


def test_kernel_source_hash_of_named_files_ignores_the_others(tmp_path):
    (tmp_path / "a.hip").write_text("__global__ void a(int* p) { p[0] = 1; }\n")
    (tmp_path / "b.hip").write_text("__global__ void b(int* p) { p[0] = 1; }\n")
    h0 = bench.kernel_source_hash(str(tmp_path), ["a.hip"])
    (tmp_path / "b.hip").write_text("__global__ void b(int* p) { p[0] = 2; }\n")
    assert bench.kernel_source_hash(str(tmp_path), ["a.hip"]) == h0
    assert bench.kernel_source_hash(str(tmp_path)) != bench.kernel_source_hash(str(tmp_path), ["a.hip"])
    (tmp_path / "a.hip").write_text("__global__ void a(int* p) { p[0] = 3; }\n")
    assert bench.kernel_source_hash(str(tmp_path), ["a.hip"]) != h0
