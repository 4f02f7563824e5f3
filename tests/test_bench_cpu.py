"""Host logic of bench.py (no GPU): the one-GPU guard, roofline pricing of
the dominant launch slot, per-slot grouping of profiler dispatches, and the
source digest that keys the recorded counter traffic."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _row(name, flops, nbytes, total_ms, launches):
    return {"name": name, "flops": flops, "bytes": nbytes, "total_ms": total_ms, "launches": launches}


def test_roofline_prices_the_slot_with_most_time_against_mfma():
    rows = [_row("small", 1e9, 1e6, 1.0, 10),
            _row("big", 137438953472.0, 268435456.0, 11.6, 10),   # 4096^3 f32, 1.16 ms per launch
            _row("idle", 5.0, 5.0, 0.0, 0)]
    r = bench.roofline(rows, "f32", 10)
    assert r["kernel"] == "big" and r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["peak"] == bench.PEAK["f32_mfma_tflops"]
    assert r["achieved"] == pytest.approx(137438953472.0 / 1.16e-3 / 1e12, rel=1e-3)
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert r["avg_us"] == pytest.approx(1160.0)
    assert r["traffic"] is None


def test_roofline_below_the_ridge_is_hbm_bound():
    # intensity 4 flop/B: below the f32 ridge (157.3 TFLOP/s / 8 TB/s = 19.7)
    rows = [_row("stream", 4.0 * 360e6, 360e6, 0.65, 10)]
    r = bench.roofline(rows, "f32", 10)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(360e6 / 65e-6 / 1e9, rel=1e-3)
    # the same slot in a bf16 session is priced against the bf16 ridge (314.6)
    rows = [_row("mid", 100.0 * 1e9, 1e9, 1.0, 10)]
    assert bench.roofline(rows, "f32", 10)["bound"] == "mfma"
    assert bench.roofline(rows, "bf16", 10)["bound"] == "hbm"


def test_per_slot_groups_split_k_epilogues_with_their_product():
    prod = "void mlp::(anonymous namespace)::gemm_bf16_big_kernel<(mlp::Layout)2, (mlp::Epi)3>(mlp::GemmParams)"
    epi = "void mlp::(anonymous namespace)::splitk_epilogue_kernel<(mlp::Epi)3>(mlp::GemmParams)"
    fwd = "void mlp::(anonymous namespace)::gemm_bf16_big_kernel<(mlp::Layout)0, (mlp::Epi)1>(mlp::GemmParams)"
    other = "void at::native::vectorized_elementwise_kernel<4>"
    disp = [(other, 99.0)]
    for step in range(3):
        disp += [(fwd, 10.0 + step), (prod, 5.0), (epi, 2.0)]
    names, avg = bench._per_slot(disp, 2, 2)
    assert len(names) == 2
    assert "splitk_epilogue_kernel" in names[1] and "gemm_bf16_big_kernel" in names[1]
    assert avg[0] == pytest.approx(11.5)      # the last two steps
    assert avg[1] == pytest.approx(7.0)       # product + its epilogue


def test_per_slot_rejects_a_changing_sequence():
    a = "void mlp::(anonymous namespace)::xent_wave<16>(mlp::XentParams)"
    b = "void mlp::(anonymous namespace)::cast_bf16_kernel(float const*)"
    with pytest.raises(SystemExit):
        bench._per_slot([(a, 1.0), (b, 1.0), (b, 1.0), (a, 1.0)], 2, 2)
    with pytest.raises(SystemExit):
        bench._per_slot([(a, 1.0)], 2, 2)


def test_source_digest_ignores_non_source_files(tmp_path, monkeypatch):
    csrc = tmp_path / "mlp_gemm_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel")
    (csrc / "h.hpp").write_text("header")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.source_digest()
    (csrc / "k.hip.o").write_bytes(b"\x7fELF")
    (csrc / "notes.txt").write_text("scratch")
    assert bench.source_digest() == d0
    (csrc / "k.hip").write_text("kernel changed")
    assert bench.source_digest() != d0


def test_recorded_traffic_needs_the_same_sources_and_kernel(tmp_path, monkeypatch):
    csrc = tmp_path / "mlp_gemm_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("kernel")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"w": {"kernel": "slot", "source_sha": bench.source_digest(), "bytes_per_launch": 123}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("w", "slot") == 123
    assert bench.recorded_traffic("w", "other_slot") is None
    assert bench.recorded_traffic("missing", "slot") is None
    (csrc / "k.hip").write_text("kernel changed")
    assert bench.recorded_traffic("w", "slot") is None
