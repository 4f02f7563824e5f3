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
    prod = "void mlp::(anonymous namespace)::gemm_big_kernel<true, (mlp::Layout)2, (mlp::Epi)3>(mlp::GemmParams)"
    epi = "void mlp::(anonymous namespace)::splitk_epilogue_kernel<(mlp::Epi)3>(mlp::GemmParams)"
    fwd = "void mlp::(anonymous namespace)::gemm_big_kernel<true, (mlp::Layout)0, (mlp::Epi)1>(mlp::GemmParams)"
    other = "void at::native::vectorized_elementwise_kernel<4>"
    disp = [(other, 99.0)]
    for step in range(3):
        disp += [(fwd, 10.0 + step), (prod, 5.0), (epi, 2.0)]
    names, avg = bench._per_slot(disp, 2, 2)
    assert len(names) == 2
    assert "splitk_epilogue_kernel" in names[1] and "gemm_big_kernel" in names[1]
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


def test_source_digest_ignores_comments_only(tmp_path, monkeypatch):
    """Comment and blank-line edits keep the kernel-source digest (the code
    is the same); any code edit, a constant or an added file, changes it."""
    csrc = tmp_path / "mlp_gemm_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("int f() { return 1; }  // one\n")
    base = bench.source_digest()
    (csrc / "k.hip").write_text("/* a block\n comment */\nint f() { return 1; }  // two\n\n")
    assert bench.source_digest() == base
    (csrc / "k.hip").write_text("int f() { return 2; }  // one\n")
    assert bench.source_digest() != base
    (csrc / "k.hip").write_text("int f() { return 1; }  // one\n")
    (csrc / "g.hpp").write_text("#pragma once\n")
    assert bench.source_digest() != base


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
    # per-slot records: any slot of the profiled run, same sources only
    rec = {"w": {"kernel": "a", "source_sha": bench.source_digest(), "bytes_per_launch": 1,
                 "slots": {"a": {"bytes_per_launch": 1}, "b": {"bytes_per_launch": 2}}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("w", "b") == 2 and bench.recorded_traffic("w", "a") == 1
    assert bench.recorded_traffic("w", "c") is None
    (csrc / "k.hip").write_text("kernel changed again")
    assert bench.recorded_traffic("w", "b") is None


def _write_csv(path, header, rows):
    import csv
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_prices_counters_per_slot(tmp_path, monkeypatch):
    """The profile summary from synthetic rocprofv3 output: per-slot grouping
    (a split-K epilogue joins its product), copy-calibrated HBM bytes, and
    the matrix-core busy share and clock of the dominant slot."""
    root = tmp_path / "root"
    (root / "mlp_gemm_softmax_amd" / "csrc").mkdir(parents=True)
    (root / "mlp_gemm_softmax_amd" / "csrc" / "k.hip").write_text("kernel")
    monkeypatch.setattr(bench, "ROOT", str(root))
    out = tmp_path / "out"
    out.mkdir()
    w = "toy"
    ka = "void mlp::(anonymous namespace)::ka(mlp::GemmParams)"
    kb = "void mlp::(anonymous namespace)::kb(mlp::GemmParams)"
    fol = "void mlp::(anonymous namespace)::splitk_epilogue_kernel<(mlp::Epi)3>(mlp::GemmParams)"
    copy = "__amd_rocclr_copyBuffer"
    line = {"value": 1.0, "ms_per_step": 1.0, "achieved_tflops": 1.0, "config": {"precision": "f32"},
            "roofline": {"kernel": "slot_b", "achieved": 1.0, "unit": "TFLOP/s", "frac": 0.5, "peak": 157.3,
                         "bound": "mfma", "algorithmic_flops": 2e9, "algorithmic_bytes": 1e6}}
    (out / f"bench_{w}.log").write_text("[bench] per-launch (ms avg): slot_a=0.0100, slot_b=0.2000\n"
                                        + json.dumps(line) + "\n")
    # three steps in the trace: ka 10 us, kb 150 us + its split-K epilogue 50 us
    trace, t, d = [], 0, 0
    for _ in range(3):
        for name, us in ((ka, 10), (kb, 150), (fol, 50)):
            d += 1
            trace.append([d, name, t, t + us * 1000])
            t += us * 1000 + 500
    _write_csv(str(out / f"trace_{w}" / f"{w}_kernel_trace.csv"),
               ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    _write_csv(str(out / f"trace_{w}" / f"{w}_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "Percentage"],
               [[kb, 3, 150000, 70.0], [fol, 3, 50000, 20.0], [ka, 3, 10000, 10.0]])
    # counters: a 256 MiB copy counted as 131072 KiB fetched (scale 2) and 262144 KiB written (scale 1)
    for cname, d_, copy_kib in (("FETCH_SIZE", "fetch", 131072.0), ("WRITE_SIZE", "write", 262144.0)):
        rows, i = [[1, copy, cname, copy_kib]], 1
        for _ in range(2):
            for name, kib in ((ka, 10.0), (kb, 100.0), (fol, 20.0)):
                i += 1
                rows.append([i, name, cname, kib])
        _write_csv(str(out / f"{d_}_{w}" / f"{w}_counter_collection.csv"),
                   ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    # matrix cores: kb busy for 0.6 of 1024 SIMDs x 240000 cycles over 100 us (2.4 GHz)
    rows, i, t = [], 0, 0
    for _ in range(2):
        for name, busy, mops, grbm, us in ((ka, 0.0, 0.0, 8 * 24000.0, 10), (kb, 0.6 * 1024 * 240000, 2e9 / 512,
                                                                             8 * 200000.0, 100), (fol, 0.0, 0.0, 8 * 40000.0, 20)):
            i += 1
            for cname, v in (("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_INSTS_VALU_MFMA_MOPS_F32", mops),
                             ("GRBM_GUI_ACTIVE", grbm), ("SQ_BUSY_CU_CYCLES", 1.0)):
                rows.append([i, name, cname, v, t, t + us * 1000])
            t += us * 1000 + 1000
    _write_csv(str(out / f"mfma_{w}" / f"{w}_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"], rows)

    bench.summarize(str(out), w, 3, 1)
    rec = json.loads((root / "profiles" / "traffic.json").read_text())[w]
    assert rec["kernel"] == "slot_b" and rec["source_sha"] == bench.source_digest()
    assert rec["fetch_bytes"] == round((100 + 20) * 2.0 * 1024)
    assert rec["write_bytes"] == round((100 + 20) * 1.0 * 1024)
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # busy over the slot's cycles (product + epilogue: 240000 per XCD)
    assert rec["mfma_busy"] == pytest.approx(0.6, abs=1e-4)
    assert rec["clock_ghz"] == pytest.approx(240000 / 120e3, abs=1e-3)   # 120 us for the slot
    assert rec["slots"]["slot_b"]["bytes_per_launch"] == rec["bytes_per_launch"]
    assert set(rec["slots"]) == {"slot_a", "slot_b"}
    md = (root / "profiles" / f"{w}.md").read_text()
    assert "`kb + splitk_epilogue_kernel<(mlp::Epi)3>`" in md
    assert "| slot_b |" in md and "Matrix cores per launch slot" in md
