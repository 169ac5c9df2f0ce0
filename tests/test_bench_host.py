"""Host logic of bench.py: kernel-name shortening, stage attribution and the
rocprofv3 counter summary (on synthetic counter files)."""
import csv
import os

import pytest

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size", "Kernel_Id",
        "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
        "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
GATE_UP = ("void moe::(anonymous namespace)::gemm_bf16_dma_kernel<true, false, false, false, 8, 5, true>"
           "(unsigned short const*, unsigned short const*, int, long)")
DOWN = "void moe::(anonymous namespace)::gemm_bf16_dma_kernel<false, false, false, false, 8, 5, true>(int)"
SCORES = "void moe::(anonymous namespace)::gemm_bf16_dma_kernel<false, false, true, false, 8, 4, true>(int)"
COPY = ("void at::native::vectorized_elementwise_kernel<16, at::native::bitwise_not_kernel_cuda(at::TensorIteratorBase&)"
        "::{lambda(unsigned char)#1}, std::array<char*, 2ul> >(int, at::native::bitwise_not_kernel_cuda(at::TensorIteratorBase&)"
        "::{lambda(unsigned char)#1}, std::array<char*, 2ul>)")


def test_short_names_and_stages():
    assert bench.short_kernel_name(GATE_UP) == "gemm_bf16_dma_kernel<true, false, false, false, 8, 5, true>"
    assert bench.stage_of_kernel(bench.short_kernel_name(GATE_UP)) == "gate_up"
    assert bench.stage_of_kernel(bench.short_kernel_name(DOWN)) == "down"
    assert bench.stage_of_kernel(bench.short_kernel_name(SCORES)) == "router"
    assert bench.stage_of_kernel("gemm_bf16_skinny_kernel<true>") == "gate_up"
    assert bench.stage_of_kernel("gemm_bf16_skinny_kernel<false>") == "down"
    assert bench.stage_of_kernel("scatter_rows_kernel<4>") == "scatter"
    assert bench.stage_of_kernel("slot_scatter_kernel<2>") == "scatter"
    assert bench.stage_of_kernel("combine_kernel<true, 4>") == "combine"
    assert bench.stage_of_kernel("scan_kernel") == "slots"
    assert bench.stage_of_kernel("slots_from_ranks_kernel") == "slots"
    assert bench.stage_of_kernel("route_kernel<16, 8, true, false>") == "route"
    assert bench.stage_of_kernel(bench.short_kernel_name(COPY)) is None
    assert "bitwise_not" in bench.short_kernel_name(COPY)


def _write_pass(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({c: 0 for c in COLS} | {"Dispatch_Id": i // 8, "Correlation_Id": i // 8, "Kernel_Name": kernel,
                                                "Counter_Name": counter, "Counter_Value": value})


def test_counter_summary_scales_by_the_copy_kernel(tmp_path):
    wl = "deepseek_v3_prefill"
    root = tmp_path / "pmc"
    # the copy reads 1 GiB and writes 1 GiB; FETCH_SIZE counts half of it
    _write_pass(root / wl / "fetch", [(COPY, "FETCH_SIZE", 512 * 1024), (GATE_UP, "FETCH_SIZE", 1000.0),
                                      (DOWN, "FETCH_SIZE", 10.0)])
    _write_pass(root / wl / "write", [(COPY, "WRITE_SIZE", 1024 * 1024), (GATE_UP, "WRITE_SIZE", 24.0),
                                      (DOWN, "WRITE_SIZE", 6.0)])
    mf = [(GATE_UP, c, v) for c, v in (("MfmaUtil", 40.0), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0), ("SQ_WAVE_CYCLES", 10.0),
                                       ("SQ_WAIT_INST_ANY", 5.0), ("SQ_LDS_BANK_CONFLICT", 1.0),
                                       ("SQ_ACTIVE_INST_LDS", 50.0))]
    _write_pass(root / wl / "mfma", mf)
    _write_pass(root / wl / "l2", [(GATE_UP, "TCC_HIT_sum", 3.0), (GATE_UP, "TCC_MISS_sum", 1.0)])
    txt = bench.counters_summary(str(root), wl)
    assert "FETCH_SIZE factor 2.00000" in txt and "WRITE_SIZE factor 1.00000" in txt
    line = next(l for l in txt.splitlines() if l.startswith("gemm_bf16_dma_kernel<true"))
    assert "gate_up" in line and "2.0726e+06" in line and "1.0240e+03" in line and "0.750" in line and "0.500" in line
    assert line.split()[-2] == "nan"      # no GRBM_GUI_ACTIVE in this synthetic pass
    # gate/up: (1000 x 2 + 24) KiB
    assert f"gate_up_hbm_bytes_per_launch: {2024 * 1024:.6e}" in txt
    assert f"gate_up_sources_sha256: {bench.sources_sha('gate_up')}" in txt


def test_traffic_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = bench.counters_file("mixtral_prefill")
    with open(path, "w") as f:
        f.write(f"gate_up_hbm_bytes_per_launch: 1.5e+09\ngate_up_sources_sha256: {bench.sources_sha('gate_up')}\n")
    assert bench.read_traffic("mixtral_prefill", "gate_up") == pytest.approx(1.5e9)
    with open(path, "w") as f:
        f.write("gate_up_hbm_bytes_per_launch: 1.5e+09\ngate_up_sources_sha256: 00ff\n")
    assert bench.read_traffic("mixtral_prefill", "gate_up") is None
    assert bench.read_traffic("tiny_f32", "gate_up") is None
