"""Host logic of bench.py (CPU only): the algorithmic work it prices the
kernels against, the step floor, the kernel-name mapping, and the two
rocprofv3 summaries, fed synthetic counter files."""
import argparse
import csv
import json
import os

import pytest

import bench

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _args(**kw):
    a = dict(B=4, H=16, N=4096, D=128, dtype="fp32", causal=False)
    a.update(kw)
    return argparse.Namespace(**a)


@pytest.mark.parametrize("D", [32, 64, 128, 256])
def test_algorithmic_totals_are_the_methods(D):
    """The launches of one fused non-causal step add up to the method's own
    work: 12 B H N D^2 flops and 11 B H N D s bytes (Q, K, V, dO read;
    O, dQ, dK, dV written)."""
    BH, N, s = 64, 4096, 4
    launches = ["state_local", "forward", "bwd_q", "bwd_kv", "state_scan", "state_scan"]
    fl = sum(bench.algorithmic(k, BH, N, D, s, True)[0] for k in launches)
    by = sum(bench.algorithmic(k, BH, N, D, s, True)[1] for k in launches)
    assert fl == 12 * BH * N * D * D
    assert by == 11 * BH * N * D * s
    # unfused: dQ alone, the gradient record from a second reduction
    unf = ["state_local", "forward", "bwd_q", "grad_state_local", "bwd_kv"]
    assert sum(bench.algorithmic(k, BH, N, D, s, False)[0] for k in unf) == 12 * BH * N * D * D


def test_step_floor_matches_the_roofline_table():
    """B4 H16 N4096 D128: fp32 operands bind on the matrix peak (327.7 us),
    bf16 storage on the bf16 matrix path binds on HBM (92.3 us)."""
    assert bench.step_floor_us(4, 16, 4096, 128, 4, False) == pytest.approx(327.7, abs=0.1)
    assert bench.step_floor_us(4, 16, 4096, 128, 2, True) == pytest.approx(92.3, abs=0.1)
    assert bench.uses_bf16_mfma("bf16", 128, True) and not bench.uses_bf16_mfma("bf16", 256, 0)
    assert not bench.uses_bf16_mfma("fp16", 128, False)


@pytest.mark.parametrize("name,launch", [
    ("la::nc::k_reduce_nc<la::StF32, 128, false>", "state_local"),
    ("la::nc::k_reduce_nc<la::StF32, 128, true>", "grad_state_local"),
    ("la::bf::k_reduce_bf<128, true>", "grad_state_local"),
    ("la::nc::k_apply_nc<la::StF32, 128, 0>", "forward"),
    ("la::nc::k_apply_nc<la::StF16, 128, 2>", "bwd_kv"),
    ("la::nc::k_bwd_q_nc<la::StF32, 128, true>", "bwd_q"),
    ("la::cz::k_bwd_kv_causal<la::StF32, 128>", "bwd_kv"),
    ("la::k_state_scan", "state_scan"),
    ("la::stg::k_pad<la::StF32>", "stage"),
    ("la::dec::k_decode<la::StF32, 128>", "decode"),
])
def test_launch_names(name, launch):
    assert bench.launch_name(name) == launch


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value, t0, t1) in enumerate(rows):
            w.writerow({**{k: 0 for k in FIELDS}, "Dispatch_Id": i // 9 + 1,
                        "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1})


def test_traffic_summary_scales_by_the_copy_kernel(tmp_path, monkeypatch, capsys):
    """FETCH_SIZE counts 2x and WRITE_SIZE 1x on the copy kernel of known
    size; the library's launches are scaled by the same factors, and the
    result lands in the traffic file under the workload's key."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy_kib = bench.COPY_MIB * 1024
    k = "void la::nc::k_bwd_q_nc<la::StF32, 128, true>(float const*)"
    _write_counters(str(tmp_path / "f"), [("void neg_kernel(float*)", "FETCH_SIZE", copy_kib / 2, 0, 1),
                                          (k, "FETCH_SIZE", 1000.0, 0, 1)])
    _write_counters(str(tmp_path / "w"), [("void neg_kernel(float*)", "WRITE_SIZE", copy_kib, 0, 1),
                                          (k, "WRITE_SIZE", 500.0, 0, 1)])
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), _args())
    out = capsys.readouterr().out
    assert "| bwd_q | 1 |" in out
    doc = json.load(open(tmp_path / "traffic.json"))
    e = doc["entries"]["bwd_q B4 H16 N4096 D128 fp32 causal=0"]
    assert e["read_bytes"] == 2 * 1000 * 1024 and e["write_bytes"] == 500 * 1024
    assert doc["kernel_source_hash"] == bench.kernel_source_hash()


def test_counter_summary_ratios(tmp_path, capsys):
    """MOPS x 512 over the algorithmic flops, MFMA busy cycles over
    GRBM_GUI_ACTIVE / 8 x 1024 SIMDs, instructions per MFMA."""
    k = "void la::nc::k_apply_nc<la::StF32, 128, 0>(float const*)"
    BH, N, D = 64, 4096, 128
    flops = 2 * BH * N * D * D
    mfma = flops // 4096
    vals = {"SQ_INSTS_VALU_MFMA_MOPS_F32": flops / 512, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0,
            "SQ_INSTS_MFMA": mfma, "SQ_INSTS_VALU": 3 * mfma, "SQ_INSTS_LDS": mfma // 2,
            "SQ_INSTS_SALU": mfma // 4, "SQ_VALU_MFMA_BUSY_CYCLES": 64 * mfma,
            "GRBM_GUI_ACTIVE": 8 * 64 * mfma / 1024 * 2, "SQ_BUSY_CU_CYCLES": 1}
    _write_counters(str(tmp_path / "c"), [(k, c, v, 0, 100_000) for c, v in vals.items()])
    bench.counter_summary(str(tmp_path / "c"), _args())
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| forward")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[3] == "1.000"                 # matrix work = algorithmic
    assert cells[4] == "0.500"                 # busy half of the SIMD cycles
    assert cells[5] == "2.00" and cells[6] == "0.50" and cells[7] == "0.25"


def test_lds_summary_ratios(tmp_path, capsys):
    """Bank-conflict cycles over the useful LDS cycles, LDS busy over the
    cycles of one XCD times 256 compute units, wait cycles per LDS
    instruction in 4-cycle units."""
    k = "void la::nc::k_bwd_q_nc<la::StF32, 128, true>(float const*)"
    vals = {"SQ_LDS_BANK_CONFLICT": 100.0, "SQ_LDS_ADDR_CONFLICT": 7.0,
            "SQ_LDS_IDX_ACTIVE": 500.0, "SQ_INSTS_LDS": 50.0, "SQ_WAIT_INST_LDS": 25.0,
            "SQ_LDS_MEM_VIOLATIONS": 0.0, "SQ_BUSY_CU_CYCLES": 1.0,
            "GRBM_GUI_ACTIVE": 8 * 1000 / 256 * 4}
    _write_counters(str(tmp_path / "l"), [(k, c, v, 0, 100_000) for c, v in vals.items()])
    bench.lds_summary(str(tmp_path / "l"), _args())
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| bwd_q")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[3] == "0.250"                 # 100 / (500 - 100)
    assert cells[4] == "0.125"                 # 500 / (1000 / 256 * 4 * 256)
    assert cells[6] == "2.00" and cells[7] == "0"


def test_kernel_source_hash_ignores_comments(tmp_path, monkeypatch):
    """The traffic entries stay valid across comment edits of the kernel
    sources and become stale on a code edit."""
    src = tmp_path / "k.hpp"
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    src.write_text("// a\nint f(int x) { return x + 1; }  /* b */\n")
    h0 = bench.kernel_source_hash()
    src.write_text("// another comment\n/* a\n block */ int f(int x)  {\n return x + 1; }\n")
    assert bench.kernel_source_hash() == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0
