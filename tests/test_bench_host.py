"""Host logic of bench.py (no GPU): the one-GPU guard, launch labels, the
algorithmic bytes behind the roofline, the counter summaries that profiles/
is written from, and the source hash that retires stored counters."""

import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

GEMM = "void mx::grouped_gemm_kernel<{}>(mx::GemmArgs)"


def _name(kg, bf, acc=False, sw=None):
    args = ["true" if v else "false" for v in (kg, bf, acc)]
    if sw is not None:
        args.append("true" if sw else "false")
    return GEMM.format(", ".join(args))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_launch_labels():
    names = [_name(False, False, sw=False), _name(False, False, sw=False),
             _name(True, False, sw=False), _name(True, False, True, sw=False),
             "void mx::quant_rowcol_kernel(float*)", _name(False, True, sw=True),
             _name(False, True), _name(False, True), _name(True, True)]
    assert bench._labels(names) == [
        "forward_NT", "dgrad_NN", "wgrad_TN", "wgrad_accumulate_TN", "quant_rowcol_kernel",
        "forward_NT_swiglu_quantize", "forward_NT_bf16", "dgrad_NN_bf16", "wgrad_TN_bf16"]
    cyc = {"quant_rowcol_kernel": ["w1", "w2"]}
    q = "void mx::quant_rowcol_kernel(float*)"
    assert bench._labels([q, q, q], cyc) == ["w1", "w2", "w1"]


def test_algorithmic_bytes_of_the_bench_workload():
    """Codes plus 1/32 scale bytes per operand element, fp32 outputs once."""
    b = bench.algorithmic_bytes("moe8_h4096_f14336")
    t, k, n, g = 16384, 4096, 14336, 8
    sc = 33 / 32
    assert b["forward_NT"] == pytest.approx(t * k * sc + g * n * k * sc + 4 * t * n)
    assert b["dgrad_NN"] == pytest.approx(t * n * sc + g * n * k * sc + 4 * t * k)
    assert b["wgrad_TN"] == pytest.approx(t * n * sc + t * k * sc + 4 * g * n * k)
    # the accumulating wgrad reads and writes main_grad
    assert b["wgrad_accumulate_TN"] - b["wgrad_TN"] == pytest.approx(4 * g * n * k)
    # the row + column quantize reads bf16 and writes two MXFP8 copies
    assert b["quant_rowcol_kernel"] == pytest.approx(g * n * k * (2 + 2 * sc))


def _pmc_dir(tmp, sub, launches):
    """A p_counter_collection.csv as rocprofv3 --pmc writes it: one row per
    dispatch and counter.  launches: [(kernel name, dur_ns, {counter: value})]."""
    d = os.path.join(tmp, sub)
    os.makedirs(d)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        t0 = 1000
        for i, (name, dur, ctrs) in enumerate(launches):
            for c, v in ctrs.items():
                w.writerow([i + 1, name, c, v, t0, t0 + dur])
            t0 += dur + 10
    return d


def test_summarize_trace(tmp_path):
    """Per-label calls, mean / median / min / max and share from a
    --kernel-trace CSV: the M-grouped GEMM alternates forward and dgrad in
    dispatch order, and a kernel launched for several purposes takes the
    names it is given in turn."""
    d = os.path.join(str(tmp_path), "trace")
    os.makedirs(d)
    fw, kg = _name(False, False, sw=False), _name(True, False, sw=False)
    rc = "void mx::quant_rowcol_kernel(unsigned short const*, long)"
    launches = [(rc, 40000), (rc, 20000), (fw, 100000), (fw, 200000), (kg, 300000),
                (rc, 44000), (rc, 22000), (fw, 110000), (fw, 210000), (kg, 310000)]
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t0 = 5000
        for name, dur in launches:
            w.writerow(["KERNEL_DISPATCH", name, t0, t0 + dur])
            t0 += dur + 100
    md = bench.summarize_trace(d, "t", ["cmd"],
                               cycles={"quant_rowcol_kernel": ["quant_w1", "quant_w2"]})
    total = sum(dur for _, dur in launches) / 1e3
    assert f"| `wgrad_TN` | 2 | 305.0 | 310.0 | 300.0 | 310.0 | 0.610 | {100 * 610 / total:.1f} |" in md
    assert "| `dgrad_NN` | 2 | 205.0 |" in md and "| `forward_NT` | 2 | 105.0 |" in md
    assert "| `quant_w1` | 2 | 42.0 |" in md and "| `quant_w2` | 2 | 21.0 |" in md
    # rows by total time, longest first
    assert md.index("| `wgrad_TN`") < md.index("| `dgrad_NN`") < md.index("| `forward_NT`")


def test_summarize_mfma(tmp_path):
    fw, dg = _name(False, False, sw=False), _name(False, False, sw=False)
    # 100 us at 2 GHz: 200000 active cycles per XCD; MFMA busy half the
    # 1024 SIMDs' cycles; 1 TFLOP of F8 work
    ctr = {"GRBM_GUI_ACTIVE": 8 * 200000, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 200000 * 1024,
           "SQ_INSTS_VALU_MFMA_MOPS_F8": 1e12 / 512}
    d = _pmc_dir(str(tmp_path), "mfma", [(fw, 100000, ctr), (dg, 100000, ctr)])
    md = bench.summarize_mfma(d, "t", ["cmd"])
    assert "| forward_NT | 1 | 100 | 2.00 (range 2.00-2.00) | 50.0 % | 1.000 |" in md
    assert "| dgrad_NN | 1 |" in md


def test_summarize_cache(tmp_path):
    fw = _name(False, False, sw=False)
    hit = _pmc_dir(str(tmp_path), "hit", [(fw, 10, {"TCC_HIT_sum": 60, "TCC_MISS_sum": 40})])
    lvl = _pmc_dir(str(tmp_path), "lvl", [(fw, 10, {"TCC_EA0_RDREQ_sum": 1000,
                                                    "TCC_EA0_RDREQ_LEVEL_sum": 750000})])
    sq = _pmc_dir(str(tmp_path), "sq", [(fw, 10, {"SQ_WAIT_INST_ANY": 45,
                                                  "SQ_WAVE_CYCLES": 100})])
    ta = _pmc_dir(str(tmp_path), "ta", [(fw, 10, {"TA_BUSY_avr": 50, "GRBM_GUI_ACTIVE": 800})])
    md = bench.summarize_cache([hit, lvl, sq, ta], "t", ["cmd"])
    assert "| forward_NT | 60 % | 750 | 45 % | 50 % |" in md


def test_summarize_traffic_scales_by_the_copy_calibration(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    kib = bench.COPY_BYTES // 1024
    cal_f = _pmc_dir(str(tmp_path), "cf", [(copy, 10, {"FETCH_SIZE": kib / 2})])
    cal_w = _pmc_dir(str(tmp_path), "cw", [(copy, 10, {"WRITE_SIZE": kib})])
    fw = _name(False, False, sw=False)
    fetch = _pmc_dir(str(tmp_path), "f", [(fw, 1000, {"FETCH_SIZE": 1000})])
    write = _pmc_dir(str(tmp_path), "w", [(fw, 1000, {"WRITE_SIZE": 3000})])
    md = bench.summarize_traffic("moe8_h4096_f14336", cal_f, cal_w, fetch, write, "t", ["cmd"])
    # fetch counts half the copied bytes (factor 2), write all of them
    assert '"read_bytes": 2048000' in md and '"write_bytes": 3072000' in md
    assert f'"source_sha256": "{bench.gemm_source_hash()}"' in md


def test_source_hash_covers_included_headers():
    files = bench._source_files(bench.GEMM_SOURCE)
    assert files[0] == bench.GEMM_SOURCE
    assert "moe_expert_grouped_group_amd/csrc/mx_tile_quant.h" in files
    assert "moe_expert_grouped_group_amd/csrc/mx_convert.h" in files
    q = bench._source_files(bench.QUANTIZE_SOURCE)
    assert "moe_expert_grouped_group_amd/csrc/mx_tile_quant.h" in q


def test_stored_traffic_is_retired_when_the_gemm_source_changes(tmp_path):
    h = bench.gemm_source_hash()
    with open(tmp_path / "grouped_gemm_hbm_traffic_w.md", "w") as f:
        f.write('# t\n\n```json\n{"source_sha256": "%s", "hbm_bytes_per_launch": 123}\n```\n' % h)
    assert bench.stored_traffic("w", str(tmp_path)) == 123
    with open(tmp_path / "grouped_gemm_hbm_traffic_w.md", "w") as f:
        f.write('# t\n\n```json\n{"source_sha256": "%s", "hbm_bytes_per_launch": 123}\n```\n'
                % ("0" * 64))
    assert bench.stored_traffic("w", str(tmp_path)) is None
    assert bench.stored_traffic("missing", str(tmp_path)) is None
