"""Host logic of bench.py (CPU only): the algorithmic byte count the roofline
divides by, the digest check that keeps stale counter summaries out of the
bench line, and the summaries written from rocprofv3 CSV output."""
import argparse
import os

import numpy as np

import bench
from workloads import synth as I


def _tiny(temperature=1.0, top_k=0, bf16=False):
    rng = np.random.default_rng(5)
    t = rng.normal(0, 1, (2, 4, 10)).astype(np.float32)
    d = rng.normal(0, 1, (2, 3, 10)).astype(np.float32)
    tok = np.zeros((2, 3), np.int32)
    if bf16:
        t, d = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    return I.from_arrays(t, d, tok, temperature=temperature, top_k=top_k)


def test_algorithmic_bytes_by_hand():
    # B = 2, gamma = 3, V = 10, fp32; sequence 0 rejected at 0, sequence 1 all kept
    n = np.array([0, 3], np.int32)
    io = 4 * 2 * 3 + 4 * 2 * 4 + 4 * 2
    ab = bench.algorithmic_bytes(_tiny(), n)
    # statistics: pairs 0..n_b capped at gamma: 1 + 3 pairs of 2 V b = 80 bytes
    assert ab["stats"] == 4 * 80
    # resample: the rejected pair again (80) and the bonus row (40)
    assert ab["sample"] == 80 + 40
    assert ab["io"] == io and ab["total"] == 4 * 80 + 120 + io
    # top-k draws from the kept lists: only the bonus row is read again
    assert bench.algorithmic_bytes(_tiny(top_k=5), n)["sample"] == 40
    # arg-max mode: target rows 0..n_b once each
    g = bench.algorithmic_bytes(_tiny(temperature=0.0), n)
    assert g["stats"] == (1 + 4) * 40 and g["sample"] == 0
    # bf16 halves every row
    assert bench.algorithmic_bytes(_tiny(bf16=True), n)["stats"] == 4 * 40
    # flagged sequences (n = -1) cost only their I/O
    assert bench.algorithmic_bytes(_tiny(), np.array([-1, -1], np.int32))["total"] == io


def _pmc_file(d, kernel, workload, digest, hbm):
    with open(os.path.join(d, f"{kernel}_{workload}_pmc.txt"), "w") as f:
        f.write(f"# HBM traffic of {kernel}, workload {workload}\ncommand: x\nsource_digest: {digest}\n"
                f"dispatches: 3\nhbm_bytes_per_launch: {hbm}\n")


def test_read_traffic_requires_the_current_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    _pmc_file(tmp_path, "k_rows", "c4b", bench.source_digest(), 123456)
    _pmc_file(tmp_path, "k_rows", "c4a", "0000000000000000", 999)
    assert bench.read_traffic("k_rows", "c4b") == 123456.0
    assert bench.read_traffic("k_rows", "c4a") is None        # taken on other sources
    assert bench.read_traffic("k_judge", "c4b") is None       # no summary


def test_source_digest_ignores_comments(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "a.h").write_text("int f(int x) { return x + 1; }  // one\n")
    monkeypatch.setattr(bench, "CSRC", str(src))
    d0 = bench.source_digest()
    (src / "a.h").write_text("/* a note */\nint f(int x) {\n  return x + 1;  // another\n}\n")
    assert bench.source_digest() == d0
    (src / "a.h").write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_digest() != d0


HEADER = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size",'
          '"Kernel_Id","Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count",'
          '"Accum_VGPR_Count","SGPR_Count","Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"\n')


def _counter_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(HEADER)
        for disp, kernel, counter, value in rows:
            f.write(f'{disp},{disp},1,1,1,1,1,1,"{kernel}",256,0,0,44,0,64,"{counter}",{value},0,1\n')


def test_busy_summary_per_instantiation(tmp_path):
    k0 = "void sv::k_rows<1, 0>(sv::Args, int, int, int, int, int, int)"
    k1 = "void sv::k_rows<1, 1>(sv::Args, int, int, int, int, int, int)"
    rows = []
    for disp, k, vb, ta, gui in ((1, k0, 40.0, 50, 1000), (2, k0, 60.0, 150, 1000), (3, k1, 30.0, 7, 700)):
        rows += [(disp, k, "VALUBusy", vb), (disp, k, "TA_BUSY_avr", ta), (disp, k, "GRBM_GUI_ACTIVE", gui),
                 (disp, k, "SQ_INSTS_VALU", 1000 * disp), (disp, k, "SQ_INSTS_VALU_TRANS_F32", 10 * disp)]
    _counter_csv(str(tmp_path / "busy" / "h" / "run_counter_collection.csv"), rows)
    bench.busy_summary(argparse.Namespace(rocprof_busy=str(tmp_path), workload="c2", steps=5, warmup=2))
    text = (tmp_path / "busy_c2.txt").read_text().splitlines()
    assert f"source_digest: {bench.source_digest()}" in text
    # two dispatches of k_rows<1, 0>: VALU busy 50 %, memory unit 10 %; one of k_rows<1, 1>
    assert "k_rows<1, 0> | 2 | 50.0 | 10.0 | 1500 | 15" in text
    assert "k_rows<1, 1> | 1 | 30.0 | 1.0 | 3000 | 30" in text


def test_rocprof_summary_scales_by_the_copy(tmp_path):
    k = "void sv::k_rows<0, 2>(sv::Args, int, int, int, int, int, int)"
    os.makedirs(tmp_path / "trace" / "h")
    with open(tmp_path / "trace" / "h" / "run_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{k}",4,200000,50000,90.0,40000,60000,1\n')
    # the kernel: 1000 KiB fetched, 10 KiB written per dispatch; the 1 MiB copy
    # reads 512 KiB by FETCH_SIZE (scale 2) and writes 1024 KiB (scale 1)
    _counter_csv(str(tmp_path / "fetch" / "h" / "run_counter_collection.csv"),
                 [(1, k, "FETCH_SIZE", 1000), (2, k, "FETCH_SIZE", 1000)])
    _counter_csv(str(tmp_path / "write" / "h" / "run_counter_collection.csv"),
                 [(1, k, "WRITE_SIZE", 10), (2, k, "WRITE_SIZE", 10)])
    _counter_csv(str(tmp_path / "cfetch" / "h" / "run_counter_collection.csv"),
                 [(1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 512)])
    _counter_csv(str(tmp_path / "cwrite" / "h" / "run_counter_collection.csv"),
                 [(1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1024)])
    bench.rocprof_summary(argparse.Namespace(rocprof_summary=str(tmp_path), workload="c4b", steps=5, warmup=2,
                                             draft_only=False, copy_calib_mb=1))
    trace = (tmp_path / "kernel_trace_c4b.txt").read_text()
    assert "k_rows | 4 | 50.00 | 40.00 | 60.00 | 200.0 | 90.00" in trace
    pmc = (tmp_path / "k_rows_c4b_pmc.txt").read_text().splitlines()
    assert "fetch_scale: 2.0000" in pmc and "write_scale: 1.0000" in pmc
    assert f"hbm_bytes_per_launch: {(1000 * 2 + 10) * 1024}" in pmc
