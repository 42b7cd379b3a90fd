"""CPU tests of the measurement tooling around the library: bench.py's
one-GPU guard and profile reader, and the rocprofv3 summaries in
compressed_decode_attention_kv_amd.profiling (synthetic CSV files in the
profiler's column layout)."""
import csv
import os
import subprocess
import sys

import pytest

from compressed_decode_attention_kv_amd import profiling as pf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bench_traffic_needs_matching_sources(tmp_path, monkeypatch):
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("kqv") is None                        # no summary
    (prof / "traffic_isotropic_kqv.txt").write_text(
        "# header\ndecode_sources_sha1 = %s\ndecode_chain_bytes = 2.5e+09\n"
        "quantize_sources_sha1 = %s\nquantize_chain_bytes = 1.1e+10\n"
        % (pf.decode_sources_sha(), pf.quantize_sources_sha()))
    assert bench.measured_traffic("kqv") == 2.5e9
    assert bench.measured_traffic("kqv", "quantize") == 1.1e10
    (prof / "traffic_isotropic_kqv.txt").write_text(
        "decode_sources_sha1 = 0000\ndecode_chain_bytes = 2.5e+09\n"
        "quantize_sources_sha1 = %s\nquantize_chain_bytes = 1.1e+10\n" % pf.quantize_sources_sha())
    assert bench.measured_traffic("kqv") is None                        # taken on other sources
    assert bench.measured_traffic("kqv", "quantize") == 1.1e10


def test_bench_reads_quantize_mfma_util(tmp_path, monkeypatch):
    import bench
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    head = "%-90s %5s " % ("kernel", "disp") + " ".join("%16s" % c for c in
                                                       ("VALU insts", "VALUBusy%", "LdsUtil%", "LDSBankConflict%",
                                                        "MfmaUtil%"))
    row = "%-90s %5d " % ("quant_mfma_kernel<3, 2, _Float16>(tq::QuantParamsENS_9QuantGrid)", 4) + \
        " ".join("%16.4g" % v for v in (6.4e8, 74.7, 37.1, 0.5, 38.47))
    body = "\n".join([head, row]) + "\n"
    (prof / "counters_isotropic_kqv.txt").write_text("# quantize_sources_sha1 = %s\n" % pf.quantize_sources_sha()
                                                     + body)
    assert bench.measured_mfma_util("kqv") == {"quant_mfma_kernel<3, 2, _Float16>(tq::QuantParamsENS_9QuantGrid)":
                                               38.47}
    (prof / "counters_isotropic_kqv.txt").write_text("# quantize_sources_sha1 = 00\n" + body)
    assert bench.measured_mfma_util("kqv") is None


def _trace_row(name, grid, t0, dur_ns):
    return {"Kind": "KERNEL_DISPATCH", "Kernel_Name": name, "Grid_Size_X": grid, "Grid_Size_Y": 1,
            "Grid_Size_Z": 1, "Start_Timestamp": t0, "End_Timestamp": t0 + dur_ns}


def test_stats_keeps_full_size_dispatches(tmp_path):
    """Averages over each kernel's largest grid only; calls count all."""
    k = "_ZN2tq12_GLOBAL__N_117quant_mfma_kernelILi3ELi2EDF16_EEvNS_11QuantParamsENS_9QuantGridE"
    rows = [_trace_row(k, 524288, 0, 2_000_000), _trace_row(k, 524288, 10**7, 2_200_000),
            _trace_row(k, 512, 2 * 10**7, 9_000)] + \
           [_trace_row("tq::(anonymous namespace)::combine_kernel(tq::CombineParams)", 8192, 3 * 10**7, 9_000)]
    rows.append(_trace_row("void at::native::distribution_kernel<float>(int)", 1024, 4 * 10**7, 5_000))
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    (tmp_path / "run_kernel_stats.csv").write_text("")
    lines = pf.stats(str(tmp_path / "run_kernel_stats.csv")).split("\n")
    quant = [l for l in lines if l.startswith("quant_mfma_kernel<3, 2, _Float16>")]
    assert len(quant) == 1
    calls, full, avg = quant[0].split()[-3:]
    assert (int(calls), int(full), float(avg)) == (3, 2, 2100.0)
    assert any(l.startswith("combine_kernel") for l in lines)
    # Kernels that are not the library's are listed too.
    assert any(l.startswith("at::native::distribution_kernel") for l in lines)
    # --last N: the average over the last N full-size dispatches (in time order).
    lines = pf.stats(str(tmp_path / "run_kernel_stats.csv"), last=1).split("\n")
    quant = [l for l in lines if l.startswith("quant_mfma_kernel<3, 2, _Float16>")][0].split()
    assert (float(quant[-2]), float(quant[-1])) == (2100.0, 2200.0)


def test_counters_derived_utilisations(tmp_path):
    """VALUBusy = SQ_ACTIVE_INST_VALU / CUs / (GRBM_GUI_ACTIVE / XCDs), per
    dispatch, median over the full-size dispatches."""
    name = "tq::(anonymous namespace)::stream_read_kernel(unsigned int __vector(4) const*)"
    rows = []
    for did, grid, valu, grbm, mfma in ((1, 4096, 256 * 500.0, 8 * 1000.0, 1024 * 100.0),
                                        (2, 4096, 256 * 700.0, 8 * 1000.0, 1024 * 300.0),
                                        (3, 64, 256 * 10.0, 8 * 1000.0, 0.0)):
        for c, v in (("SQ_ACTIVE_INST_VALU", valu), ("GRBM_GUI_ACTIVE", grbm), ("SQ_VALU_MFMA_BUSY_CYCLES", mfma),
                     ("SQ_INSTS_VALU", valu)):
            rows.append({"Dispatch_Id": did, "Grid_Size": grid, "Kernel_Name": name, "Counter_Name": c,
                         "Counter_Value": v})
    _write_csv(tmp_path / "run_counter_collection.csv", rows)
    _write_csv(tmp_path / "run_agent_info.csv", [{"Agent_Type": "GPU", "Cu_Count": 256, "Simd_Count": 1024,
                                                   "Num_Xcc": 8}])
    out = pf.counters([str(tmp_path / "run_counter_collection.csv")]).split("\n")
    row = [l for l in out if l.startswith("stream_read_kernel")][0].split()
    n, valu_insts, valu_busy, mfma_util = int(row[-6]), float(row[-5]), float(row[-4]), float(row[-1])
    assert row[-3] == row[-2] == "-"                  # no LDS counters in this pass
    assert n == 2                                     # the 64-thread dispatch is left out
    assert valu_insts == pytest.approx(256 * 600.0)
    assert valu_busy == pytest.approx(60.0)           # median of 50 % and 70 %
    assert mfma_util == pytest.approx(20.0)           # median of 10 % and 30 %


def test_short_names():
    assert pf.short("_ZN2tq12_GLOBAL__N_117quant_mfma_kernelILi4ELi1EDF16_EEvNS_11QuantParamsENS_9QuantGridE") == \
        "quant_mfma_kernel<4, 1, _Float16>(tq::QuantParamsENS_9QuantGrid)"
    assert pf.short("void tq::(anonymous namespace)::decode_lut_kernel<128, 4, false, 3, true>(tq::DecodeParams)") \
        .startswith("decode_lut_kernel<128, 4, false, 3, true>")
