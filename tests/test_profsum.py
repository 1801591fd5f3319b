"""The rocprofv3 summariser (host logic only): kernel names as rocprofv3 prints them map to the
library's trace names, and FETCH/WRITE counters scale to bytes by the calibration copy."""
import csv
import json
import os

from chunked_scan_amd import profsum

_PIPE_ARGS = "EEEvPKDF16bS3_S3_PKfS5_PDF16bPflS7_S7_S5_liilliiifS6_S7_lPhPi"
PIPE_OUT = "_ZN2la12_GLOBAL__N_115pipe_fwd_kernelILi0ELb0ELb0" + _PIPE_ARGS
PIPE_ST = "_ZN2la12_GLOBAL__N_115pipe_fwd_kernelILi2ELb1ELb0" + _PIPE_ARGS
DQ_OUT = "_ZN2la12_GLOBAL__N_115pipe_fwd_kernelILi1ELb0ELb1" + _PIPE_ARGS
DQ_ST = "_ZN2la12_GLOBAL__N_115pipe_fwd_kernelILi0ELb1ELb1" + _PIPE_ARGS
DKDV_WIN = "_ZN2la12_GLOBAL__N_115bwd_dkdv_kernelILi128ELi1ELb0ELb1EEEvPKDF16bS3_S3_S3_PKfS5_lPDF16bS6_PfS7_S7_S5_PdS6_lliiifPi"
DKDV_FACT = "_ZN2la12_GLOBAL__N_115bwd_dkdv_kernelILi128ELi1ELb0ELb0ELb1EEEvPKDF16bS3_S3_S3_PKfS5_lPDF16bS6_PfS7_S7_S5_PdS6_lliiifPi"
DKDV_HEAD = "_ZN2la12_GLOBAL__N_120bwd_dkdv_head_kernelILi128EEEvPKDF16bS3_S3_S3_PKfS5_lPDF16bS6_PfS7_S7_S5_PdS6_lliiifPi"
DQ_GATE_ST = "_ZN2la12_GLOBAL__N_118bwd_dq_gate_kernelILi128ELb1EEEvPKDF16bS3_S3_PKfS5_S5_lPDF16bPfS7_S5_liiS3_S7_lliiifPi"
SCAN = "void la::(anonymous namespace)::state_scan_vec_kernel<5, 4>(float const*, float const*, float*, int, int, int, long, int)"
COPY = "__amd_rocclr_copyBuffer"


def test_labels():
    names = profsum._demangle([PIPE_OUT, PIPE_ST, DQ_OUT, DQ_ST, DKDV_WIN, DKDV_FACT, DKDV_HEAD, DQ_GATE_ST, SCAN, COPY])
    assert profsum.label(names[PIPE_OUT]) == ("chunk_fwd_pipe_output_pass", "pipe_fwd_kernel<NONE, outputs>")
    assert profsum.label(names[PIPE_ST]) == ("chunk_fwd_pipe_state_pass", "pipe_fwd_kernel<GATE, state pass>")
    assert profsum.label(names[DQ_OUT]) == ("chunk_bwd_dq", "pipe_fwd_kernel<HEAD, outputs, dq>")
    assert profsum.label(names[DQ_ST]) == ("chunk_bwd_dq_state_pass", "pipe_fwd_kernel<NONE, state pass, dq>")
    assert profsum.label(names[DKDV_WIN]) == ("chunk_bwd_dkdv_windows", "bwd_dkdv_kernel<128, HEAD, outputs, windows>")
    assert profsum.label(names[DKDV_FACT]) == ("chunk_bwd_dkdv", "bwd_dkdv_kernel<128, HEAD, outputs, factorised>")
    assert profsum.label(names[DKDV_HEAD]) == ("chunk_bwd_dkdv", "bwd_dkdv_head_kernel<128>")
    assert profsum.label(names[DQ_GATE_ST]) == ("chunk_bwd_dq_state_pass", "bwd_dq_gate_kernel<128, state pass>")
    assert profsum.label(names[SCAN]) == ("state_scan", "state_scan_vec_kernel<5, 4>")
    assert profsum.label(names[COPY])[0] is None


def _pmc_csv(d, counter, rows):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, v in rows:
            wr.writerow(dict(Kernel_Name=name, Counter_Name=counter, Counter_Value=v))


def test_pmc_scaling_and_traffic_json(tmp_path, capsys):
    # a 64 MiB copy that FETCH_SIZE counts at half its bytes and WRITE_SIZE at all of them
    _pmc_csv(tmp_path / "f", "FETCH_SIZE", [(COPY, 32768.0), (PIPE_OUT, 1000.0), (PIPE_OUT, 3000.0), (SCAN, 10.0)])
    _pmc_csv(tmp_path / "w", "WRITE_SIZE", [(COPY, 65536.0), (PIPE_OUT, 500.0), (PIPE_OUT, 500.0), (SCAN, 5.0)])
    out = tmp_path / "t.json"
    profsum.main(["pmc", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"), "--calib-mib", "64",
                  "--traffic-json", str(out), "--workload", "wl", "--kernel", "chunk_fwd_pipe_output_pass",
                  "--command", "rocprofv3 ..."])
    text = capsys.readouterr().out
    assert "| chunk_fwd_pipe_output_pass | pipe_fwd_kernel<NONE, outputs> | 2 | 2000 | 500 |" in text
    tr = json.loads(out.read_text())
    assert tr["fetch_scale"] == 2.0 and tr["write_scale"] == 1.0
    assert tr["bytes_per_launch"] == 2000 * 1024 * 2 + 500 * 1024
    assert tr["source_sha256_16"] == profsum.source_hash() and tr["workload"] == "wl"


def test_stats_rows(tmp_path):
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "kt_kernel_stats.csv", "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        wr.writerow([PIPE_OUT, 4, 200000, 50000, 80.0, 45000, 60000, 1.0])
        wr.writerow([SCAN, 4, 40000, 10000, 16.0, 9000, 11000, 1.0])
        wr.writerow([COPY, 1, 10000, 10000, 4.0, 10000, 10000, 0.0])
    rows = profsum.stats_rows(str(d))
    assert [r[0] for r in rows] == ["chunk_fwd_pipe_output_pass", "state_scan"]
    assert rows[0][2:] == (4, 50.0, 45.0, 60.0)
