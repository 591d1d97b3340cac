"""Host-side checks of the profiling summaries (CPU only)."""
import os

from nvfp4_block_scaled_03_amd import profiling

ROOT = os.path.dirname(os.path.dirname(__file__))


def test_committed_traffic_summary_parses():
    path = os.path.join(ROOT, "profiles", "grouped_gemm1_swiglu_decode_traffic.txt")
    t = profiling.read_traffic(path)
    for k in ("bytes_per_call", "fetch_scale", "write_scale", "sources_sha256_16"):
        assert k in t, k
    fetch, write = float(t["fetch_bytes_per_call"]), float(t["write_bytes_per_call"])
    assert float(t["bytes_per_call"]) == round(fetch) + round(write) or \
        abs(float(t["bytes_per_call"]) - fetch - write) <= 1
    assert len(t["sources_sha256_16"]) == 16


def test_traffic_summary_from_counter_rows(tmp_path, capsys):
    def write(name, counter, rows):
        p = tmp_path / name
        with open(p, "w") as f:
            f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
            for d, k, v in rows:
                f.write(f'{d},"{k}",{counter},{v}\n')
        return str(p)
    k = "void nvfp4::grouped_gemm_stream4_kernel<0, 0, 1, 2, 4>(KParams)"
    # Two dispatches of the kernel, one counter row per XCD piece summed.
    f = write("f.csv", "FETCH_SIZE", [(1, k, 100.0), (1, k, 28.0), (2, k, 128.0), (3, "other", 9.0)])
    w = write("w.csv", "WRITE_SIZE", [(1, k, 4.0), (2, k, 4.0)])
    cf = write("cf.csv", "FETCH_SIZE", [(7, "__amd_rocclr_copyBuffer", 512.0)])
    cw = write("cw.csv", "WRITE_SIZE", [(7, "__amd_rocclr_copyBuffer", 1024.0)])
    profiling.main(["traffic", "--fetch", f, "--write", w, "--copy-fetch", cf, "--copy-write", cw,
                    "--mib", "1", "--copy-re", "rocclr_copyBuffer"])
    out = tmp_path / "s.txt"
    out.write_text(capsys.readouterr().out)
    t = profiling.read_traffic(str(out))
    assert t["dispatches_fetch"] == "2" and float(t["fetch_scale"]) == 2.0
    assert float(t["fetch_bytes_per_call"]) == 128 * 1024 * 2
    assert float(t["write_bytes_per_call"]) == 4 * 1024
    assert t["sources_sha256_16"] == profiling.sources_hash()


def test_counters_summary_derived_fractions(tmp_path, capsys):
    """rocprofv3's MfmaUtil / VALUBusy formulas on synthetic rows: the per-XCC
    GUI cycles are the 8-XCC sum / 8, MFMA busy is per SIMD (1024), VALU
    active per CU (256)."""
    p = tmp_path / "c.csv"
    k = "void nvfp4::grouped_gemm_wide_kernel<1, 0>(KParams)"
    rows = [(1, "GRBM_GUI_ACTIVE", 8 * 1000.0), (1, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1000 * 1024),
            (1, "SQ_ACTIVE_INST_VALU", 0.25 * 1000 * 256), (2, "GRBM_GUI_ACTIVE", 8 * 1000.0),
            (2, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1000 * 1024), (2, "SQ_ACTIVE_INST_VALU", 0.25 * 1000 * 256)]
    with open(p, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for d, c, v in rows:
            f.write(f'{d},"{k}",{c},{v}\n')
    profiling.main(["counters", "--csv", str(p), "--kernel-re", "wide_kernel<1, 0>"])
    out = capsys.readouterr().out
    vals = dict(l.split(" = ")[0:2] for l in out.splitlines() if " = " in l and not l.startswith("#"))
    assert float(vals["mfma_util"].split()[0]) == 0.5
    assert float(vals["valu_busy"].split()[0]) == 0.25
