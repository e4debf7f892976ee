"""The rocprofv3 summaries the benchmark and the profiles rely on, on synthetic
counter output (no GPU): kernel names, copy-calibrated traffic, the source
digest that ties a traffic summary to the kernels it measured, and the clock
and matrix-core busy share derived from GRBM/SQ counters."""
import csv
import io
import os
from contextlib import redirect_stdout

from newton_schulz_03_amd import rocprof_summary as rs

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]

COPY = ("void at::native::vectorized_elementwise_kernel<4, at::native::AUnaryFunctor<float, "
        "float, float, at::native::binary_internal::MulFunctor<float> > >")
WIDE = "void muon::k_gemm_bf16_wide<false>(muon::LaunchCtx, muon::GemmArgs)"
WIDE_FIRST = "void muon::k_gemm_bf16_wide<true>(muon::LaunchCtx, muon::GemmArgs)"
GRAM = "void muon::k_gemm_bf16<0, false, false, false>(muon::LaunchCtx, muon::GemmArgs)"
FINISH = "void muon::k_gemm_bf16<2, true, false, false>(muon::LaunchCtx, muon::GemmArgs)"


def write_counters(d, rows):
    """rows: (dispatch, kernel name, counter, value, start ns, end ns)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for disp, name, counter, value, t0, t1 in rows:
            r = {c: 0 for c in COLS}
            r.update(Correlation_Id=disp, Dispatch_Id=disp, Kernel_Name=name,
                     Counter_Name=counter, Counter_Value=value, Start_Timestamp=t0,
                     End_Timestamp=t1)
            w.writerow(r)


def run(argv):
    out = io.StringIO()
    with redirect_stdout(out):
        rs.main(argv)
    return out.getvalue()


def test_kernel_names():
    assert rs.short_name(WIDE) == "prod"
    assert rs.short_name(WIDE_FIRST) == "prod_first"
    assert rs.short_name(GRAM) == "gram"
    assert rs.short_name(FINISH) == "prod_finish"
    assert rs.short_name(COPY) == "copy"
    assert rs.short_name("void muon::k_prepare<unsigned short>(muon::LaunchCtx)") == "prepare"


def test_traffic_is_scaled_by_the_copy(tmp_path):
    gib = 1 << 30
    # the fetch counter reads half the copy's bytes, the write counter all of them
    write_counters(tmp_path / "f", [(1, COPY, "FETCH_SIZE", gib // 2048, 0, 1),
                                    (2, WIDE, "FETCH_SIZE", 3_000_000, 0, 1),
                                    (3, WIDE, "FETCH_SIZE", 1_000_000, 0, 1)])
    write_counters(tmp_path / "w", [(1, COPY, "WRITE_SIZE", gib // 1024, 0, 1),
                                    (2, WIDE, "WRITE_SIZE", 2_000_000, 0, 1),
                                    (3, WIDE, "WRITE_SIZE", 2_000_000, 0, 1)])
    text = run(["traffic", str(tmp_path / "f"), str(tmp_path / "w"), "--copy-bytes", str(gib),
                "--workload", "wl", "--command", "cmd"])
    want = (2_000_000 * 2.0 + 2_000_000 * 1.0) * 1024  # mean per dispatch, scaled
    summary = tmp_path / "traffic.md"
    summary.write_text(text)
    assert rs.read_traffic(str(summary), "wl") == int(want)
    assert rs.read_traffic(str(summary), "another workload") is None
    # a summary taken on other kernel sources is not read back
    summary.write_text(text.replace(rs.kernel_source_digest(), "0" * 64))
    assert rs.read_traffic(str(summary), "wl") is None
    assert rs.read_traffic(str(tmp_path / "missing.md"), "wl") is None


def test_clock_and_busy_share(tmp_path):
    # one 1 ms dispatch at 1.8 GHz (GRBM cycles summed over the XCDs) with the
    # matrix cores busy half of the SIMD cycles; waves waiting 10% of their time
    cyc = 1.8e9 * 1e-3
    rows = [(1, WIDE, "GRBM_GUI_ACTIVE", cyc * rs.N_XCD, 0, 1_000_000),
            (1, WIDE, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * rs.N_SIMD, 0, 1_000_000),
            (1, WIDE, "SQ_WAVE_CYCLES", 1000.0, 0, 1_000_000),
            (1, WIDE, "SQ_WAIT_ANY", 100.0, 0, 1_000_000),
            (1, WIDE, "SQ_WAIT_INST_ANY", 400.0, 0, 1_000_000)]
    write_counters(tmp_path / "c", rows)
    text = run(["clock", str(tmp_path / "c"), "--workload", "wl", "--command", "cmd"])
    line = next(l for l in text.splitlines() if l.startswith("| prod |"))
    cells = [c.strip() for c in line.strip("|").split("|")]
    assert cells[1] == "1" and cells[2] == "1.000"
    assert cells[3] == "1.80" and cells[4] == "50.0%" and cells[5] == "10.0%" and cells[6] == "40.0%"

