"""CPU checks of the bench harness: the FLOP count, the timing statistics and
the kernel-name check that ties a rocprofv3 trace to the library."""
import glob
import os

import pytest

import bench
import synthetic as syn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_count_is_the_stated_formula():
    """4*B*H*N^2*d forward, exactly halved when causal, 2.5x for the backward."""
    w = syn.WORKLOADS["C5"]
    assert w.flops_fwd() == 4 * 1 * 32 * 32768 ** 2 * 128 / 2
    w = syn.WORKLOADS["C4"]
    assert w.flops_bwd() == 2.5 * 4 * 2 * 16 * 16384 ** 2 * 64 / 2
    assert syn.WORKLOADS["C2a_nc"].flops_fwd() == 2 * syn.WORKLOADS["C2a"].flops_fwd()


def test_stats():
    s = bench.stats([5.0, 1.0, 3.0, 2.0, 4.0])
    assert s["ms"] == 3.0 and s["reps"] == 5
    assert abs(s["ms_p10"] - 1.4) < 1e-12 and abs(s["ms_p90"] - 4.6) < 1e-12


def test_kernel_check_logic():
    rows = [("void fa::fwd_fp8_pp_kernel<128, true, true>(fa::FwdParams)", 7, 6000.0),
            ("__amd_rocclr_fillBufferAligned", 3, 10.0)]
    assert bench.check_kernels(rows, "C5")["ok"]
    bad = rows + [("void fa::mystery_kernel<1>(fa::FwdParams)", 1, 1.0)]
    assert not bench.check_kernels(bad, "C5")["ok"]
    wrong = [("void fa::fwd_bf16_pp_kernel<128, true, 64, false, true, false>(fa::FwdParams)", 7, 6000.0)]
    assert not bench.check_kernels(wrong, "C5")["ok"]
    assert not bench.check_kernels([], "C5")["ok"]


def test_committed_headline_summary_names_library_kernels():
    """The committed kernel-trace summary of the headline workload shows the
    kernel the instance table dispatches for it, and only library kernels."""
    rows = bench.read_summary(bench.HEADLINE_SUMMARY)
    res = bench.check_kernels(rows, bench.HEADLINE)
    assert res["ok"], res


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))))
def test_profile_summaries_name_library_kernels(path):
    """Every kernel named in a committed summary table is one of the library's
    (or a runtime copy/fill kernel)."""
    for name, _, _ in bench.read_summary(path):
        if "fa::" in name:
            assert bench.base_name(name) in bench.LIB_KERNELS, (path, name)


def test_counter_summary_from_rocprof_csv(tmp_path):
    """The counter summary joins a counter run's per-dispatch counters with its
    kernel trace and forms the derived columns from the stated formulas."""
    d = tmp_path / "W"
    d.mkdir()
    k = "void fa::fwd_fp8_pp_kernel<128, true, true>(fa::FwdParams)"
    cnt = {"GRBM_GUI_ACTIVE": 8 * 2.0e6, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * 1024 * 2.0e6,
           "SQ_VALU_MFMA_COEXEC_CYCLES": 0.25 * 1024 * 2.0e6, "SQ_INSTS_MFMA": 100.0, "SQ_INSTS_VALU": 700.0,
           "SQ_INSTS_VALU_TRANS_F32": 0.1 * 1024 * 2.0e6 / 16}
    with open(d / "c_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for disp in (1, 2):
            for n, v in cnt.items():
                f.write(f'{disp},"{k}",{n},{v / 2}\n{disp},"{k}",{n},{v / 2}\n')   # two partial rows a counter
    with open(d / "c_kernel_trace.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n")
        f.write(f'1,"{k}",1000,1001000\n2,"{k}",5000,1005000\n')
    rows = bench.counter_summary_rows([("W", bench.counter_table(str(d)))])
    assert len(rows) == 1
    r = rows[0]
    assert r["us"] == 1000.0 and abs(r["clock_ghz"] - 2.0) < 1e-12
    assert abs(r["mfma_busy"] - 0.5) < 1e-12 and abs(r["coexec"] - 0.25) < 1e-12
    assert r["valu_insts"] == 600.0 and abs(r["trans_share"] - 0.1) < 1e-12
    out = tmp_path / "s.md"
    bench.write_counter_summary(rows, str(out), ["W=" + str(d)])
    text = out.read_text()
    assert "| W | `fa::fwd_fp8_pp_kernel<128, true, true>` | 1000.0 | 2.00 | 50.0% | 25.0% |" in text
    assert bench.read_summary(str(out)) == []
