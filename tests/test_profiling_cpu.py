"""Host-side checks of the rocprofv3 summarizers that bench.py reads: the
counter arithmetic on synthetic CSV rows, and the source-hash guard that
withholds a summary once the kernels it was taken on have changed."""
import csv

import pytest

from zigzag_ring_attention_amd import profiling

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value",
          "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow({k: r.get(k, 0) for k in FIELDS})


def test_traffic_calibration_and_per_launch_bytes(tmp_path):
    copy = 1 << 30
    # the permute copies `copy` bytes each way; its counters read half the
    # fetched bytes and all the written bytes (KiB), as on the device
    fetch = [dict(Dispatch_Id=1, Kernel_Name="permute_kernel(...)", Counter_Name="FETCH_SIZE",
                  Counter_Value=copy / 2048.0),
             dict(Dispatch_Id=2, Kernel_Name="void zz::bwd_dkv_kernel<bf16, 128>(...)", Counter_Name="FETCH_SIZE",
                  Counter_Value=1000.0),
             dict(Dispatch_Id=3, Kernel_Name="void zz::bwd_dkv_kernel<bf16, 128>(...)", Counter_Name="FETCH_SIZE",
                  Counter_Value=3000.0)]
    write = [dict(Dispatch_Id=1, Kernel_Name="permute_kernel(...)", Counter_Name="WRITE_SIZE",
                  Counter_Value=copy / 1024.0),
             dict(Dispatch_Id=2, Kernel_Name="void zz::bwd_dkv_kernel<bf16, 128>(...)", Counter_Name="WRITE_SIZE",
                  Counter_Value=500.0),
             dict(Dispatch_Id=3, Kernel_Name="void zz::bwd_dkv_kernel<bf16, 128>(...)", Counter_Name="WRITE_SIZE",
                  Counter_Value=500.0)]
    write_csv(tmp_path / "f.csv", fetch)
    write_csv(tmp_path / "w.csv", write)
    text = profiling.traffic_text(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "cmd", float(copy))
    out = tmp_path / "traffic.txt"
    out.write_text(text)
    # fetch calibration 2, write calibration 1: mean of (1000, 3000) KiB x 2 + 500 KiB
    expect = 2000.0 * 1024 * 2.0 + 500.0 * 1024
    assert profiling.read_traffic(str(out), "bwd_dkv_kernel") == pytest.approx(expect, rel=1e-6)
    assert profiling.read_traffic(str(out), "fwd_step_kernel") is None


def test_util_clock_and_busy(tmp_path):
    # one dispatch of 1 ms: 2e6 cycles on each of the 8 XCDs -> 2 GHz;
    # busy cycles = half of cycles x SIMDs
    cyc = 2.0e6
    rows = []
    name = "void zz::fwd_step_kernel<bf16, 128>(zz::FwdArgs)"
    for c, v in (("SQ_INSTS_MFMA", 1e6), ("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * profiling.SIMDS),
                 ("GRBM_GUI_ACTIVE", cyc * profiling.XCDS)):
        rows.append(dict(Dispatch_Id=7, Kernel_Name=name, Counter_Name=c, Counter_Value=v,
                         Start_Timestamp=0, End_Timestamp=1_000_000))
    write_csv(tmp_path / "u.csv", rows)
    out = tmp_path / "util.md"
    out.write_text(profiling.util_markdown(str(tmp_path / "u.csv"), "cmd"))
    u = profiling.read_util(str(out))
    assert u == {"fwd_step": (2.0, 0.5)}


def test_stale_summaries_are_withheld(tmp_path):
    h = profiling.sources_hash()
    stale = "0" * len(h)
    t = tmp_path / "traffic.txt"
    t.write_text("kernel_sources_sha256 %s\nkernel bwd_dkv_kernel dispatches 1 fetch_kib 1 write_kib 1 "
                 "hbm_bytes_per_launch 1.0e+09\n" % stale)
    assert profiling.read_traffic(str(t), "bwd_dkv_kernel") is None
    t.write_text(t.read_text().replace(stale, h))
    assert profiling.read_traffic(str(t), "bwd_dkv_kernel") == pytest.approx(1e9)
    u = tmp_path / "util.md"
    row = "| fwd_step_kernel | 16 | 16.938 | 17.609 | 1039.6 | 1.817 | 0.546 | 0.413 |\n"
    u.write_text("kernel_sources_sha256 %s\n\n%s" % (stale, row))
    assert profiling.read_util(str(u)) is None
    u.write_text("kernel_sources_sha256 %s\n\n%s" % (h, row))
    assert profiling.read_util(str(u)) == {"fwd_step": (1.817, 0.546)}
    assert profiling.read_util(str(tmp_path / "missing.md")) is None


def test_issue_mix_ratios(tmp_path):
    name = "void zz::bwd_dq_kernel<bf16, 128>(zz::BwdArgs)"
    a = {"SQ_INSTS_VALU": 500.0, "SQ_INSTS_MFMA": 100.0, "SQ_INSTS_LDS": 150.0, "SQ_INSTS_SALU": 50.0,
         "SQ_INSTS_VMEM_RD": 10.0, "SQ_WAVES": 4.0, "SQ_WAVE_CYCLES": 1000.0, "SQ_BUSY_CYCLES": 300.0}
    b = {"SQ_VALU_MFMA_BUSY_CYCLES": 3200.0 * profiling.SIMDS / 1e4, "SQ_VALU_MFMA_COEXEC_CYCLES": 80.0,
         "SQ_ACTIVE_INST_VALU": 1.0, "SQ_ACTIVE_INST_LDS": 1.0, "SQ_WAIT_INST_LDS": 50.0, "SQ_WAIT_ANY": 250.0,
         "SQ_INSTS_VALU_TRANS_F32": 60.0, "GRBM_GUI_ACTIVE": 6400.0 * profiling.XCDS / 1e4 * 1e4}
    for fn, counters in (("a.csv", a), ("b.csv", b)):
        write_csv(tmp_path / fn, [dict(Dispatch_Id=1, Kernel_Name=name, Counter_Name=c, Counter_Value=v)
                                  for c, v in counters.items()])
    text = profiling.issue_markdown([str(tmp_path / "a.csv"), str(tmp_path / "b.csv")], "cmd")
    row = [l for l in text.splitlines() if l.startswith("| bwd_dq_kernel")][0]
    cells = [float(x) for x in row.strip("|").split("|")[1:]]
    # (500-100)/100, 60/100, 150/100, 50/100, 10/100, busy 3200*S/1e4 / (6400 * S), co-exec 80/busy, 250/1000, 50/1000
    busy = b["SQ_VALU_MFMA_BUSY_CYCLES"]
    want = [4.0, 0.6, 1.5, 0.5, 0.1, busy / (6400.0 * profiling.SIMDS), 80.0 / busy, 0.25, 0.05]
    assert cells == pytest.approx(want, abs=1e-3)
