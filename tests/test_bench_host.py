"""Host logic of bench.py, on the CPU: the allowed-pair count that every
TFLOP/s figure divides by, the refusal of more than one GPU, and the
committed counter summaries being read only while they match the kernel
source they were taken on."""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _brute_pairs(n_q, n_k, causal, window):
    i = np.arange(n_q)[:, None]
    j = np.arange(n_k)[None, :]
    delta = n_k - n_q
    ok = np.ones((n_q, n_k), dtype=bool)
    if causal:
        ok &= j <= i + delta
    if window >= 0:
        ok &= j >= i + delta - window
    return int(ok.sum())


@pytest.mark.parametrize("n_q,n_k,causal,window", [
    (1, 1, False, -1), (7, 5, True, -1), (5, 7, True, -1), (33, 33, True, 4),
    (40, 29, False, 3), (29, 40, True, 0), (64, 64, True, 100), (17, 80, False, -1)])
def test_pairs_match_brute_force(n_q, n_k, causal, window):
    assert bench.pairs_dense(n_q, n_k, causal, window) == _brute_pairs(n_q, n_k, causal, window)


def test_pairs_closed_forms():
    # non-causal: every pair; causal square: the lower triangle with the diagonal
    assert bench.pairs_dense(2048, 2048, False, -1) == 2048 * 2048
    assert bench.pairs_dense(8000, 8000, True, -1) == 8000 * 8001 // 2
    # causal with W keys left of the diagonal: a triangle of W + 1 rows, then W + 1 per row
    W = 1024
    for L in (100, 1025, 1026, 4096):
        expect = L * (L + 1) // 2 if L <= W + 1 else (W + 1) * (W + 2) // 2 + (W + 1) * (L - W - 1)
        assert bench.pairs_dense(L, L, True, W) == expect


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def test_traffic_summary_is_read_only_for_its_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("kernel source v1\n")
    summary = tmp_path / "traffic.txt"
    assert bench.read_traffic(str(summary), str(src)) is None  # absent
    summary.write_text(f"kernel: k\nhbm_bytes_per_launch: 12345\n"
                       f"kernel_source_sha256: {_sha(src)}\n")
    assert bench.read_traffic(str(summary), str(src)) == 12345.0
    src.write_text("kernel source v2\n")
    assert bench.read_traffic(str(summary), str(src)) is None  # stale


def test_mfma_summary_round_trip(tmp_path):
    """Synthetic counter CSVs in rocprofv3's column layout through
    mfma_summary, then read back per kernel while the source matches."""
    src = tmp_path / "kernel.hip"
    src.write_text("kernel source\n")
    util_dir, raw_dir = tmp_path / "util", tmp_path / "raw"
    util_dir.mkdir()
    raw_dir.mkdir()
    kname = "void fa::(anonymous namespace)::fwd_bf16_kernel<128, false>(fa::FwdArgs)"
    other = "void at::native::elementwise_kernel<128, 4>(int)"
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    (util_dir / "a_counter_collection.csv").write_text(
        head + f'1,"{kname}",MfmaUtil,40.0,0,1000\n2,"{kname}",MfmaUtil,50.0,0,1000\n'
               f'3,"{kname}",MfmaUtil,60.0,0,1000\n4,"{other}",MfmaUtil,99.0,0,1000\n')
    rows = []
    for i, (mops, grbm) in enumerate([(100, 8000), (300, 9000), (200, 10000)]):
        rows.append(f'{i},"{kname}",SQ_INSTS_VALU_MFMA_MOPS_BF16,{mops},0,{2000 + 1000 * i}')
        rows.append(f'{i},"{kname}",GRBM_GUI_ACTIVE,{grbm},0,{2000 + 1000 * i}')
    (raw_dir / "b_counter_collection.csv").write_text(head + "\n".join(rows) + "\n")
    out = tmp_path / "summary.txt"
    old = bench.PREFILL_KERNEL_SRC
    bench.PREFILL_KERNEL_SRC = str(src)
    try:
        bench.mfma_summary(str(util_dir), str(raw_dir), "prefill_2k", str(out), "cmd", 1)
    finally:
        bench.PREFILL_KERNEL_SRC = old
    text = out.read_text()
    assert "kernel: fwd_bf16_kernel<128, false>" in text
    assert "elementwise" not in text  # only the library's kernels
    assert "mfma_util_pct: 50.00" in text  # median of 40, 50, 60
    assert "mfma_flops_bf16: 102400" in text  # median MOPS 200 x 512
    assert "dispatch_us_under_counters: 3.00" in text  # median of 2, 3, 4 us
    assert bench.read_mfma_util(str(out), str(src), "fwd_bf16_kernel<128, false>") == 50.0
    src.write_text("changed\n")
    assert bench.read_mfma_util(str(out), str(src), "fwd_bf16_kernel<128, false>") is None


def test_source_digest_covers_included_headers(tmp_path):
    """A kernel's digest changes when a local header it includes changes,
    and not when an unrelated file does."""
    (tmp_path / "common.h").write_text("inline int f() { return 1; }\n")
    (tmp_path / "other.h").write_text("unrelated\n")
    src = tmp_path / "kernel.hip"
    src.write_text('#include "common.h"\n#include <hip/hip_runtime.h>\nint g();\n')
    d0 = bench.sha256(str(src))
    (tmp_path / "other.h").write_text("changed\n")
    assert bench.sha256(str(src)) == d0
    (tmp_path / "common.h").write_text("inline int f() { return 2; }\n")
    assert bench.sha256(str(src)) != d0


class _FakeSmi:
    """Stands in for amdsmi: a metrics table that changes every third read,
    idle for the first two tables."""

    class AmdSmiClkType:
        GFX = 0

    def __init__(self):
        self.reads = 0

    def amdsmi_init(self):
        pass

    def amdsmi_get_processor_handles(self):
        return ["h0"]

    def amdsmi_get_gpu_device_bdf(self, h):
        return "0000:0a:00.0"

    def amdsmi_get_gpu_metrics_info(self, h):
        self.reads += 1
        t = (self.reads - 1) // 3
        busy = t >= 2
        return {"average_gfx_activity": 94 if busy else 0,
                "gfx_activity_acc": 1000 + t,
                "current_socket_power": 1200 + t if busy else 240,
                "current_gfxclks": [1800 + t, 1700 + t, "N/A"] if busy else [95, 96]}


def test_clock_sampler_keeps_distinct_loaded_tables(monkeypatch):
    import types

    fake = _FakeSmi()
    mod = types.ModuleType("amdsmi")
    for name in dir(fake):
        if name.startswith("amdsmi_") or name == "AmdSmiClkType":
            setattr(mod, name, getattr(fake, name))
    monkeypatch.setitem(sys.modules, "amdsmi", mod)

    class _Props:
        pci_domain_id, pci_bus_id = 0, 10

    class _Cuda:
        @staticmethod
        def get_device_properties(i):
            return _Props()

    class _Torch:
        cuda = _Cuda

    c = bench.ClockSampler(_Torch, period_s=0.0)
    assert c.error is None
    reads = [c._read() for _ in range(12)]
    # idle tables (the first 6 reads) are dropped; each loaded table is the
    # XCD mean of its numeric clocks
    assert reads[:6] == [None] * 6
    assert reads[6][1] == (1802 + 1702) / 2 and reads[6][2] == 1202
    keys = {r[0] for r in reads[6:]}
    assert len(keys) == 2  # tables 2 and 3, three reads each


def test_sweep_summary_splits_blocks_and_recovers_the_fit(tmp_path):
    # synthetic trace: each shape's launches take (steps*t + items*x + c)
    # cycles at that shape's clock in its timed window and a different time
    # elsewhere (the clock and settle phases), with an unrelated kernel
    # interleaved
    t, x, c = 3400.0, 9000.0, 15000.0
    clock = {1024: 2000.0, 2048: 1900.0, 3072: 1880.0, 4096: 1850.0, 6144: 1820.0, 8192: 1800.0}
    kt = tmp_path / "kt"
    kt.mkdir()
    lines, log = [], []
    ts = 1000
    for n in bench.SWEEP_N:
        items = 4 * 16 * n // bench.SWEEP_ROWS_PER_ITEM // bench.SWEEP_WGS
        steps = items * n // bench.SWEEP_KEYS_PER_STEP
        want = (steps * t + items * x + c) / clock[n]   # microseconds
        first, timed, launches = 7, 5, 20
        for i in range(launches):
            dur = want if first <= i < first + timed else want * 1.3
            lines.append((f"void fa::(anonymous namespace)::{bench.HEADLINE_KERNEL}(fa::FwdArgs)",
                          ts, ts + int(round(dur * 1e3))))
            ts += int(dur * 1e3) + 500
            lines.append(("elementwise_kernel", ts, ts + 100))
            ts += 600
        log.append(f"[sweep] clock n={n} mhz={clock[n]} socket_w=1300 snapshots=3 error=None")
        log.append(f"[sweep] n={n} launches={launches} timed_first={first} timed={timed} "
                   f"event_mean_ms={want / 1e3:.5f} tflops=1.0")
    with open(kt / "kt_kernel_trace.csv", "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for name, a, b in reversed(lines):   # the summary sorts by start time
            f.write(f'"{name}",{a},{b}\n')
    (tmp_path / "run.log").write_text("\n".join(log) + "\n")
    out = tmp_path / "sweep.txt"
    bench.sweep_summary(str(kt), str(tmp_path / "run.log"), str(out), "cmd")
    vals = {}
    for ln in out.read_text().splitlines():
        k, _, v = ln.strip().partition(":")
        vals[k] = v.strip()
    assert abs(float(vals["t_cycles_per_step"]) - t) < 2
    assert abs(float(vals["x_cycles_per_item"]) - x) < 30
    assert abs(float(vals["c_cycles_per_launch"]) - c) < 60
    # the factors multiply to the measured fraction at N = 2048
    assert abs(float(vals["product"]) - float(vals["frac_of_2500_tflops"])) < 1e-3
    assert abs(float(vals["clock_factor (clock / 2400 MHz)"]) - 1900 / 2400) < 1e-4


def test_sweep_summary_rejects_a_trace_that_does_not_match_the_log(tmp_path):
    kt = tmp_path / "kt"
    kt.mkdir()
    with open(kt / "kt_kernel_trace.csv", "w") as f:
        f.write('"Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        f.write(f'"fa::{bench.HEADLINE_KERNEL}(fa::FwdArgs)",1,2\n')
    (tmp_path / "run.log").write_text(
        "[sweep] n=1024 launches=3 timed_first=0 timed=1 event_mean_ms=0.1 tflops=1\n")
    with pytest.raises(SystemExit):
        bench.sweep_summary(str(kt), str(tmp_path / "run.log"), str(tmp_path / "o.txt"), "cmd")
