#!/usr/bin/env python3
"""Attention-forward bench on one MI355X.

``python bench.py [--gpus 1] [--steps K] [--warmup W]`` prints ONE JSON line.
A step is one ``fa_fwd`` launch over the B4 H16 N2048 d128 bf16 non-causal
prefill workload with its inputs resident in HBM; ``value`` is its
algorithmic throughput (4 * d FLOPs per allowed (query, key) pair) over K
timed steps.  The line also carries:

* ``roofline``: the prefill kernel's algorithmic FLOPs per launch divided by
  its mean launch duration (a pair of HIP events on the launch stream around
  the timed launches) against the
  dense bf16 matrix-core peak, plus the HBM traffic per launch read from the
  committed rocprofv3 counter summary when it was taken on the current kernel
  source (else null), and the mean launch time when a 1 GiB buffer is
  written before every launch (inputs no longer in the last-level cache);
* ``cpu_baseline``: the fp64 CPU oracle timed on this host's cores on the
  same workload;
* ``secondary``: the other workloads (causal 2k, 8000-token causal prompt,
  packed varlen with a 1024-key window, fp32 small case, KV-cache decode in
  HBM GB/s, chunked prefill of 512 new tokens against KV caches, and the
  backward pass of the headline shape, plain and causal, and the headline
  shape on e4m3 inputs against the fp8 matrix-core peak), each timed the same
  way.

Every workload first runs back to back for ``--settle-ms`` (default 400 ms)
so that the engine clock has left its idle ramp before the warmup steps.

``--profile-target NAME`` runs only NAME's launches (plus, with
``--calibrate-copy``, a plain device copy of known size) for rocprofv3;
``--trace-summary`` turns its kernel trace into the committed summary.
``--profile-target prefill_sweep`` runs the headline shape at N = 1024 ...
8192 and ``--sweep-summary`` fits the launch time per key step, per query
tile and per launch from its kernel trace.
``--pmc-summary FETCH_DIR WRITE_DIR`` turns two ``rocprofv3 --pmc`` runs into
the committed traffic summary under profiles/; ``--mfma-summary UTIL_DIR
RAW_DIR`` does the same for the matrix-pipe utilisation counters, which the
bench line reports as ``roofline.mfma_util_counters`` (per cent of GPU-active
cycles the matrix pipes were busy) while the summary matches the kernel source.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16) and % MFMA peak; decode KV-read HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 matrix-core peak
PEAK_FP32_TFLOPS = 157.3    # dense fp32 matrix-core peak
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0
PEAK_CLOCK_MHZ = 2400.0     # engine clock the published matrix-core peaks assume
# vector issue: 256 CUs x 4 SIMDs x 16 lanes per clock x 2.4 GHz, in lane
# issue slots per second (no packed fp32 arithmetic is used)
PEAK_VALU_TSLOTS = 256 * 4 * 16 * 2.4e9 / 1e12
# vector issue slots per allowed (query, key) pair in the softmax: one fma
# (scale, subtract the reference max), one exp2 (v_exp_f32 issues at half the
# fma rate: two slots), one add (row sum), half a bf16 pack (two per
# v_cvt_pk_bf16_f32); the count does not depend on d
VALU_SLOTS_PER_PAIR = 4.5
PREFILL_KERNEL_SRC = os.path.join(ROOT, "io_aware_exact_19_amd", "csrc", "fa_prefill.hip")
DECODE_KERNEL_SRC = os.path.join(ROOT, "io_aware_exact_19_amd", "csrc", "fa_decode.hip")
FP8_KERNEL_SRC = os.path.join(ROOT, "io_aware_exact_19_amd", "csrc", "fa_fp8.hip")
BACKWARD_KERNEL_SRC = [os.path.join(ROOT, "io_aware_exact_19_amd", "csrc", f)
                       for f in ("fa_backward.hip", "fa_backward_dq.hip")]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "prefill_bf16_d128_b4h16n2048_hbm_traffic.txt")
DECODE_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "decode_bf16_b64h32_hbm_traffic.txt")
MFMA_SUMMARY = os.path.join(ROOT, "profiles", "prefill_bf16_d128_b4h16n2048_mfma_util.txt")
# the headline kernel as rocprofv3 names it (template arguments: head dim,
# varlen, KV cache)
HEADLINE_KERNEL = "fwd_bf16_kernel<128, false, false>"
COPY_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _local_includes(path, seen):
    """``path`` and every header it pulls in with #include "..." from its own
    directory, depth first, each once."""
    path = os.path.abspath(path)
    if path in seen or not os.path.exists(path):
        return
    seen.append(path)
    with open(path) as f:
        for line in f:
            t = line.strip()
            if t.startswith("#include") and '"' in t:
                _local_includes(os.path.join(os.path.dirname(path), t.split('"')[1]), seen)


def sha256(path):
    """Digest of a kernel source (or a list of them) together with the local
    headers it includes (a change to a shared helper changes the compiled
    kernel too)."""
    files = []
    for p in ([path] if isinstance(path, str) else path):
        _local_includes(p, files)
    h = hashlib.sha256()
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def pairs_dense(n_q, n_k, causal, window):
    """Allowed (query, key) pairs of one head, closed form per row."""
    delta = n_k - n_q
    tot = 0
    for i in range(n_q):
        hi = min(n_k - 1, i + delta) if causal else n_k - 1
        lo = max(0, i + delta - window) if window >= 0 else 0
        tot += max(0, hi - lo + 1)
    return tot


# ------------------------------------------------------------- workloads


class Workload:
    """Inputs resident on the GPU plus a launch closure and its work figure."""

    def __init__(self, name, launch, work, unit, peak, bound, dtype, config):
        self.name, self.launch, self.work, self.unit = name, launch, work, unit
        self.peak, self.bound, self.dtype, self.config = peak, bound, dtype, config


def make_dense(torch, fa, inputs, configs, cfg, causal=None, dtype_name="bf16"):
    B, H, N, d = cfg["batch"], cfg["heads"], cfg["seqlen"], cfg["d"]
    causal = cfg["causal"] if causal is None else causal
    W = cfg["window_left"]
    dt = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    q, k, v = (x.cuda() for x in inputs.dense_qkv(B, N, N, H, d, cfg["seed"], dt))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    s = configs.default_scale(d)
    fn = fa.fa_fwd if dtype_name == "bf16" else fa.fa_fwd_fp32
    stream = torch.cuda.current_stream()

    def launch():
        st = fn(q, k, v, o, lse, B, H, N, N, d, s, int(causal), W, None, None, stream)
        if st != 0:
            raise fa.FAError(st, "fa_fwd")

    flops = 4 * d * H * B * pairs_dense(N, N, causal, W)
    peak = PEAK_BF16_TFLOPS if dtype_name == "bf16" else PEAK_FP32_TFLOPS
    name = cfg["name"].replace("_causal", "") + ("_causal" if causal else "")
    conf = dict(workload=name, batch=B, heads=H, seqlen=N, d=d, causal=bool(causal),
                window_left=W)
    return Workload(name, launch, flops, "TFLOP/s", peak, "mfma", dtype_name, conf)


def make_varlen(torch, fa, inputs, configs, cfg):
    lens = inputs.lengths(cfg["nseq"], cfg["len_lo"], cfg["len_hi"], cfg["seed"])
    cu = inputs.cu_seqlens(lens).cuda()
    H, d, W = cfg["heads"], cfg["d"], cfg["window_left"]
    q, k, v = (x.cuda() for x in inputs.varlen_qkv(lens, H, d, cfg["seed"]))
    o = torch.empty_like(q)
    total = int(lens.sum())
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    mx = int(lens.max())
    s = configs.default_scale(d)
    stream = torch.cuda.current_stream()

    def launch():
        st = fa.fa_fwd(q, k, v, o, lse, len(lens), H, mx, mx, d, s, 1, W, cu, cu, stream)
        if st != 0:
            raise fa.FAError(st, "fa_fwd varlen")

    pairs = sum(pairs_dense(int(n), int(n), True, W) for n in lens)
    conf = dict(workload=cfg["name"], nseq=len(lens), total_tokens=total, heads=H, d=d,
                causal=True, window_left=W, lengths=[int(x) for x in lens])
    return Workload(cfg["name"], launch, 4 * d * H * pairs, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma",
                    "bf16", conf)


def make_decode(torch, fa, inputs, configs, cfg):
    B, H, d, L, chunk = cfg["batch"], cfg["heads"], cfg["d"], cfg["max_len"], cfg["chunk"]
    lens = inputs.lengths(B, cfg["len_lo"], cfg["len_hi"], cfg["seed"]).to(torch.int32)
    kc = inputs.decode_cache(B, L, H, d, lens, cfg["seed"], "cuda", "k")
    vc = inputs.decode_cache(B, L, H, d, lens, cfg["seed"], "cuda", "v")
    q = inputs.normal((B, 1, H, d), inputs.subseed(cfg["seed"], "q")).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device="cuda")
    sl = lens.cuda()
    need = fa.fa_decode_workspace_size(B, H, L, d, chunk)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = configs.default_scale(d)
    stream = torch.cuda.current_stream()

    def launch():
        st = fa.fa_decode(q, kc, vc, sl, o, lse, B, H, L, d, s, chunk, ws, need, stream)
        if st != 0:
            raise fa.FAError(st, "fa_decode")

    # algorithmic bytes: every valid K and V row once, plus q in and o out
    kv_bytes = int(lens.sum()) * H * d * 2 * 2
    byts = kv_bytes + 2 * B * H * d * 2
    conf = dict(workload=cfg["name"], batch=B, heads=H, d=d, max_len=L, chunk=chunk,
                kv_rows=int(lens.sum()), kv_bytes=kv_bytes)
    w = Workload(cfg["name"], launch, byts, "GB/s", PEAK_HBM_GBS, "hbm", "bf16", conf)
    w.tensors = (kc, vc)
    return w


def make_kvcache(torch, fa, inputs, configs, cfg):
    """Chunked prefill: n_new new tokens per sequence against its KV cache."""
    B, H, d, L, n = cfg["batch"], cfg["heads"], cfg["d"], cfg["max_len"], cfg["n_new"]
    lens = inputs.lengths(B, cfg["len_lo"], cfg["len_hi"], cfg["seed"]).to(torch.int32)
    kc = inputs.decode_cache(B, L, H, d, lens, cfg["seed"], "cuda", "k")
    vc = inputs.decode_cache(B, L, H, d, lens, cfg["seed"], "cuda", "v")
    q = inputs.normal((B, n, H, d), inputs.subseed(cfg["seed"], "q")).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((B, H, n), dtype=torch.float32, device="cuda")
    sl = lens.cuda()
    s = configs.default_scale(d)
    stream = torch.cuda.current_stream()

    def launch():
        st = fa.fa_fwd_kvcache(q, kc, vc, sl, o, lse, B, H, n, L, d, s, int(cfg["causal"]), -1,
                               stream)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_kvcache")

    # allowed pairs: query i of sequence b sees keys 0 .. L_b - n + i (bottom-right causal)
    pairs = sum(n * (int(Lb) - n) + n * (n + 1) // 2 for Lb in lens.tolist())
    conf = dict(workload=cfg["name"], batch=B, heads=H, d=d, n_new=n, max_len=L,
                lengths=[int(x) for x in lens.tolist()])
    w = Workload(cfg["name"], launch, 4 * d * H * pairs, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma",
                 "bf16", conf)
    w.tensors = (kc, vc)
    return w


def make_backward(torch, fa, inputs, configs, cfg, causal=False):
    """dQ, dK, dV of the headline shape from o and lse of one forward call."""
    B, H, N, d = cfg["batch"], cfg["heads"], cfg["seqlen"], cfg["d"]
    q, k, v = (x.cuda() for x in inputs.dense_qkv(B, N, N, H, d, cfg["seed"]))
    do = inputs.normal((B, N, H, d), inputs.subseed(cfg["seed"], "dout")).cuda()
    s = configs.default_scale(d)
    o, lse = fa.attention(q, k, v, scale=s, causal=causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    need = fa.fa_bwd_workspace_size(B, H, N)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        st = fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, B, H, N, N, d, s, int(causal), -1, ws, need,
                       stream)
        if st != 0:
            raise fa.FAError(st, "fa_bwd")

    pairs = N * (N + 1) // 2 if causal else N * N
    name = f"backward_bf16_b{B}_h{H}_n{N}_d{d}" + ("_causal" if causal else "")
    # the usual count: 2.5x the forward (score recompute, dV, dP, dQ, dK products)
    conf = dict(workload=name, batch=B, heads=H, seqlen=N, d=d, causal=causal,
                flops="2.5 x forward (5 products of 2 N^2 d per head)")
    w = Workload(name, launch, 10 * d * H * B * pairs, "TFLOP/s", PEAK_BF16_TFLOPS, "mfma", "bf16",
                 conf)
    w.tensors = (q, k, v, do, o, lse)
    return w


def make_fp8(torch, fa, inputs, configs, cfg, causal=False):
    """The headline shape on e4m3 inputs with per-(batch, head) factors."""
    B, H, N, d = cfg["batch"], cfg["heads"], cfg["seqlen"], cfg["d"]
    q8, k8, v8, dq, dk, dv = (x.cuda() for x in inputs.fp8_qkv(B, N, N, H, d, cfg["seed"]))
    o = torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    s = configs.default_scale(d)
    stream = torch.cuda.current_stream()

    def launch():
        st = fa.fa_fwd_fp8(q8, k8, v8, o, lse, dq, dk, dv, B, H, N, N, d, s, int(causal), -1,
                           stream)
        if st != 0:
            raise fa.FAError(st, "fa_fwd_fp8")

    pairs = N * (N + 1) // 2 if causal else N * N
    name = f"fp8_e4m3_b{B}_h{H}_n{N}_d{d}" + ("_causal" if causal else "")
    conf = dict(workload=name, batch=B, heads=H, seqlen=N, d=d, causal=causal,
                inputs="e4m3 codes, one factor per (batch, head)", output="bf16")
    w = Workload(name, launch, 4 * d * H * B * pairs, "TFLOP/s", PEAK_FP8_TFLOPS, "mfma",
                 "fp8-e4m3", conf)
    w.tensors = (q8, k8, v8, dq, dk, dv)
    return w


# ---------------------------------------------------------------- clock


class ClockSampler:
    """Engine (graphics) clock of the GPU that torch's device 0 is, from the
    GPU metrics table that amdsmi reads: the per-XCD current clocks averaged
    over the XCDs, and the socket power.  The firmware refreshes that table
    only every few hundred milliseconds, so a background thread polls it and
    keeps each distinct table taken while the graphics engine was busy
    (average activity >= 80 %).  Read-only queries; any failure leaves the
    snapshots empty and names the reason."""

    def __init__(self, torch, period_s=0.02):
        import threading

        self.period_s = period_s
        self.snapshots = []        # (MHz averaged over the XCDs, socket W)
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._h = None
        try:
            import amdsmi

            self._amdsmi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            props = torch.cuda.get_device_properties(0)
            want = (int(getattr(props, "pci_domain_id", 0)), int(getattr(props, "pci_bus_id", -1)))
            for h in handles:
                dom, bus = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[:2]
                if (int(dom, 16), int(bus, 16)) == want:
                    self._h = h
            if self._h is None and len(handles) == 1:
                self._h = handles[0]
            if self._h is None:
                self.error = f"no amdsmi device with PCI domain/bus {want}"
        except Exception as e:  # noqa: BLE001 - report, never fail the bench
            self.error = f"amdsmi unavailable: {e}"

    @staticmethod
    def _num(x):
        return float(x) if isinstance(x, (int, float)) else None

    def _read(self):
        """(key identifying the table, MHz, W) or None when the table was not
        taken under load."""
        m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        act = self._num(m.get("average_gfx_activity"))
        if act is None or act < 80:
            return None
        xs = m.get("current_gfxclks")
        xs = [float(x) for x in xs if isinstance(x, (int, float)) and x > 0] \
            if isinstance(xs, list) else []
        mhz = sum(xs) / len(xs) if xs else self._num(m.get("current_gfxclk"))
        if mhz is None:
            return None
        key = (m.get("gfx_activity_acc"), tuple(xs), m.get("current_socket_power"))
        return key, mhz, self._num(m.get("current_socket_power"))

    def _run(self):
        seen = set()
        while not self._stop.is_set():
            try:
                r = self._read()
            except Exception as e:  # noqa: BLE001
                self.error = f"metrics read failed: {e}"
                return
            if r is not None and r[0] not in seen:
                seen.add(r[0])
                self.snapshots.append((r[1], r[2]))
            self._stop.wait(self.period_s)

    def start(self):
        import threading

        if self._h is None:
            return self
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        """Stop; returns (median MHz, median W, number of snapshots) or
        (None, None, 0)."""
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=2.0)
        if not self.snapshots:
            if self.error is None:
                self.error = "no metrics table taken under load"
            return None, None, 0
        mhz = statistics.median(x for x, _ in self.snapshots)
        ws = [w for _, w in self.snapshots if w is not None]
        return mhz, (statistics.median(ws) if ws else None), len(self.snapshots)


def measure_clock(torch, w, seconds):
    """Run ``w`` back to back for ``seconds`` while the clock sampler polls;
    returns (MHz, W, snapshots, error)."""
    clock = ClockSampler(torch).start()
    settle(torch, w, seconds * 1e3)
    mhz, watts, n = clock.stop()
    return mhz, watts, n, clock.error


# ---------------------------------------------------------------- timing


def settle(torch, w, ms):
    """Launch the workload back to back for ``ms`` milliseconds of wall time.

    The engine clock of an idle GPU ramps up over the first few tens of
    milliseconds of sustained load (measured: the first 40 launches of the
    headline workload ran ~15 % slower than launches 50 ms later), so a short
    warmup alone would time the ramp, not the kernel."""
    t_end = time.perf_counter() + ms * 1e-3
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(4):
            w.launch()
        torch.cuda.synchronize()
        n += 4
    return n


def time_launches(torch, w, steps, warmup, settle_ms=0.0):
    """Let the clock settle, warm up, then time exactly ``steps`` back-to-back
    launches between two device synchronisations: wall clock, and one pair of
    HIP events on the launch stream around the same region (mean launch
    duration = event time / steps).  Events recorded around every launch
    would add two queue packets per step (measured: +7 us of wall time and
    +2 us of event time per 130 us launch), so the spread comes from a
    second pass after the timed one, event pairs around chunks of launches.
    Returns (wall ms per step, event ms per step, [fastest, slowest] chunk's
    ms per launch); a chunk carries its own event overhead, so on short
    kernels even the fastest chunk can sit above the timed mean."""
    if settle_ms > 0:
        settle(torch, w, settle_ms)
    for _ in range(warmup):
        w.launch()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        w.launch()
    end.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / steps
    event_ms = start.elapsed_time(end) / steps
    # spread (not part of the timed region): chunks of up to 10 launches
    chunk = max(1, min(10, steps // 2))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for i in range(5):
        starts[i].record()
        for _ in range(chunk):
            w.launch()
        ends[i].record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) / chunk for a, b in zip(starts, ends)]  # ms per launch
    return wall_ms, event_ms, [round(min(per), 5), round(max(per), 5)]


def time_evicted(torch, w, launches=40, warmup=10, evict_bytes=1 << 30):
    """Median launch time with a 1 GiB buffer written before every launch, so
    the inputs start each launch outside the last-level cache (256 MB on
    MI355X); event pairs around each launch alone, the buffer writes
    outside them; the first ``warmup`` pairs are not counted."""
    junk = torch.empty(evict_bytes, dtype=torch.uint8, device="cuda")
    pairs = []
    for i in range(warmup + launches):
        junk.fill_(i & 255)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        w.launch()
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    del junk
    return statistics.median(a.elapsed_time(b) for a, b in pairs[warmup:])


# B4 H16 d128 bf16 non-causal prefill at these lengths: 1 to 8 query tiles
# of 256 rows per workgroup of the persistent grid (256 workgroups), each
# tile N / 64 key steps long
SWEEP_N = (1024, 2048, 3072, 4096, 6144, 8192)
SWEEP_ROWS_PER_ITEM = 256
SWEEP_WGS = 256
SWEEP_KEYS_PER_STEP = 64
# matrix cycles of one key step on one SIMD: two waves (one per lock-step
# group) x 32 products of 32x32x16 at 32 cycles each
SWEEP_MFMA_CYCLES_PER_STEP = 2 * 32 * 32


def profile_sweep(torch, fa, inputs, configs, args):
    """The headline shape at the lengths of SWEEP_N, one after another: for
    each, the engine clock while it runs back to back for --clock-s seconds,
    then settled, warmed up and timed like a bench workload.  Logs each
    shape's clock, launch count and the position of its timed launches, so
    that a kernel trace of the run can be split by shape."""
    for n in SWEEP_N:
        cfg = dict(configs.PREFILL_2K, seqlen=n, name=f"dense_bf16_b4_h16_n{n}_d128")
        w = make_dense(torch, fa, inputs, configs, cfg, False)
        count = [0]
        base = w.launch

        def counted(base=base, count=count):
            count[0] += 1
            base()

        w.launch = counted
        mhz, watts, snaps, err = measure_clock(torch, w, args.clock_s)
        log(f"[sweep] clock n={n} mhz={mhz} socket_w={watts} snapshots={snaps} error={err}")
        if args.settle_ms > 0:
            settle(torch, w, args.settle_ms)
        for _ in range(args.warmup):
            w.launch()
        first = count[0]
        _, mean_ms, _ = time_launches(torch, w, args.steps, 0, 0.0)
        log(f"[sweep] n={n} launches={count[0]} timed_first={first} timed={args.steps} "
            f"event_mean_ms={mean_ms:.5f} tflops={rate(w, mean_ms):.2f}")
        del w
        torch.cuda.empty_cache()
    return 0


def sweep_summary(kt_dir, log_path, out_path, cmd):
    """Split the kernel trace of a ``--profile-target prefill_sweep`` run by
    shape, take each shape's mean duration over its timed launches, turn it
    into engine cycles with the clock sampled on that shape, and fit
    cycles = steps * t + items * x + c (per workgroup: steps of 64 keys,
    query tiles).  This splits the N = 2048 launch's fraction of the
    published peak into clock / 2.4 GHz, the share of its cycles spent in the
    key loop, and the matrix pipe's share of a loop step's cycles."""
    import numpy as np

    rows = []
    for path in glob.glob(os.path.join(kt_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            rows.extend(r for r in csv.DictReader(f)
                        if HEADLINE_KERNEL in r["Kernel_Name"])
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    blocks, clocks = [], {}
    with open(log_path) as f:
        for line in f:
            if not line.startswith("[sweep]"):
                continue
            kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
            if line.startswith("[sweep] clock"):
                clocks[int(kv["n"])] = kv
            else:
                blocks.append({k: float(v) for k, v in kv.items()})
    total = sum(int(b["launches"]) for b in blocks)
    if total != len(rows):
        raise SystemExit(f"trace holds {len(rows)} prefill dispatches, the log names {total}")
    pos, pts = 0, []
    for b in blocks:
        n = int(b["n"])
        lo = pos + int(b["timed_first"])
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in rows[lo:lo + int(b["timed"])]]
        pos += int(b["launches"])
        items = 4 * 16 * n // SWEEP_ROWS_PER_ITEM // SWEEP_WGS
        steps = items * n // SWEEP_KEYS_PER_STEP
        ck = clocks.get(n, {})
        mhz = float(ck["mhz"]) if ck.get("mhz") not in (None, "None") else None
        if mhz is None:
            raise SystemExit(f"no engine clock for N = {n}: {ck.get('error')}")
        mean = statistics.mean(d)
        pts.append(dict(n=n, steps=steps, items=items, mean=mean, median=statistics.median(d),
                        event=b["event_mean_ms"] * 1e3, mhz=mhz, watts=ck.get("socket_w"),
                        cycles=mean * mhz))
    a = np.array([[p["steps"], p["items"], 1.0] for p in pts])
    y = np.array([p["cycles"] for p in pts])
    (t, x, c), *_ = np.linalg.lstsq(a, y, rcond=None)
    fit = a @ np.array([t, x, c])
    lines = ["# rocprofv3 kernel trace: bf16 prefill B4 H16 d128 non-causal at N = "
             + " / ".join(str(n) for n in SWEEP_N) + ", persistent grid of 256 workgroups",
             f"command: {cmd}",
             "(per shape: the timed launches only, located by the launch counts the run logged;",
             " clock: amdsmi, that shape back to back for a few seconds before its timing)",
             "",
             f"{'N':>6s} {'steps/WG':>9s} {'items/WG':>9s} {'trace_mean_us':>14s} "
             f"{'trace_median_us':>16s} {'event_mean_us':>14s} {'clock_mhz':>10s} {'socket_w':>9s} "
             f"{'kcycles':>9s} {'fit_kcycles':>12s}"]
    for p, fv in zip(pts, fit):
        lines.append(f"{p['n']:6d} {p['steps']:9d} {p['items']:9d} {p['mean']:14.2f} "
                     f"{p['median']:16.2f} {p['event']:14.2f} {p['mhz']:10.1f} {str(p['watts']):>9s} "
                     f"{p['cycles'] / 1e3:9.2f} {fv / 1e3:12.2f}")
    lines += ["",
              "least-squares fit of launch cycles = steps * t + items * x + c:",
              f"  t_cycles_per_step: {t:.0f}",
              f"  x_cycles_per_item: {x:.0f}",
              f"  c_cycles_per_launch: {c:.0f}",
              f"  max_residual_pct: {100 * float(np.max(np.abs(fit - y) / y)):.2f}"]
    n2 = next(p for p in pts if p["n"] == 2048)
    loop_share = n2["steps"] * t / n2["cycles"]
    occ = SWEEP_MFMA_CYCLES_PER_STEP / t
    # 256 CUs x 4 SIMDs x 1024 FLOP per cycle at 2.4 GHz is 2516.6 TFLOP/s,
    # published rounded down to 2500
    rounding = 256 * 4 * 1024 * PEAK_CLOCK_MHZ * 1e6 / 1e12 / PEAK_BF16_TFLOPS
    frac = (4 * 128 * 4 * 16 * 2048 * 2048) / (n2["mean"] * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
    lines += ["decomposition of the N = 2048 launch:",
              f"  frac_of_2500_tflops: {frac:.4f}",
              f"  clock_factor (clock / 2400 MHz): {n2['mhz'] / PEAK_CLOCK_MHZ:.4f}",
              f"  loop_share (steps * t / launch cycles): {loop_share:.4f}",
              f"  loop_mfma_occupancy ({SWEEP_MFMA_CYCLES_PER_STEP} / t): {occ:.4f}",
              f"  peak_rounding (2516.6 / 2500): {rounding:.4f}",
              f"  product: {n2['mhz'] / PEAK_CLOCK_MHZ * loop_share * occ * rounding:.4f}",
              f"kernel_source_sha256: {sha256(PREFILL_KERNEL_SRC)}"]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def rate(w, ms):
    scale = 1e12 if w.unit == "TFLOP/s" else 1e9
    return w.work / (ms * 1e-3) / scale


def read_traffic(summary, src):
    """HBM bytes per launch from a committed counter summary, or None when the
    summary is absent or was taken on another version of the kernel source."""
    if not os.path.exists(summary):
        return None
    vals = {}
    with open(summary) as f:
        for line in f:
            if ":" in line:
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256") != sha256(src):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(cfg):
    """The fp64 oracle, as it stands, timed on this host: every (batch, head)
    slice of the headline workload (the ``value``), then a bounded sample of
    each of the other workloads (``per_workload``), each rate against the same
    algorithmic work as the GPU figure (FLOPs of allowed pairs; for decode,
    the K/V bytes of the valid cache rows).  Inputs are generated outside the
    timed calls."""
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from io_aware_exact_19_amd import configs, inputs

    def f64(t):
        return t.float().double().numpy()

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    B, H, N, d = cfg["batch"], cfg["heads"], cfg["seqlen"], cfg["d"]
    q, k, v = (f64(x) for x in inputs.dense_qkv(B, N, N, H, d, cfg["seed"]))
    sc = configs.default_scale(d)
    dt = timed(lambda: oracle.attention_dense(q, k, v, sc, False, -1))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    flops = 4 * d * H * B * N * N
    out = dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=threads, kind="oracle",
               sample=f"all {B * H} (batch, head) slices of the B{B} H{H} N{N} d{d} non-causal "
                      f"workload once: {dt:.2f} s, fp64, score matrix materialised",
               seconds=round(dt, 3), host_cpus=len(os.sched_getaffinity(0)))

    per = []

    def add(workload, sample, seconds, work, unit):
        scale = 1e9
        per.append(dict(workload=workload, sample=sample, seconds=round(seconds, 5),
                        value=round(work / seconds / scale, 3), unit=unit))
        log(f"[bench] oracle {workload}: {seconds:.4f} s, {work / seconds / scale:.2f} {unit}")

    # small fp32 workload, whole
    c = configs.SMALL_FP32
    n, hh, dd = c["seqlen"], c["heads"], c["d"]
    qs, ks, vs = (x.double().numpy()
                  for x in inputs.dense_qkv(c["batch"], n, n, hh, dd, c["seed"], torch.float32))
    t = timed(lambda: oracle.attention_dense(qs, ks, vs, configs.default_scale(dd), False, -1))
    add(c["name"], "whole workload", t, 4 * dd * hh * c["batch"] * n * n, "GFLOP/s")

    # headline shape, causal: every slice (the oracle masks the full matrix)
    t = timed(lambda: oracle.attention_dense(q, k, v, sc, True, -1))
    add(cfg["name"] + "_causal", f"all {B * H} slices", t,
        4 * d * H * B * pairs_dense(N, N, True, -1), "GFLOP/s")
    del q, k, v

    # 8000-token causal prompt: one head of 32
    c = configs.LONG_8K
    n, dd = c["seqlen"], c["d"]
    ql, kl, vl = (f64(x[:, :, :1]) for x in inputs.dense_qkv(1, n, n, 1, dd, c["seed"]))
    t = timed(lambda: oracle.attention_dense(ql, kl, vl, configs.default_scale(dd), True, -1))
    add(c["name"], f"head 0 of {c['heads']}", t, 4 * dd * pairs_dense(n, n, True, -1), "GFLOP/s")
    del ql, kl, vl

    # packed batch: one head of 16, every sequence
    c = configs.VARLEN
    lens = inputs.lengths(c["nseq"], c["len_lo"], c["len_hi"], c["seed"])
    cu = inputs.cu_seqlens(lens).numpy()
    qv, kv, vv = (f64(x[:, :1]) for x in inputs.varlen_qkv(lens, 1, c["d"], c["seed"]))
    t = timed(lambda: oracle.attention_varlen(qv, kv, vv, cu, cu, configs.default_scale(c["d"]),
                                              True, c["window_left"]))
    pairs = sum(pairs_dense(int(x), int(x), True, c["window_left"]) for x in lens)
    add(c["name"], f"head 0 of {c['heads']}, all {c['nseq']} sequences", t, 4 * c["d"] * pairs,
        "GFLOP/s")
    del qv, kv, vv

    # decode: all heads of the 8 first sequences (their valid cache rows drawn
    # on the host: same shapes and distribution as the GPU workload)
    c = configs.DECODE
    lens = inputs.lengths(c["batch"], c["len_lo"], c["len_hi"], c["seed"])[:8]
    hh, dd = c["heads"], c["d"]
    qd = f64(inputs.normal((8, 1, hh, dd), inputs.subseed(c["seed"], "q")))
    tot, byts = 0.0, 0
    for b in range(8):
        nb = int(lens[b])
        kc = f64(inputs.normal((1, nb, hh, dd), inputs.subseed(c["seed"], "k", b)))
        vc = f64(inputs.normal((1, nb, hh, dd), inputs.subseed(c["seed"], "v", b)))
        tot += timed(lambda: oracle.attention_decode(qd[b:b + 1], kc, vc, [nb],
                                                     configs.default_scale(dd)))
        byts += nb * hh * dd * 2 * 2
    add(c["name"], f"all {hh} heads of 8 of {c['batch']} sequences", tot, byts, "GB/s")
    out["per_workload"] = per
    return out


# ----------------------------------------------------- counter summaries


def _pmc_rows(d):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_kernel(rows, counter):
    """Counter values per kernel name, in dispatch order."""
    out = {}
    rows = sorted(rows, key=lambda r: int(r.get("Dispatch_Id", 0)))
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "")
        out.setdefault(name, []).append(float(r["Counter_Value"]))
    return out


def pmc_summary(fetch_dir, write_dir, target, out_path, cmd):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the target kernel,
    each scaled by what the counter reads for a device copy of COPY_BYTES."""
    fetch = _per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = _per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")

    def pick(d, key):
        names = [n for n in d if key in n]
        if not names:
            raise SystemExit(f"no kernel matching {key!r} in {sorted(d)}")
        return names[0], d[names[0]]

    kname = "fwd_bf16_kernel" if target.startswith("prefill") else "decode_split_kernel"
    fk, fvals = pick(fetch, kname)
    _, wvals = pick(write, kname)
    # the calibration copies are the last three device-to-device copies of the run
    ck, cf = pick(fetch, "copyBuffer")
    _, cw = pick(write, ck)
    cf, cw = cf[-3:], cw[-3:]
    f_kib, w_kib = statistics.median(fvals), statistics.median(wvals)
    cf_kib, cw_kib = statistics.median(cf), statistics.median(cw)
    f_scale = COPY_BYTES / (cf_kib * 1024.0)
    w_scale = COPY_BYTES / (cw_kib * 1024.0)
    extra = []
    if target.startswith("decode"):
        cb = [n for n in fetch if "decode_combine_kernel" in n]
        if cb:
            extra.append(("combine_fetch_kib_per_dispatch", statistics.median(fetch[cb[0]])))
    hbm = f_kib * 1024.0 * f_scale + w_kib * 1024.0 * w_scale
    src = PREFILL_KERNEL_SRC if target.startswith("prefill") else DECODE_KERNEL_SRC
    lines = [
        f"# HBM traffic of {fk.replace('void fa::(anonymous namespace)::', '').split('(fa::')[0]}"
        f" ({target} workload) from two rocprofv3 --pmc passes",
        f"command: {cmd}",
        f"kernel: {fk}",
        f"dispatches_fetch: {len(fvals)}",
        f"dispatches_write: {len(wvals)}",
        f"fetch_kib_per_dispatch: {f_kib:.1f}",
        f"write_kib_per_dispatch: {w_kib:.1f}",
        f"copy_kernel: {ck}",
        f"copy_bytes_read_and_written: {COPY_BYTES}",
        f"copy_fetch_kib: {cf_kib:.1f}",
        f"copy_write_kib: {cw_kib:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        *[f"{k}: {v:.1f}" for k, v in extra],
        f"hbm_bytes_per_launch: {hbm:.0f}",
        f"kernel_source_sha256: {sha256(src)}",
    ]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES",
                 "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE")

def _kernel_short(name):
    name = name.replace("void ", "", 1) if name.startswith("void ") else name
    return name.replace("fa::(anonymous namespace)::", "").split("(")[0]


def _agent_info(d):
    """(shader arrays, SIMDs) of the GPU agent from a rocprofv3 output dir."""
    for path in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if str(r.get("Name", "")).startswith("gfx"):
                    return int(r.get("Array_Count") or 0), int(r.get("Simd_Count") or 0)
    return 0, 0


def mfma_summary(util_dir, raw_dir, target, out_path, cmd, algo_flops):
    """Matrix-pipe utilisation of every library kernel of one workload from two
    rocprofv3 --pmc passes: the derived MfmaUtil (MFMA busy cycles over all
    SIMDs / (GPU active cycles x SIMDs)), and raw counters, medians per
    dispatch (GRBM_GUI_ACTIVE comes back summed over the XCDs).

    Clock: the SQ counters come back summed over the shader arrays, and
    SQ_BUSY_CYCLES / arrays / dispatch time is the shader clock the kernel
    ran at (a lower bound: an array stops counting once its XCD has
    drained).  GRBM_GUI_ACTIVE spans the profiler's sampling window around
    the dispatch (11-28 us more than the dispatch at the shader clock,
    whatever the kernel's length), so GRBM_GUI_ACTIVE / XCDs / dispatch time
    overstates the clock and the derived MfmaUtil, which divides by it,
    understates the matrix pipes' busy share.  The summary therefore also
    reports that share against shader cycles: SQ_VALU_MFMA_BUSY_CYCLES /
    (SIMDs x SQ_BUSY_CYCLES / arrays)."""
    util = {}
    for r in _pmc_rows(util_dir):
        if r.get("Counter_Name") == "MfmaUtil" and "fa::" in r.get("Kernel_Name", ""):
            util.setdefault(_kernel_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    raw, dur = {}, {}
    for r in _pmc_rows(raw_dir):
        n = r.get("Kernel_Name", "")
        if "fa::" not in n:
            continue
        k = _kernel_short(n)
        raw.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            dur.setdefault(k, []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    lines = [f"# MFMA utilisation of the {target} workload's kernels from two rocprofv3 --pmc passes",
             f"command: {cmd}",
             f"algorithmic_flops_per_launch: {algo_flops}",
             "(medians over the dispatches of each kernel; the settle launches before the timed"
             " ones are included)"]
    for k in sorted(util):
        med = {c: statistics.median(v) for c, v in raw.get(k, {}).items()}
        lines.append(f"kernel: {k}")
        lines.append(f"  dispatches: {len(util[k])}")
        lines.append(f"  mfma_util_pct: {statistics.median(util[k]):.2f}")
        for c in MFMA_COUNTERS:
            if c in med:
                lines.append(f"  {c}: {med[c]:.0f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
            lines.append(f"  mfma_flops_bf16: {med['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512:.0f}")
        if "SQ_INSTS_VALU_MFMA_MOPS_F8" in med:
            lines.append(f"  mfma_flops_f8: {med['SQ_INSTS_VALU_MFMA_MOPS_F8'] * 512:.0f}")
        if k in dur:
            us = statistics.median(dur[k]) * 1e6
            lines.append(f"  dispatch_us_under_counters: {us:.2f}")
            arrays, simds = _agent_info(raw_dir)
            if arrays and simds and "SQ_BUSY_CYCLES" in med and us > 0:
                shader_cycles = med["SQ_BUSY_CYCLES"] / arrays
                lines.append(f"  shader_arrays: {arrays}  simds: {simds}")
                lines.append(f"  shader_clock_mhz_from_sq_busy: {shader_cycles / us:.1f}")
                if "GRBM_GUI_ACTIVE" in med:
                    lines.append(f"  grbm_gui_active_mhz_per_xcd: {med['GRBM_GUI_ACTIVE'] / 8 / us:.1f}")
                if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
                    busy = 100.0 * med["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * shader_cycles)
                    lines.append(f"  mfma_busy_pct_of_shader_cycles: {busy:.2f}")
    src = (FP8_KERNEL_SRC if target.startswith("fp8") else
           BACKWARD_KERNEL_SRC if target.startswith("backward") else PREFILL_KERNEL_SRC)
    lines.append("kernel_source: " + ", ".join(
        os.path.relpath(p, ROOT) for p in ([src] if isinstance(src, str) else src)))
    lines.append(f"kernel_source_sha256: {sha256(src)}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


ANATOMY_PASSES = (
    ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY",
     "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_MISC"),
    ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_WAIT_INST_LDS",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_SMEM", "SQ_BUSY_CYCLES"),
    ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_BRANCH", "SQ_BUSY_CYCLES"),
)


def anatomy_summary(dirs, target, out_path, cmd):
    """Where each library kernel's waves spend their time, from three
    rocprofv3 --pmc passes (ANATOMY_PASSES), medians per dispatch.

    The SQ counters come back summed over the shader arrays; the wave-state
    ones (SQ_WAVE_CYCLES, SQ_WAIT_*, SQ_ACTIVE_INST_*) count in units of four
    cycles, which the file checks: SQ_WAVE_CYCLES x 4 / (waves x shader
    cycles) is the waves' residency, at most 1.  Each pass is normalised by
    its own SQ_BUSY_CYCLES (shader cycles = SQ_BUSY_CYCLES / arrays)."""
    med, grid = {}, {}
    for i, d in enumerate(dirs):
        vals = {}
        for r in _pmc_rows(d):
            n = r.get("Kernel_Name", "")
            if "fa::" not in n:
                continue
            k = _kernel_short(n)
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
            if r.get("Grid_Size"):
                grid[k] = int(r["Grid_Size"])
        for k, cs in vals.items():
            for c, v in cs.items():
                med.setdefault(k, {})[(i, c)] = statistics.median(v)
    arrays, simds = _agent_info(dirs[0])
    lines = [f"# Wave-state anatomy of the {target} workload's kernels from three rocprofv3 --pmc passes",
             f"command: {cmd}",
             "(medians over the dispatches of each kernel; wave-state counters in units of 4 cycles)"]
    for k in sorted(med):
        m = med[k]

        def get(c, i=None):
            for j in ([i] if i is not None else range(len(dirs))):
                if (j, c) in m:
                    return m[(j, c)], j
            return None, None

        lines.append(f"kernel: {k}")
        waves = grid.get(k, 0) // 64
        lines.append(f"  waves: {waves}")
        for i, names in enumerate(ANATOMY_PASSES):
            for c in names:
                v = m.get((i, c))
                if v is not None:
                    lines.append(f"  pass{i}.{c}: {v:.0f}")
        if not arrays or not simds:
            continue
        wave, _ = get("SQ_WAVE_CYCLES", 0)
        busy0, _ = get("SQ_BUSY_CYCLES", 0)
        if wave and busy0 and waves:
            sc0 = busy0 / arrays
            lines.append(f"  wave_residency (SQ_WAVE_CYCLES x 4 / (waves x shader cycles)): "
                         f"{4 * wave / (waves * sc0):.3f}")
            for c, label in (("SQ_ACTIVE_INST_ANY", "issuing"), ("SQ_WAIT_ANY", "waiting_on_waitcnt"),
                             ("SQ_WAIT_INST_ANY", "waiting_to_issue")):
                v = m.get((0, c))
                if v is not None:
                    lines.append(f"  wave_time_pct.{label}: {100 * v / wave:.1f}")
            for c, label in (("SQ_ACTIVE_INST_VALU", "vector"), ("SQ_ACTIVE_INST_LDS", "lds"),
                             ("SQ_ACTIVE_INST_MISC", "misc")):
                v = m.get((0, c))
                if v is not None:
                    lines.append(f"  simd_issue_pct.{label}: {100 * 4 * v / (simds * sc0):.1f}")
        busy1 = m.get((1, "SQ_BUSY_CYCLES"))
        mf = m.get((1, "SQ_INSTS_MFMA"))
        if busy1 and mf:
            mb = m.get((1, "SQ_VALU_MFMA_BUSY_CYCLES"))
            if mb is not None:
                lines.append(f"  simd_busy_pct.matrix: {100 * mb / (simds * busy1 / arrays):.1f}")
            for c, label in (("SQ_INSTS_VALU", "vector_incl_matrix"), ("SQ_INSTS_LDS", "lds"),
                             ("SQ_INSTS_SALU", "scalar"), ("SQ_INSTS_SMEM", "scalar_mem")):
                v = m.get((1, c))
                if v is not None:
                    lines.append(f"  instructions_per_matrix_product.{label}: {v / mf:.2f}")
        busy2 = m.get((2, "SQ_BUSY_CYCLES"))
        lds = m.get((2, "SQ_LDS_IDX_ACTIVE"))
        if busy2 and lds is not None:
            cus = simds // 4
            lines.append(f"  lds_active_pct (SQ_LDS_IDX_ACTIVE / (CUs x shader cycles)): "
                         f"{100 * lds / (cus * busy2 / arrays):.1f}")
    src = (FP8_KERNEL_SRC if target.startswith("fp8") else
           BACKWARD_KERNEL_SRC if target.startswith("backward") else PREFILL_KERNEL_SRC)
    lines.append("kernel_source: " + ", ".join(
        os.path.relpath(p, ROOT) for p in ([src] if isinstance(src, str) else src)))
    lines.append(f"kernel_source_sha256: {sha256(src)}")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def trace_summary(kt_dir, log_path, target, out_path, cmd, title):
    """The library kernels' rows of a rocprofv3 --kernel-trace --stats run of
    ``--profile-target`` (calls, average / min / max / stddev duration in
    microseconds), with the bench's own event timing from the same run."""
    rows = []
    for path in glob.glob(os.path.join(kt_dir, "**", "*kernel_stats.csv"), recursive=True):
        with open(path) as f:
            rows.extend(r for r in csv.DictReader(f) if "fa::" in r.get("Name", ""))
    prof = []
    if os.path.exists(log_path):
        with open(log_path) as f:
            prof = [ln.strip() for ln in f if ln.startswith("[profile]")]
    lines = [f"# rocprofv3 kernel trace: {title}",
             f"command: {cmd}",
             "(calls include the settle launches that precede the timed ones)",
             "",
             f"{'kernel':64s} {'calls':>7s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
             f"{'stddev_us':>10s}"]
    for r in rows:
        lines.append(f"{_kernel_short(r['Name']):64s} {r['Calls']:>7s} "
                     f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['StdDev']) / 1e3:10.2f}")
    lines += ["", "bench.py's own event timing in the same run:", *prof]
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def read_summary_value(summary, src, kernel, key):
    """A per-kernel value of a committed counter summary, or None when absent
    or taken on another version of the kernel source."""
    if not os.path.exists(summary):
        return None
    vals, cur, sha = {}, None, None
    with open(summary) as f:
        for line in f:
            k, _, val = line.strip().partition(":")
            if k == "kernel":
                cur = val.strip()
            elif k == key and cur:
                vals[cur] = float(val)
            elif k == "kernel_source_sha256":
                sha = val.strip()
    if sha != sha256(src):
        return None
    return vals.get(kernel)


def read_mfma_util(summary, src, kernel):
    """MfmaUtil (per cent) of one kernel from a committed counter summary, or
    None when absent or taken on another version of the kernel source."""
    if not os.path.exists(summary):
        return None
    util, cur, sha = {}, None, None
    with open(summary) as f:
        for line in f:
            key, _, val = line.strip().partition(":")
            if key == "kernel":
                cur = val.strip()
            elif key == "mfma_util_pct" and cur:
                util[cur] = float(val)
            elif key == "kernel_source_sha256":
                sha = val.strip()
    if sha != sha256(src):
        return None
    return util.get(kernel)


# ------------------------------------------------------------------ main


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="back-to-back launches before the warmup steps (engine clock ramp)")
    ap.add_argument("--clock-s", type=float, default=2.5,
                    help="seconds of back-to-back headline launches while the clock is sampled")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--profile-target", default=None,
                    choices=["prefill_2k", "prefill_2k_causal", "long_8k", "varlen", "small_fp32",
                             "decode", "kvcache", "backward", "backward_causal", "fp8",
                             "fp8_causal", "prefill_sweep"])
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--pmc-target", default="prefill_2k")
    ap.add_argument("--pmc-out", default=None)
    ap.add_argument("--pmc-cmd", default="")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("UTIL_DIR", "RAW_DIR"))
    ap.add_argument("--algo-flops", type=int, default=0)
    ap.add_argument("--trace-summary", nargs=2, metavar=("KT_DIR", "LOG"),
                    help="write the kernel-trace summary of a --profile-target run")
    ap.add_argument("--trace-title", default="")
    ap.add_argument("--anatomy-summary", nargs=3, metavar=("DIR_A", "DIR_B", "DIR_C"),
                    help="write the wave-state summary of three --pmc passes (ANATOMY_PASSES)")
    ap.add_argument("--sweep-summary", nargs=2, metavar=("KT_DIR", "LOG"),
                    help="write the length-sweep summary of a --profile-target prefill_sweep run")
    args = ap.parse_args()

    if args.anatomy_summary:
        anatomy_summary(args.anatomy_summary, args.pmc_target, args.pmc_out, args.pmc_cmd)
        return 0

    if args.sweep_summary:
        sweep_summary(args.sweep_summary[0], args.sweep_summary[1], args.pmc_out, args.pmc_cmd)
        return 0

    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.trace_summary[1], args.pmc_target,
                      args.pmc_out, args.pmc_cmd, args.trace_title)
        return 0

    if args.mfma_summary:
        mfma_summary(args.mfma_summary[0], args.mfma_summary[1], args.pmc_target, args.pmc_out,
                     args.pmc_cmd, args.algo_flops)
        return 0

    if args.pmc_summary:
        out = args.pmc_out or (TRAFFIC_SUMMARY if args.pmc_target.startswith("prefill")
                               else DECODE_TRAFFIC_SUMMARY)
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.pmc_target, out, args.pmc_cmd)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("this bench measures one GPU only: the attention forward path is built and "
              "measured on a single MI355X (heads and batch entries shard across GPUs with no "
              "exchange); run it with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import io_aware_exact_19_amd as fa
    from io_aware_exact_19_amd import configs, inputs

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    fa.load_library()
    dev = torch.cuda.get_device_properties(0)
    log(f"[bench] device {dev.name} CUs {dev.multi_processor_count}")

    builders = {
        "prefill_2k": lambda: make_dense(torch, fa, inputs, configs, configs.PREFILL_2K, False),
        "prefill_2k_causal": lambda: make_dense(torch, fa, inputs, configs, configs.PREFILL_2K,
                                                True),
        "long_8k": lambda: make_dense(torch, fa, inputs, configs, configs.LONG_8K),
        "varlen": lambda: make_varlen(torch, fa, inputs, configs, configs.VARLEN),
        "small_fp32": lambda: make_dense(torch, fa, inputs, configs, configs.SMALL_FP32,
                                         dtype_name="f32"),
        "decode": lambda: make_decode(torch, fa, inputs, configs, configs.DECODE),
        "kvcache": lambda: make_kvcache(torch, fa, inputs, configs, configs.KVCACHE),
        "backward": lambda: make_backward(torch, fa, inputs, configs, configs.PREFILL_2K),
        "backward_causal": lambda: make_backward(torch, fa, inputs, configs, configs.PREFILL_2K,
                                                 causal=True),
        "fp8": lambda: make_fp8(torch, fa, inputs, configs, configs.PREFILL_2K),
        "fp8_causal": lambda: make_fp8(torch, fa, inputs, configs, configs.PREFILL_2K, causal=True),
    }

    if args.profile_target == "prefill_sweep":
        return profile_sweep(torch, fa, inputs, configs, args)

    if args.profile_target:
        w = builders[args.profile_target]()
        wall, mean_ms, chunks = time_launches(torch, w, args.steps, args.warmup, args.settle_ms)
        log(f"[profile] {w.name}: {args.steps} launches, mean {mean_ms:.4f} ms, "
            f"{rate(w, mean_ms):.2f} {w.unit}")
        if args.calibrate_copy:
            src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"[profile] copied {COPY_BYTES} bytes x3")
        return 0

    # ---- headline: B4 H16 N2048 d128 bf16 non-causal prefill
    head = builders["prefill_2k"]()
    log(f"[bench] timing {head.name}: settle {args.settle_ms:.0f} ms, warmup {args.warmup}, "
        f"steps {args.steps}")
    wall_ms, mean_ms, chunks = time_launches(torch, head, args.steps, args.warmup, args.settle_ms)
    achieved = rate(head, mean_ms)
    # the engine clock while the same launches run back to back (right after
    # the timed region, same inputs): the firmware's metrics table refreshes
    # only every few hundred milliseconds, too rarely to sample the timed
    # launches themselves
    clock_mhz, clock_w, clock_n, clock_err = measure_clock(torch, head, args.clock_s)
    evicted_ms = time_evicted(torch, head)
    traffic = read_traffic(TRAFFIC_SUMMARY, PREFILL_KERNEL_SRC)
    result = {
        "metric": METRIC,
        "value": round(head.work / (wall_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: i.i.d. N(0,1) bf16 Q/K/V from fixed seeds, inputs resident in HBM",
        "config": dict(head.config, settle_ms=args.settle_ms),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "mfma_util_counters": read_mfma_util(MFMA_SUMMARY, PREFILL_KERNEL_SRC,
                                                 HEADLINE_KERNEL),
            # the same matrix-pipe busy cycles against the shader cycles the
            # counters' own run measured (SQ_BUSY_CYCLES per shader array)
            "mfma_busy_pct_of_shader_cycles": read_summary_value(
                MFMA_SUMMARY, PREFILL_KERNEL_SRC, HEADLINE_KERNEL,
                "mfma_busy_pct_of_shader_cycles"),
            "shader_clock_mhz_counters": read_summary_value(
                MFMA_SUMMARY, PREFILL_KERNEL_SRC, HEADLINE_KERNEL,
                "shader_clock_mhz_from_sq_busy"),
            "kernel": HEADLINE_KERNEL,
            "flops_per_launch": head.work,
            "mean_launch_ms": round(mean_ms, 5),
            "chunk_ms_range": chunks,
            "median_launch_ms_cache_evicted": round(evicted_ms, 5),
            # the published peak assumes the 2.4 GHz maximum engine clock;
            # the same fraction against the peak at the clock measured while
            # this kernel ran back to back
            "clock_mhz": round(clock_mhz, 1) if clock_mhz else None,
            "clock_snapshots": clock_n,
            "socket_power_w": clock_w,
            "clock_source": (f"amdsmi GPU metrics table: current gfx clock averaged over the "
                             f"XCDs, median of the distinct tables taken under load during "
                             f"{args.clock_s:.1f} s of back-to-back launches after the timed "
                             f"region" if clock_mhz else clock_err),
            "peak_at_measured_clock": (round(PEAK_BF16_TFLOPS * clock_mhz / PEAK_CLOCK_MHZ, 1)
                                       if clock_mhz else None),
            "frac_at_measured_clock": (round(achieved / (PEAK_BF16_TFLOPS * clock_mhz /
                                                         PEAK_CLOCK_MHZ), 4)
                                       if clock_mhz else None),
        },
    }
    if clock_mhz:
        log(f"[bench] engine clock {clock_mhz:.0f} MHz, {clock_w} W ({clock_n} metrics tables)")
    log(f"[bench] {head.name}: {result['value']} TFLOP/s wall, kernel {achieved:.1f} TFLOP/s")
    del head
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = []
        for key in ("prefill_2k_causal", "long_8k", "varlen", "small_fp32", "decode", "kvcache",
                    "backward", "backward_causal", "fp8", "fp8_causal"):
            w = builders[key]()
            steps = 20 if key != "decode" else 10
            log(f"[bench] timing {w.name}")
            wall, mean2, chunks2 = time_launches(torch, w, steps, 3, args.settle_ms)
            r = rate(w, mean2)
            entry = {"workload": w.name, "value": round(r, 3), "unit": w.unit,
                     "frac_of_peak": round(r / w.peak, 4), "peak": w.peak, "bound": w.bound,
                     "dtype": w.dtype, "mean_launch_ms": round(mean2, 5),
                     "chunk_ms_range": chunks2, "steps": steps}
            if key == "decode":
                entry["kv_bytes_per_launch"] = w.config["kv_bytes"]
                entry["traffic"] = read_traffic(DECODE_TRAFFIC_SUMMARY, DECODE_KERNEL_SRC)
            if key in ("varlen", "kvcache"):
                entry["lengths"] = w.config["lengths"]
            if key == "varlen":
                # at d = 64 the softmax's vector work per pair equals the
                # matrix work's share, so report the vector-issue bound too
                pairs = w.work / (4 * w.config["d"])
                got = pairs * VALU_SLOTS_PER_PAIR / (mean2 * 1e-3) / 1e12
                entry["valu_roofline"] = {
                    "bound": "alu", "achieved": round(got, 3), "peak": round(PEAK_VALU_TSLOTS, 3),
                    "unit": "T lane-slots/s", "frac": round(got / PEAK_VALU_TSLOTS, 4),
                    "slots_per_pair": VALU_SLOTS_PER_PAIR}
            sec.append(entry)
            log(f"[bench] {w.name}: {r:.2f} {w.unit} ({100 * r / w.peak:.1f}% of peak)")
            del w
            torch.cuda.empty_cache()
        result["secondary"] = sec

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle (headline workload, then a sample of each other one)")
        result["cpu_baseline"] = cpu_baseline(configs.PREFILL_2K)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
