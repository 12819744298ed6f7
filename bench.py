"""Benchmark of the frame-windowed sparse attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload sr720] [--no-cpu-baseline] [--center]

One step is one pass of every stage of the path over one batch of synthetic
input already resident in HBM: the host plan (fsa_plan into pinned memory and
an async copy of its CSR to the device), fsa_bounds (norm array and per-head
eligibility) and fsa_attention. The plan's upload runs on a copy stream into one
of two device plan buffers, so step i + 1's upload overlaps step i's kernels. Consecutive steps rotate over three copies of
q, k, v (more than the 256 MB last-level cache holds at the 720p and 1080p
shapes), so the bounds pass reads from HBM. W untimed steps, then K timed steps
between two device synchronisations. Prints ONE JSON line:

* value = active-block FLOPs (4 D per visible query/key pair) x K / time of the
  K steps, in TFLOP/s, and pct_of_peak against the bf16 dense MFMA peak;
* roofline: fsa_attention (the dominant kernel, MFMA-bound) with its mean
  duration from HIP events recorded on its launch stream around each launch
  (the event after it also marks the plan buffer free for reuse); the
  bounds pass is bracketed by its own events on every fourth timed step
  only, since each event recorded between two kernels holds the stream for
  several microseconds, and is also timed on its own after the timed steps
  (bounds.alone_*: 60 calls back to back over the rotating input copies);
* cpu_baseline: the fp64 oracle (not tuned) timed on four heads of the same
  workload on the host cores, scaled to the same unit;
* check: the last timed step's output on those four heads against that oracle
  run (max-abs, rel-L2 and whether both are within the parity bars), so the
  line shows that the computation it timed is correct;
* roofline.traffic: HBM bytes per launch from the committed rocprofv3
  FETCH_SIZE / WRITE_SIZE passes (profiles/traffic.json), reported only while
  the kernel source still matches the one those counters were taken on.
* two_streams: after the timed steps, 100 steps (after 20 untimed ones) with
  consecutive steps on two streams in turn (own bounds and output buffers per
  stream), timed as a whole: a step's kernels then start on the CUs the
  previous step's attention kernel leaves idle during its last workgroups.
  value, roofline and check come from the sequential steps only.

--kernel pre_attention times fsa_pre_attention alone (workload pre720 unless
another pre-attention workload is named) and prints its own JSON line;
--kernel chain times x -> fsa_pre_attention -> fsa_bounds -> fsa_attention on
the 720p shape.

--groups G splits fsa_attention into G head groups on G streams (the grouped
dense configuration); roofline then covers the span of the grouped launches.

--center runs fsa_bounds with key mean-centring (and fsa_attention with the
resulting key mean); the default is off, as on the headline workload.

Only one GPU is used: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective TFLOP/s on active blocks + % of bf16 MFMA peak, 25k-token SR attn"
# fsa_bounds and fsa_attention are bracketed by timing events on every
# EVENTS_EVERY-th timed step only: an event recorded between two kernels holds
# the stream for a few microseconds, so the other steps record just the plan
# buffer's reuse marker after the attention kernel
EVENTS_EVERY = 4
# after the timed steps, this many bounds calls run back to back on their own
BOUNDS_ALONE = 60
# the two-stream pass: a fixed count of its own (the overlap needs a few steps
# in flight before it reaches its steady state)
TWO_STREAM_STEPS = 100
TWO_STREAM_WARMUP = 20
PEAK_BF16_TFLOPS = 2516.6          # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0             # MI355X HBM3E
KERNEL_SOURCE = os.path.join(ROOT, "frame_windowed_block_amd", "csrc", "fsa_kernels.hip")
PRE_SOURCE = os.path.join(ROOT, "frame_windowed_block_amd", "csrc", "fsa_preattn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_code_digest(source: str = KERNEL_SOURCE) -> str:
    """sha256 of the kernel source with its // comments, trailing blanks and
    empty lines removed: the code the counters were taken on, not its prose."""
    import hashlib
    import re
    lines = []
    with open(source, encoding="utf-8") as fh:
        for line in fh:
            code = re.sub(r"//.*$", "", line.rstrip("\n")).rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def measured_traffic(kernel: str, workload: str, source: str = KERNEL_SOURCE):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    passes (copy-calibrated), or None when they were taken on other kernel code."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)[kernel][workload]
        digest = kernel_code_digest(source)
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if rec.get("kernel_code_sha256") == digest else None


def preroll(step, ms: float) -> tuple[float, int]:
    """Run step(i) for ``ms`` of wall time (the engine clock ramps up under
    load); returns the time taken and the step count."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, i


def plan_flops(info, batch: int, heads: int, head_dim: int) -> int:
    """Active-block FLOPs from the library's own plan: every listed (bq x bk)
    block-head does 2 D FLOPs per (query, key) pair for q.k and 2 D for p.v."""
    return 4 * head_dim * info.block_q * info.block_k * info.nnz * batch * heads


def projection_flops(batch: int, seq_len: int, channels: int, heads: int, head_dim: int) -> int:
    """FLOPs of the q/k/v projection: 2 C per projected feature."""
    return 2 * batch * seq_len * channels * 3 * heads * head_dim


def parse_dpm_mhz(line: str):
    """MHz of one ``pp_dpm_sclk`` line ("1: 1989Mhz *"), or None."""
    import re
    m = re.search(r"(\d+(?:\.\d+)?)\s*[Mm][Hh]z", line)
    return float(m.group(1)) if m else None


class ClockSampler:
    """Engine clock (sclk, MHz) of GPU 0, sampled by a background thread while a
    region runs. The source is the driver's sysfs ``pp_dpm_sclk`` (the level
    marked current), which follows the clock within a fraction of a second;
    amdsmi's clock query is the fallback, but its value is refreshed only about
    once a second, so over a short region it can still show an earlier (even
    idle) clock. Any failure leaves the samples empty and records why; the run
    itself is unaffected."""

    def __init__(self, period_s: float = 0.004):
        self.period = period_s
        self.samples: list[float] = []
        self.error = None
        self.source = None
        self._stop = None
        self._thread = None
        self._smi = None
        self._handle = None
        self._sysfs = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._handle = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as exc:                       # noqa: BLE001
            self.error = f"{type(exc).__name__}: {exc}"
            self._smi = None
        self._sysfs = self._find_sysfs()
        try:
            if self._sysfs is not None and self._read_sysfs() is not None:
                self.source = "sysfs pp_dpm_sclk"
            elif self._smi is not None and self._read_smi() is not None:
                self.source = "amdsmi clock info (refreshed about once a second)"
        except Exception as exc:                       # noqa: BLE001
            self.error = f"{type(exc).__name__}: {exc}"

    def _find_sysfs(self):
        import glob
        paths = []
        if self._smi is not None:
            try:
                bdf = self._smi.amdsmi_get_gpu_device_bdf(self._handle)
                paths.append(f"/sys/bus/pci/devices/{bdf}/pp_dpm_sclk")
            except Exception:                          # noqa: BLE001
                pass
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if len(cards) == 1:                            # the only GPU: no need to match it
            paths.append(cards[0])
        for path in paths:
            if os.path.exists(path):
                return path
        return None

    def _read_sysfs(self):
        with open(self._sysfs) as f:
            for line in f:
                if line.rstrip().endswith("*"):        # e.g. "1: 1989Mhz *"
                    return parse_dpm_mhz(line)
        return None

    def _read_smi(self):
        info = self._smi.amdsmi_get_clock_info(self._handle, self._smi.AmdSmiClkType.GFX)
        clk = info.get("clk")
        return float(clk) if isinstance(clk, (int, float)) else None

    def read(self):
        if self.source is None:
            return None
        return self._read_sysfs() if self.source.startswith("sysfs") else self._read_smi()

    def _loop(self):
        while not self._stop.is_set():
            try:
                c = self.read()
                if c:
                    self.samples.append(c)
            except Exception as exc:                   # noqa: BLE001
                self.error = f"{type(exc).__name__}: {exc}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        self.samples = []
        if self._smi is None:
            return
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._loop, daemon=True)
        self._thread.start()

    def stop(self) -> dict:
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        if not self.samples:
            return {"samples": 0, "error": self.error or "no samples", "source": self.source}
        x = sorted(self.samples)
        return {"samples": len(x), "mean": round(sum(x) / len(x), 1), "min": x[0], "max": x[-1],
                "source": self.source}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preroll-ms", type=float, default=1000.0,
                    help="before the counted warm-up, run steps for this long (wall time) so "
                         "that the engine clock has left its idle state when the timed steps start")
    ap.add_argument("--workload", default="sr720")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's device copy of a MIB-sized buffer 5 times (known bytes "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads of the workload the CPU oracle is timed on")
    ap.add_argument("--copies", type=int, default=3,
                    help="copies of q, k, v that consecutive steps rotate over")
    ap.add_argument("--groups", type=int, default=1,
                    help="run fsa_attention as this many head groups on as many streams "
                         "(roofline then times the span from the bounds to the last group)")
    ap.add_argument("--center", action="store_true",
                    help="mean-centre the keys in fsa_bounds (key_offset workload)")
    ap.add_argument("--kernel", default="attention", choices=["attention", "pre_attention", "chain"],
                    help="pre_attention: time fsa_pre_attention alone on a pre-attention workload "
                         "(default pre720) and print its own JSON line; chain: x -> fused "
                         "pre-attention -> bounds -> attention on the 720p shape, its own JSON line")
    return ap.parse_args()


def cpu_baseline(wl, qc, kc, vc, heads: int):
    """Time the fp64 oracle on the first `heads` heads of batch item 0; returns
    the JSON record and the oracle's output for those heads."""
    import numpy as np

    import oracle
    import synthetic
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:                                  # noqa: BLE001
        threads = os.cpu_count() or 1
    sl = slice(0, heads)
    q, k, v = (synthetic.to_f64(x[:1, sl]) for x in (qc, kc, vc))
    t0 = time.perf_counter()
    o = oracle.attention(q, k, v, wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
    dt = time.perf_counter() - t0
    assert np.isfinite(o).all()
    flops = oracle.active_flops(1, heads, wl.head_dim, wl.frames, wl.tokens_per_frame,
                                wl.window, wl.ref_frame)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batch 0, heads 0..{heads - 1} of {wl.heads}, all {wl.frames} frames "
                      f"({flops:.3e} active FLOPs; dense fp64 masked softmax), {dt:.2f} s wall"}, o


def output_check(got, ref, m2, score_bound, n_keys, head_dim: int, what: str) -> dict:
    """The timed run's bf16 output against the oracle: max-abs and rel-L2 (bar
    5e-3), every element within the oracle's per-element bar (1e-2, raised only
    where bf16 / fp32 arithmetic itself can exceed it)."""
    import numpy as np

    import oracle
    m, r = oracle.max_abs_and_rel_l2(got, ref)
    bar = oracle.element_bar(ref, m2, score_bound, n_keys, head_dim)
    excess = float((np.abs(got - ref) - bar).max())
    ok = bool(excess <= 0.0 and r <= oracle.REL_L2_BAR)
    return {"against": "fp64 oracle", "outputs": what, "max_abs": m, "rel_l2": r,
            "worst_excess_over_element_bar": excess, "elements_with_bar_above_1e-2": int((bar > 1e-2).sum()),
            "within_bars": ok}


def bench_pre_attention(args):
    """fsa_pre_attention alone: normalisation + q/k/v projection + rotary
    embedding + head packing, inputs resident in HBM (rotating over copies of
    x), one JSON line."""
    import numpy as np
    import torch

    import frame_windowed_block_amd as fsa
    import synthetic

    name = args.workload if args.workload in synthetic.PRE_WORKLOADS else "pre720"
    wl = synthetic.PRE_WORKLOADS[name]
    x, gain, w = synthetic.make_pre_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xs = [x.to(dev) for _ in range(max(1, args.copies))]
    # the norm gain is folded into the weight once, as a model load would do
    wd = (w.float() * gain[None, :]).to(torch.bfloat16).to(dev)
    shape = (wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    outs = [torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3)]
    stream = torch.cuda.current_stream()

    def step(i, strm=None, o3=None):
        o3 = outs if o3 is None else o3
        fsa.pre_attention(xs[i % len(xs)], wd, wl.heads, wl.head_dim, q=o3[0], k=o3[1],
                          v=o3[2], stream=stream if strm is None else strm)

    preroll_ms, _ = preroll(step, args.preroll_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    total_ms = t0.elapsed_time(t1)
    # the same calls, consecutive calls on two streams in turn (own outputs)
    pstreams = [stream, torch.cuda.Stream()]
    pouts = [[torch.empty_like(t) for t in outs] for _ in range(2)]
    for i in range(TWO_STREAM_WARMUP):
        step(i, pstreams[i % 2], pouts[i % 2])
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    pstreams[1].wait_event(p0)
    for i in range(TWO_STREAM_STEPS):
        step(i, pstreams[i % 2], pouts[i % 2])
    fin = torch.cuda.Event()
    fin.record(pstreams[1])
    stream.wait_event(fin)
    p1.record(stream)
    torch.cuda.synchronize()
    pipe_ms = p0.elapsed_time(p1) / TWO_STREAM_STEPS
    flops = projection_flops(wl.batch, wl.seq_len, wl.channels, wl.heads, wl.head_dim)
    kbytes = 2 * wl.batch * wl.seq_len * wl.channels + \
        2 * 3 * wl.heads * wl.head_dim * wl.channels + 3 * 2 * wl.batch * wl.heads * wl.seq_len * wl.head_dim
    med = float(np.median(ms))
    value = flops * args.steps / (total_ms * 1e-3) / 1e12
    line = {
        "metric": "fused pre-attention (norm + qkv projection + rotary + head packing) TFLOP/s",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "channels": wl.channels, "heads": wl.heads, "head_dim": wl.head_dim,
                   "flops": flops, "algorithmic_bytes": kbytes, "input_copies": len(xs)},
        "roofline": {
            "kernel": "fsa_pre_attention", "bound": "mfma",
            "achieved": round(flops / (float(ms.mean()) * 1e-3) / 1e12, 3),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(flops / (float(ms.mean()) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("fsa_pre_attention", wl.name, PRE_SOURCE),
            "mean_ms": round(float(ms.mean()), 5), "median_ms": round(med, 5),
            "hbm_gbps_algorithmic": round(kbytes / (med * 1e-3) / 1e9, 1),
        },
    }
    line["timing"] = {"preroll_ms": round(preroll_ms, 1)}
    line["two_streams"] = {"steps": TWO_STREAM_STEPS, "warmup": TWO_STREAM_WARMUP,
                           "ms_per_step": round(pipe_ms, 5),
                           "value": round(flops / (pipe_ms * 1e-3) / 1e12, 3),
                           "note": "the same calls, consecutive calls on two streams in turn"}
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline_pre(wl, x, gain, w)
        # the last timed step's q, k, v against the oracle given the same folded
        # weight (and a unit gain), i.e. the function the kernel computes
        ref = oracle.pre_attention(synthetic.to_f64(x[:1]), np.ones(wl.channels), synthetic.to_f64(wd.cpu()),
                                   wl.heads, wl.head_dim)
        worst = (0.0, 0.0)
        for got, want in zip(outs, ref):
            m, r = oracle.max_abs_and_rel_l2(synthetic.to_f64(got[:1].cpu()), want)
            worst = (max(worst[0], m), max(worst[1], r))
        line["check"] = {"against": "fp64 oracle", "outputs": "q, k, v of batch 0",
                         "max_abs": worst[0], "rel_l2": worst[1], "within_bars": bool(worst[1] <= 5e-3)}
    print(json.dumps(line), flush=True)


def bench_chain(args):
    """The attention layer's hot path end to end on the 720p shape: x [1, N, C]
    -> fsa_pre_attention -> fsa_bounds -> fsa_attention, inputs resident in
    HBM (rotating over copies of x). One JSON line; value = the projection's
    and the attention's algorithmic FLOPs per second of whole steps."""
    import torch

    import frame_windowed_block_amd as fsa
    import synthetic

    pw = synthetic.PRE_WORKLOADS["pre720"]
    aw = synthetic.WORKLOADS["sr720"]
    assert (pw.seq_len, pw.heads, pw.head_dim) == (aw.seq_len, aw.heads, aw.head_dim)
    x, gain, w = synthetic.make_pre_inputs(pw)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xs = [x.to(dev) for _ in range(max(1, args.copies))]
    wd = (w.float() * gain[None, :]).to(torch.bfloat16).to(dev)
    shape = (pw.batch, pw.heads, pw.seq_len, pw.head_dim)
    q, k, v, o = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(4))
    dplan = fsa.DevicePlan(aw.frames, aw.tokens_per_frame, aw.window, aw.ref_frame, device=dev)
    info = dplan.info
    qn = torch.empty(shape[:3], dtype=torch.float32, device=dev)
    km = torch.empty((pw.batch, pw.heads, info.n_kblocks), dtype=torch.float32, device=dev)
    el = torch.empty((pw.batch, pw.heads), dtype=torch.int32, device=dev)
    bm = torch.empty((pw.batch, pw.heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    main_bufs = (q, k, v, o, qn, km, el, bm)

    def step(i, strm=None, bufs=None):
        s_ = stream if strm is None else strm
        q, k, v, o, qn, km, el, bm = main_bufs if bufs is None else bufs
        fsa.pre_attention(xs[i % len(xs)], wd, pw.heads, pw.head_dim, q=q, k=k, v=v, stream=s_)
        fsa.bounds(dplan, q, k, aw.scale, 0.0, 0, 0, qn, km, el, bm, stream=s_)
        fsa.attention(dplan, q, k, v, qn, km, el, aw.scale, 0, 0, out=o, stream=s_)

    preroll_ms, _ = preroll(step, args.preroll_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    # the same steps, consecutive steps on two streams in turn (own buffers)
    pstreams = [stream, torch.cuda.Stream()]
    pbufs = [tuple(torch.empty_like(t) for t in main_bufs) for _ in range(2)]
    for i in range(TWO_STREAM_WARMUP):
        step(i, pstreams[i % 2], pbufs[i % 2])
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    pstreams[1].wait_event(p0)
    for i in range(TWO_STREAM_STEPS):
        step(i, pstreams[i % 2], pbufs[i % 2])
    fin = torch.cuda.Event()
    fin.record(pstreams[1])
    stream.wait_event(fin)
    p1.record(stream)
    torch.cuda.synchronize()
    pipe_ms = p0.elapsed_time(p1) / TWO_STREAM_STEPS
    pre_flops = projection_flops(pw.batch, pw.seq_len, pw.channels, pw.heads, pw.head_dim)
    attn_flops = plan_flops(info, pw.batch, pw.heads, pw.head_dim)
    line = {
        "metric": "attention-layer hot path x -> q,k,v -> o (fused pre-attention + bounds + attention) TFLOP/s",
        "value": round((pre_flops + attn_flops) / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "pre720 + sr720", "tokens": pw.seq_len, "channels": pw.channels,
                   "heads": pw.heads, "head_dim": pw.head_dim, "pre_flops": pre_flops,
                   "attention_flops": attn_flops, "eligible_heads": int(el.sum().item())},
        "pct_of_peak": round(100.0 * (pre_flops + attn_flops) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "timing": {"preroll_ms": round(preroll_ms, 1)},
        "two_streams": {"steps": TWO_STREAM_STEPS, "warmup": TWO_STREAM_WARMUP,
                        "ms_per_step": round(pipe_ms, 5),
                        "value": round((pre_flops + attn_flops) / (pipe_ms * 1e-3) / 1e12, 3),
                        "note": "the same steps, consecutive steps on two streams in turn"},
    }
    print(json.dumps(line), flush=True)


def cpu_baseline_pre(wl, x, gain, w, tokens: int = 1 << 30):
    """Time the fp64 oracle on (at most) the first `tokens` tokens of batch item 0
    (by default the whole sequence: the oracle's projection is one BLAS call)."""
    import numpy as np

    import oracle
    import synthetic
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:                                  # noqa: BLE001
        threads = os.cpu_count() or 1
    xs = synthetic.to_f64(x[:1, :tokens])
    t0 = time.perf_counter()
    out = oracle.pre_attention(xs, gain.double().numpy(), synthetic.to_f64(w), wl.heads, wl.head_dim)
    dt = time.perf_counter() - t0
    assert all(np.isfinite(o).all() for o in out)
    flops = oracle.pre_attention_flops(1, xs.shape[1], wl.channels, wl.heads, wl.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batch 0, tokens 0..{xs.shape[1] - 1} of {wl.seq_len} ({flops:.3e} FLOPs, "
                      f"fp64), {dt:.2f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "head across GPUs but no multi-GPU run is built.", file=sys.stderr)
        sys.exit(2)

    if args.kernel == "pre_attention" and not args.copy_calibration:
        bench_pre_attention(args)
        return
    if args.kernel == "chain" and not args.copy_calibration:
        bench_chain(args)
        return

    import numpy as np
    import torch

    import frame_windowed_block_amd as fsa
    import synthetic

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4}))
        return

    wl = synthetic.WORKLOADS[args.workload]
    qc, kc, vc = synthetic.make_inputs(wl)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inputs = [tuple(x.to(dev) for x in (qc, kc, vc)) for _ in range(max(1, args.copies))]
    q = inputs[0][0]
    o = torch.empty_like(q)

    # plan: computed on the host every step into pinned memory and uploaded as
    # one copy (row_ptr and col_idx side by side) on a copy stream, into one of
    # two device plan buffers: the upload for step i + 1 overlaps step i
    info0, rp0, ci0 = fsa.plan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    n_rp, n_ci = rp0.size, ci0.size
    dplans, pinned = [], []
    for _ in range(2):
        dp = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, device=dev)
        buf = torch.empty(n_rp + n_ci, dtype=torch.int32, device=dev)
        dp.row_ptr, dp.col_idx = buf[:n_rp], buf[n_rp:]
        dp.buf = buf
        dplans.append(dp)
        pinned.append(torch.empty(n_rp + n_ci, dtype=torch.int32).pin_memory())
    copied = [None, None]           # copy of slot s done (pinned buffer free, device plan ready)
    used = [None, None]             # kernels of the last step that read device plan s done
    copy_stream = torch.cuda.Stream()
    import ctypes
    L = fsa.lib()
    P32 = ctypes.POINTER(ctypes.c_int32)
    bsz, heads, n, d = q.shape
    qn = torch.empty((bsz, heads, n), dtype=torch.float32, device=dev)
    km = torch.empty((bsz, heads, info0.n_kblocks), dtype=torch.float32, device=dev)
    el = torch.empty((bsz, heads), dtype=torch.int32, device=dev)
    bm = torch.empty((bsz, heads), dtype=torch.float32, device=dev)
    mu = torch.empty((bsz, heads, d), dtype=torch.float32, device=dev) if args.center else None
    stream = torch.cuda.current_stream()
    main_stream, main_bufs = stream, (qn, km, el, bm, o)
    if args.groups > 1 and heads % args.groups:
        print(f"--groups {args.groups} does not divide {heads} heads", file=sys.stderr)
        sys.exit(2)
    group_streams = [torch.cuda.Stream() for _ in range(args.groups)] if args.groups > 1 else []

    def step(i, ev=None, strm=None, bufs=None):
        q, k, v = inputs[i % len(inputs)]
        stream = main_stream if strm is None else strm
        qn, km, el, bm, o = main_bufs if bufs is None else bufs
        slot = i & 1
        if copied[slot] is not None:
            copied[slot].synchronize()                  # pinned buffer free again
        hp = pinned[slot]
        info = fsa.PlanInfo()
        st = L.fsa_plan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, 0, 0,
                        ctypes.byref(info), ctypes.cast(hp.data_ptr(), P32), n_rp,
                        ctypes.cast(hp.data_ptr() + 4 * n_rp, P32), n_ci)
        assert st == 0
        dplan = dplans[slot]
        with torch.cuda.stream(copy_stream):
            if used[slot] is not None:
                copy_stream.wait_event(used[slot])      # step i - 2 is done reading this buffer
            dplan.buf.copy_(hp, non_blocking=True)
            e = torch.cuda.Event()
            e.record(copy_stream)
        copied[slot] = e
        stream.wait_event(e)
        timed = ev is not None and i % EVENTS_EVERY == 0
        if timed:
            ev[0].record(stream)
        fsa.bounds(dplan, q, k, wl.scale, 0.0, 0, 0, qn, km, el, bm, stream=stream, kmean=mu)
        if timed:
            ev[1].record(stream)
        if args.groups <= 1:
            fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, 0, 0, out=o, stream=stream, kmean=mu)
        else:
            # head groups on their own streams, each waiting for the bounds
            # (the one-GPU part of head-group pipelining); the step stream
            # waits for all of them
            ready = torch.cuda.Event()
            ready.record(stream)
            hg = heads // args.groups
            for g, gs in enumerate(group_streams):
                gs.wait_event(ready)
                fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, g * hg, hg, out=o, stream=gs,
                              kmean=mu)
                done = torch.cuda.Event()
                done.record(gs)
                stream.wait_event(done)
        if timed:
            ev[2].record(stream)
            used[slot] = ev[2]
        else:
            u = torch.cuda.Event()
            u.record(stream)
            used[slot] = u

    clocks = ClockSampler()
    # pre-roll: the engine clock idles between runs and ramps up under load;
    # steps run for a fixed wall time first, so the timed steps do not pay
    # for the ramp (they are not counted anywhere)
    clocks.start()
    preroll_ms, pre_steps = preroll(step, args.preroll_ms)
    clk_preroll = clocks.stop()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    host_s = []
    torch.cuda.synchronize()
    clocks.start()
    t_start.record(stream)
    for i in range(args.steps):
        h0 = time.perf_counter()
        step(i, evs[i])
        host_s.append(time.perf_counter() - h0)
    t_end.record(stream)
    torch.cuda.synchronize()
    clk_timed = clocks.stop()
    total_ms = t_start.elapsed_time(t_end)
    sampled = [e for i, e in enumerate(evs) if i % EVENTS_EVERY == 0]
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in sampled])
    bnd_ms = np.array([e[0].elapsed_time(e[1]) for e in sampled])

    # the bounds pass on its own, after the timed steps: BOUNDS_ALONE calls
    # back to back over the rotating input copies, one event pair around them
    # all (no event between its two kernels or before the attention kernel)
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b0.record(stream)
    for i in range(BOUNDS_ALONE):
        bq_, bk_, _ = inputs[i % len(inputs)]
        fsa.bounds(dplans[0], bq_, bk_, wl.scale, 0.0, 0, 0, qn, km, el, bm, stream=stream, kmean=mu)
    b1.record(stream)
    torch.cuda.synchronize()
    bounds_alone_ms = b0.elapsed_time(b1) / BOUNDS_ALONE

    # the same steps with consecutive steps on two streams in turn (each with
    # its own bounds and output buffers): a step's kernels may then start on
    # the CUs that the previous step's attention kernel leaves idle while its
    # last workgroups finish. Whole-job throughput only (launches overlap, so
    # no per-kernel timing); the line's own figures stay sequential.
    pstreams = [stream, torch.cuda.Stream()]
    pbufs = [(torch.empty_like(qn), torch.empty_like(km), torch.empty_like(el), torch.empty_like(bm),
              torch.empty_like(o)) for _ in range(2)]
    torch.cuda.synchronize()
    for i in range(TWO_STREAM_WARMUP):
        step(i, strm=pstreams[i % 2], bufs=pbufs[i % 2])
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    pstreams[1].wait_event(p0)
    for i in range(TWO_STREAM_STEPS):
        step(i, strm=pstreams[i % 2], bufs=pbufs[i % 2])
    fin = torch.cuda.Event()
    fin.record(pstreams[1])
    stream.wait_event(fin)
    p1.record(stream)
    torch.cuda.synchronize()
    pipe_ms = p0.elapsed_time(p1) / TWO_STREAM_STEPS

    flops = plan_flops(info0, bsz, heads, d)
    ms_per_step = total_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_mean = float(attn_ms.mean())
    achieved = flops / (attn_mean * 1e-3) / 1e12
    # q and k read once, the norm arrays written; centring reads k once more
    # (the mean must be known before the centred norms) and writes the mean
    bounds_bytes = 2 * bsz * heads * n * d * 2 + 4 * bsz * heads * (n + info0.n_kblocks + 2)
    if args.center:
        bounds_bytes += bsz * heads * n * d * 2 + 4 * bsz * heads * d
    eligible = el.cpu().numpy()
    traffic_key = wl.name + ("+center" if args.center else "")

    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "heads": wl.heads, "head_dim": wl.head_dim,
            "frames": wl.frames, "tokens_per_frame": wl.tokens_per_frame, "seq_len": wl.seq_len,
            "window": wl.window, "ref_frame": wl.ref_frame, "block_q": info0.block_q,
            "block_k": info0.block_k, "nnz": info0.nnz, "active_flops": flops,
            "eligible_heads": int(eligible.sum()), "key_centring": bool(args.center),
            "head_groups": args.groups,
        },
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "sclk_mhz": clk_timed.get("mean"),
        "pct_of_peak_at_sclk": (round(100.0 * value / (256 * 4096 * clk_timed["mean"] * 1e-6), 2)
                                if clk_timed.get("mean") else None),
        "timing": {
            "preroll_ms": round(preroll_ms, 1), "preroll_steps": pre_steps,
            "sclk_preroll_mhz": clk_preroll, "sclk_timed_mhz": clk_timed,
            "host_us_per_step": round(1e6 * float(np.mean(host_s)), 1),
            "attention_ms_first5": [round(float(x), 4) for x in attn_ms[:5]],
            "attention_ms_last5": [round(float(x), 4) for x in attn_ms[-5:]],
        },
        "roofline": {
            "kernel": "fsa_attention",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("fsa_attention", traffic_key) if args.groups <= 1 else None,
            "timed_steps": int(attn_ms.size),
            "mean_ms": round(attn_mean, 5),
            "median_ms": round(float(np.median(attn_ms)), 5),
            "p10_ms": round(float(np.percentile(attn_ms, 10)), 5),
            "p90_ms": round(float(np.percentile(attn_ms, 90)), 5),
        },
        "two_streams": {
            "steps": TWO_STREAM_STEPS,
            "warmup": TWO_STREAM_WARMUP,
            "ms_per_step": round(pipe_ms, 5),
            "value": round(flops / (pipe_ms * 1e-3) / 1e12, 3),
            "note": "the same steps, consecutive steps on two streams in turn",
        },
        "bounds": {
            "kernels": "fsa_bounds (norms + bound reduce)",
            "timed_steps": int(bnd_ms.size),
            "mean_ms": round(float(bnd_ms.mean()), 5),
            "median_ms": round(float(np.median(bnd_ms)), 5),
            "gbps": round(bounds_bytes / (float(bnd_ms.mean()) * 1e-3) / 1e9, 1),
            "alone_calls": BOUNDS_ALONE,
            "alone_mean_ms": round(bounds_alone_ms, 5),
            "alone_gbps": round(bounds_bytes / (bounds_alone_ms * 1e-3) / 1e9, 1),
            "input_copies": len(inputs),
            "peak_gbps": PEAK_HBM_GBPS,
            "algorithmic_bytes": bounds_bytes,
            "traffic": measured_traffic("fsa_bounds_norms", traffic_key),
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"], ref = cpu_baseline(wl, qc, kc, vc, args.cpu_heads)
        # the last timed step's output (every input copy holds the same values),
        # against that oracle run; the per-element bar also needs the second
        # moment of v under each row's weights (the oracle's visible-key form,
        # untimed) and each row's score bound
        sl = slice(0, args.cpu_heads)
        q64, k64, v64 = (synthetic.to_f64(x[:1, sl]) for x in (qc, kc, vc))
        margs = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
        _, m2 = oracle.attention_visible(q64, k64, v64, *margs, moments=True)
        sb = oracle.row_bound_by_frames(q64, k64, *margs)
        nk = np.array([len(oracle.visible_frames(i // wl.tokens_per_frame, wl.frames, wl.window,
                                                 wl.ref_frame)) * wl.tokens_per_frame for i in range(n)])
        got = synthetic.to_f64(o[:1, sl].cpu())
        line["check"] = output_check(got, ref, m2, sb, np.broadcast_to(nk, sb.shape), d,
                                     f"o, batch 0, heads 0..{args.cpu_heads - 1}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
