#!/usr/bin/env python3
"""Benchmark of the block-scaled FP8 linear on one MI355X.

Default workload: the Qwen3-8B-shaped prefill linears at M = 2048 tokens
(qkv 6144x4096, o 4096x4096, gate_up 24576x4096, down 4096x12288).  One step
is the whole hot path for all four: the activation is quantized per 1x128
group (quantize_fp8_groups) and multiplied with the pre-quantized weight
(fp8_gemm_nt, bf16 out).  Weights are quantized once before timing (an
offline step, as the pages' plugin keeps weights and scales as persistent
parameters).  Inputs are seeded synthetic data resident in HBM before the
timed region.

    python bench.py [--gpus 1] [--steps 100] [--warmup 50] [--workload prefill]

Prints ONE JSON line: value = TFLOP/s over the step (2*M*N*K summed over the
four linears, divided by the time of quantize + product), the median of 5
trials of K steps.  The step time is the HIP-event time from the first timed
launch to the end of the last.  The host enqueues a prefill step in about a
third of its device time, so the launches run back to back on the device by
themselves; where the host would fall behind (small kernels), the steps are
enqueued while a bounded spin kernel holds the GPU (the host-side Python
launch path, ~10-30 us per call, is not part of the device's work; callers
that launch from C++ or a HIP graph see the same device time).  Trials of
100 steps measure the sustained rate: the GPU's power management takes tens
of milliseconds to settle after an idle or sleeping gap.  Also reported:
* roofline: the dominant kernel's algorithmic TFLOP/s from HIP events on the
  launch stream, recorded around that kernel's launches only (created without
  the system-scope fence, so that recording them barely disturbs the step),
  against the 5.0 PFLOP/s dense FP8 peak;
* decode: M = 1, 4, 16 linears (act-quant included per call) in GB/s against 8 TB/s,
  timed by graph replay over 8 rotating weight sets so that the weights stream
  from HBM rather than the 256 MB last-level cache;
* cpu_baseline: the CPU oracle on a bounded sample of the same workload.
Other --workload values time one shape for profiling: prefill_ue8m0 (the
same step with power-of-two scales, the matrix cores applying them), prefill_mx
(the MXFP8 recipe: one power-of-two scale per 1x32 block of every row of both
operands), decode (M=1 linears),
moe (contiguous grouped, 32 experts), moe_masked (masked grouped over a
decode-time dispatch buffer), moe_layer (the whole MoE layer: routing, gather,
two grouped products, SiLU-times-up and combine, 8192 tokens top-4 over 32
experts, H = 7168, I = 2048), square8k, square16k, copy (counter calibration),
stream (the plain streaming read at 48 MiB and 768 MiB: the HBM ceiling at the
decode weight's size), quantize (the activation quantizer at the prefill shapes
beside torch's bf16 -> FP8 cast of the same tensor, which moves the same bytes).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 (E4M3) MFMA peak
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
STEPS_ARE = {
    "prefill": "act-quant (1x128) + block-scaled FP8 GEMM (bf16 out) for every linear; weights pre-quantized",
    "prefill_mx": "act-quant (1x32 E8M0) + MXFP8 GEMM (bf16 out) for every linear; weights pre-quantized (1x32 E8M0)",
    "moe": "act-quant (1x128) of the padded expert layout + M-grouped contiguous block-scaled FP8 GEMM; "
           "weights pre-quantized",
    "moe_masked": "act-quant (1x128) of the dispatch buffer's real rows (counts read on the device) + masked "
                  "grouped block-scaled FP8 GEMM; weights pre-quantized",
    "decode": "act-quant (1x128) + decode-shaped FP8 GEMM (two launches) for M = 1 at both decode shapes; the "
              "decode object times the fused single-launch form",
    "moe_layer": "route + gather/act-quant + grouped GEMM (gate_up) with SiLU*up/act-quant in its epilogue + "
                 "grouped GEMM (down) + weighted combine; expert weights pre-quantized; value counts routed rows only",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="prefill", choices=["prefill", "prefill_ue8m0", "prefill_mx", "decode", "moe", "moe_masked", "moe_layer", "square8k", "square16k", "copy", "stream", "quantize"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--trials", type=int, default=TRIALS, help="timed trials of --steps steps each")
    p.add_argument("--no-clock", action="store_true",
                   help="skip the sustained run that reads the GPU clock (profiling runs)")
    p.add_argument("--no-extra", action="store_true",
                   help="prefill: skip the 8192^3, 16384^2x8192 and 32-expert grouped objects")
    p.add_argument("--moe-unfused", action="store_true",
                   help="moe_layer: run the gate_up product and SiLU.mul+quantize as two launches")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--decode-reps", type=int, default=50, help="rounds over the 8 weight sets per decode timing")
    return p.parse_args()


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------- setup
def dev_bf16(bits, torch):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class PreparedLinear:
    """Device buffers for one linear: bf16 activation, pre-quantized weight,
    and preallocated outputs (nothing is allocated inside the timed region)."""

    def __init__(self, lin, fg, torch, recipe="fp32"):
        self.lin = lin
        self.recipe = recipe
        self.ue8m0 = recipe == "ue8m0"
        self.x = dev_bf16(lin.a, torch)
        w = dev_bf16(lin.b, torch)
        if recipe == "mx":
            self.qb, self.sb = fg.quantize_fp8_mx(w)
        else:
            self.qb, self.sb = fg.quantize_fp8_blocks(w, ue8m0=self.ue8m0)
        del w
        m, k = lin.m, lin.k
        self.q = torch.empty((m, k), dtype=torch.float8_e4m3fn, device="cuda")
        self.sa = torch.empty((k // 128, fg.padded_rows(m)), dtype=torch.int32 if recipe == "mx" else torch.float32,
                              device="cuda")
        self.d = torch.empty((m, lin.n), dtype=torch.bfloat16, device="cuda")
        # the product's workspace (allocated once, zero-filled), for shapes
        # whose plan splits K over two workgroups per tile
        self.ws = fg.gemm_workspace(m, lin.n, k) if recipe == "fp32" else None
        plan = fg.describe_gemm(m, lin.n, k)
        self.plan = plan.split("with workspace: ")[1] if self.ws is not None else plan.split(";")[0]
        # the FP32-scale bf16 call may walk its tiles persistently; the other recipes do not
        walk = recipe == "fp32" and self.plan.endswith(" persistent")
        self.kernel = self.plan.split()[0] + (" persistent" if walk else "")

    def run(self, fg, ev=None):
        """Act-quant then product; ev = (before, between, after) events, any
        of them None."""
        if ev is not None and ev[0] is not None:
            ev[0].record()
        if self.recipe == "mx":
            fg.quantize_fp8_mx(self.x, out=(self.q, self.sa))
        else:
            fg.quantize_fp8_groups(self.x, out=(self.q, self.sa), ue8m0=self.ue8m0)
        if ev is not None and ev[1] is not None:
            ev[1].record()
        if self.recipe == "mx":
            fg.fp8_gemm_nt_mx((self.q, self.sa), (self.qb, self.sb), self.d)
        else:
            fg.fp8_gemm_nt((self.q, self.sa), (self.qb, self.sb), self.d, ue8m0=self.ue8m0, workspace=self.ws)
        if ev is not None and ev[2] is not None:
            ev[2].record()


def quant_bytes(m, k):
    return 3 * m * k + 4 * (-(-m // 4) * 4) * (k // 128)


def gemm_bytes(m, n, k, mx=False):
    """A, its scales, B, its scales (one per 128x128 block, or with the MX
    recipe one packed word per row and chunk) and the bf16 output."""
    sb_rows = n if mx else -(-n // 128)
    return m * k + 4 * (-(-m // 4) * 4) * (k // 128) + n * k + 4 * sb_rows * (k // 128) + 2 * m * n


# --------------------------------------------------------------- prefill step
class HipEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording
    it does not flush caches to system scope, which costs ~5 us of idle GPU
    time per record with torch's default events.  Even these cost ~1 us of
    step time per record, so the timed region records only the events the
    roofline needs.  API-compatible with the two methods of
    torch.cuda.Event used here; records on torch's current stream."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self, torch):
        import ctypes

        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self._ctypes = ctypes
        self._torch = torch
        self.ev = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), HipEvent.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        stream = self._torch.cuda.current_stream().cuda_stream
        if HipEvent._hip.hipEventRecord(self.ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both complete)."""
        ms = self._ctypes.c_float()
        if HipEvent._hip.hipEventElapsedTime(self._ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        hip = getattr(HipEvent, "_hip", None) if HipEvent is not None else None
        if hip is not None and getattr(self, "ev", None):
            hip.hipEventDestroy(self.ev)


class GpuAhead:
    """Keeps the GPU busy (torch's bounded spin kernel) while the host
    enqueues the timed steps, so that the launches run back to back on the
    device: HIP events then time the kernels, not the Python launch path
    (one launch through the binding costs ~10-30 us of host time, comparable
    to the small kernels).  The spin length is calibrated once and sized to
    the measured host time of enqueueing the steps."""

    def __init__(self, torch):
        self.torch = torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cycles = 20_000_000
        torch.cuda._sleep(cycles)  # warm
        e0.record()
        torch.cuda._sleep(cycles)
        e1.record()
        torch.cuda.synchronize()
        self.cycles_per_s = cycles / (e0.elapsed_time(e1) * 1e-3)

    def spin(self, seconds: float) -> None:
        self.torch.cuda._sleep(int(self.cycles_per_s * seconds))

    def lead_in(self, host_s: float, gpu_s: float) -> None:
        """Before a timed region of steps that take `gpu_s` on the device and
        `host_s` to enqueue: spin only where the host would fall behind the
        device.  Where it keeps ahead by itself the first launch starts at
        once and no spin is run, because a few milliseconds of a sleeping GPU
        let its power management drop the clock, and the steps that follow
        then run during the climb back (measured on the prefill step: 20-step
        trials after a 6 ms spin 0.459 ms per step, 100-step trials with no
        spin 0.410, the same as a long back-to-back run)."""
        if host_s > 0.5 * gpu_s:
            self.spin(1.5 * host_s + 2e-3)


TRIALS = 5  # timed trials per measurement; min and median are reported
NO_CLOCK = False  # --no-clock


class SmiSampler:
    """The GPU's graphics clock and socket power as amdsmi reports them,
    polled from a host thread, keeping only the samples taken while a window
    is open.  The firmware refreshes these metrics about once a second, so a
    reading describes the run only once the run has lasted well over a
    second.  summary() is None where amdsmi is not usable."""

    def __init__(self, period: float = 0.01):
        self.samples = []
        self.period = period
        self._open = False
        self._stop = None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        except Exception as e:  # not on every box
            log(f"amdsmi unavailable: {e!r}")
            self._smi = None

    def __enter__(self):
        import threading

        if self._smi is None:
            return self
        self._stop = threading.Event()

        def poll():
            while not self._stop.is_set():
                if self._open:
                    try:
                        m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                        xcc = [v for v in (m.get("current_gfxclks") or []) if isinstance(v, (int, float)) and 0 < v < 65535]
                        if self._open:
                            self.samples.append((m.get("current_gfxclk"), m.get("current_socket_power"), time.time(),
                                                 float(np.median(xcc)) if xcc else None))
                    except Exception:
                        pass
                time.sleep(self.period)

        self._t = threading.Thread(target=poll, daemon=True)
        self._t.start()
        return self

    def window_open(self):
        self._open = True

    def window_close(self):
        self._open = False

    def __exit__(self, *exc):
        if self._stop is not None:
            self._stop.set()
            self._t.join()

    def summary(self):
        ok = lambda v: isinstance(v, (int, float)) and 0 < v < 65535
        clk = [x[0] for x in self.samples if ok(x[0])]
        pw = [x[1] for x in self.samples if ok(x[1])]
        xcc = [x[3] for x in self.samples if ok(x[3])]
        if not clk:
            return None
        readings = len({(x[0], x[1]) for x in self.samples if ok(x[0])})
        return {"source": "amdsmi gpu_metrics current_gfxclk / current_socket_power",
                "samples": len(clk), "distinct_readings": readings,
                "gfxclk_mhz_median": float(np.median(clk)), "gfxclk_mhz_min": float(min(clk)),
                "gfxclk_mhz_max": float(max(clk)),
                "xcd_gfxclk_mhz_median": float(np.median(xcc)) if xcc else None,
                "socket_power_w_median": float(np.median(pw)) if pw else None,
                "socket_power_w_max": float(max(pw)) if pw else None}


def sustained_clock(step, torch, step_s: float, seconds: float = 3.0, settle: float = 1.5):
    """The GPU clock and power under a sustained run of `step`: enough steps
    for `seconds` of GPU time (`step_s` each) are enqueued back to back after
    the timed trials, and amdsmi is sampled until they finish, keeping the
    samples after the first `settle` seconds.  The metrics refresh about once
    a second, so the first readings of a run still describe what came before
    it; the settle skips them.  The run's own device time per step (events
    around it) is reported beside the clock, so that the reading can be
    matched with the trials."""
    if NO_CLOCK:
        return None
    smi = SmiSampler()
    if smi._smi is None:
        return None
    n = max(1, int(seconds / max(step_s, 1e-6)))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    smi.__enter__()
    smi.window_open()
    t0 = time.time()
    e0.record()
    for _ in range(n):
        step()
    e1.record()
    torch.cuda.synchronize()
    smi.window_close()
    smi.__exit__()
    smi.samples = [x for x in smi.samples if x[2] >= t0 + settle]
    out = smi.summary()
    if out is not None:
        out["source"] = (f"amdsmi gpu_metrics current_gfxclk (and the median over the XCDs' current_gfxclks) / "
                         f"current_socket_power, polled every ~10 ms over the last ~{seconds - settle:.1f} s of "
                         f"{n} back-to-back steps right after the timed trials (the firmware refreshes them about "
                         f"once a second)")
        out["sustained_ms_per_step"] = round(e0.elapsed_time(e1) / n, 4)
    return out


def trial_stats(seconds: list, steps: int) -> dict:
    ms = sorted(x / steps * 1e3 for x in seconds)
    return {"trials": len(ms), "ms_per_step": [round(x, 4) for x in ms], "ms_per_step_min": round(ms[0], 4),
            "ms_per_step_median": round(float(np.median(ms)), 4)}


def host_enqueue_seconds(fn, torch, reps=3):
    """Host time to enqueue fn() (no synchronisation inside), max of reps."""
    worst = 0.0
    for _ in range(reps):
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        worst = max(worst, time.perf_counter() - t)
    torch.cuda.synchronize()
    return worst


def gpu_step_seconds(fn, torch, reps=10):
    """Device time per call of fn() over `reps` calls enqueued back to back
    (an upper bound where the host is the slower side)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def per_linear_pass(preps, steps, fg, torch, ahead, host_step, gpu_step):
    """Per-linear breakdown: `steps` steps with three events per linear
    (before the act-quant, between, after the product).  Runs before the
    timed region, so its event records do not weigh on the step time."""
    events = [[[HipEvent(torch) for _ in range(3)] for _ in preps] for _ in range(steps)]
    torch.cuda.synchronize()
    ahead.lead_in(host_step * steps, gpu_step * steps)
    for s in range(steps):
        for p, ev in zip(preps, events[s]):
            p.run(fg, ev)
    torch.cuda.synchronize()
    per = []
    for i, p in enumerate(preps):
        qt = np.mean([events[s][i][0].elapsed_time(events[s][i][1]) for s in range(steps)]) * 1e-3
        gt = np.mean([events[s][i][1].elapsed_time(events[s][i][2]) for s in range(steps)]) * 1e-3
        lin = p.lin
        per.append(
            {
                "name": lin.name,
                "m": lin.m,
                "n": lin.n,
                "k": lin.k,
                "kernel": p.plan,
                "quant_us": qt * 1e6,
                "quant_gbs": quant_bytes(lin.m, lin.k) / qt / 1e9,
                "gemm_us": gt * 1e6,
                "gemm_tflops": lin.flops / gt / 1e12,
                "_kernel": p.kernel + (" mx" if p.recipe == "mx" else ""),
                "_bytes": gemm_bytes(lin.m, lin.n, lin.k, mx=p.recipe == "mx"),
                "_flops": lin.flops,
                "_gemm_s": gt,
            }
        )
    return per


def dominant_kernel(per) -> str:
    """The GEMM kernel with the largest total time over the step."""
    total = {}
    for r in per:
        total[r["_kernel"]] = total.get(r["_kernel"], 0.0) + r["_gemm_s"]
    return max(total, key=total.get)


def bench_linears(linears, steps, warmup, fg, torch, recipe="fp32", trials=TRIALS):
    """Warm-up, the per-linear pass, then `trials` timed regions: `steps`
    steps each, bracketed by two events, with events recorded only around
    the launches of the dominant kernel (its mean launch duration for the
    roofline); then the GPU clock under a sustained run of the step.  Returns
    (preps, per-trial elapsed seconds, per-linear rows, timed dominant-kernel
    launches, clock summary)."""
    preps = [PreparedLinear(l, fg, torch, recipe) for l in linears]
    torch.cuda.synchronize()
    for _ in range(warmup):
        for p in preps:
            p.run(fg)
    torch.cuda.synchronize()
    ahead = GpuAhead(torch)
    probe = [[HipEvent(torch) for _ in range(3)] for _ in preps]
    host_step = host_enqueue_seconds(lambda: [p.run(fg, ev) for p, ev in zip(preps, probe)], torch)
    gpu_step = gpu_step_seconds(lambda: [p.run(fg) for p in preps], torch)
    per = per_linear_pass(preps, steps, fg, torch, ahead, host_step, gpu_step)
    dom = dominant_kernel(per)
    elapsed, launches = [], []
    for _ in range(trials):
        dom_ev = [[(None, HipEvent(torch), HipEvent(torch)) if r["_kernel"] == dom else None for r in per]
                  for _ in range(steps)]
        e_first, e_last = HipEvent(torch), HipEvent(torch)
        torch.cuda.synchronize()
        ahead.lead_in(host_step * steps, gpu_step * steps)
        e_first.record()
        for s in range(steps):
            for p, ev in zip(preps, dom_ev[s]):
                p.run(fg, ev)
        e_last.record()
        torch.cuda.synchronize()
        elapsed.append(e_first.elapsed_time(e_last) * 1e-3)
        launches += [ev[1].elapsed_time(ev[2]) * 1e-3 for row in dom_ev for ev in row if ev is not None]
    timed = {"kernel": dom, "mean_s": float(np.mean(launches)), "launches": len(launches)}
    clock = sustained_clock(lambda: [p.run(fg) for p in preps], torch, float(np.median(elapsed)) / steps)
    log(f"timed: {steps} steps x {trials} trials, ms/step " + ", ".join(f"{e * 1e3 / steps:.4f}" for e in elapsed)
        + f"; host enqueue {host_step * 1e3:.3f} ms/step (device {gpu_step * 1e3:.3f}); {dom}: {len(launches)} launches timed, "
        f"mean {timed['mean_s'] * 1e6:.2f} us; gpu clock {clock}")
    return preps, elapsed, per, timed, clock


# The sources the tile GEMM kernels are built from.
GEMM_SOURCES = ("common.hpp", "gemm.hip", "kernels.hpp")


def kernel_sources_hash() -> str:
    """SHA-256 prefix over the GEMM kernels' sources, to tie a counter record
    in profiles/ to the code it was measured on."""
    import hashlib

    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        h.update(name.encode())
        with open(os.path.join(ROOT, "fine_grained_block_fp8_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, shape=None):
    """HBM bytes per launch of `kernel` (at `shape` = [m, n, k] when given)
    from the FETCH_SIZE / WRITE_SIZE counter runs summarised in profiles/
    (scaled by a plain-copy calibration), or None when no record matches the
    current sources."""
    import glob

    want = kernel_sources_hash()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if line.startswith("traffic-record:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if (rec.get("kernel") == kernel and rec.get("sources") == want
                            and (shape is None or rec.get("shape") == list(shape))):
                        return rec["bytes_per_launch"]
    return None


def roofline_of(per, timed=None):
    """Dominant kernel (largest total time among the GEMM kernels): its
    algorithmic FLOPs per launch over its mean launch duration -- from the
    events around its launches in the timed region when `timed` is given,
    else from the per-linear rows."""
    by = {}
    for r in per:
        e = by.setdefault(r["_kernel"], {"flops": 0, "s": 0.0, "n": 0, "bytes": 0})
        e["flops"] += r["_flops"]
        e["bytes"] += r["_bytes"] if "_bytes" in r else gemm_bytes(r["m"], r["n"], r["k"])
        e["s"] += r["_gemm_s"]
        e["n"] += 1
    name, e = max(by.items(), key=lambda kv: kv[1]["s"])
    if timed is not None:
        name, e = timed["kernel"], by[timed["kernel"]]
    flops_per_launch = e["flops"] / e["n"]
    mean_s = timed["mean_s"] if timed is not None else e["s"] / e["n"]
    shapes = {(r["m"], r["n"], r["k"]) for r in per if r["_kernel"] == name}
    shape = next(iter(shapes)) if len(shapes) == 1 else None
    achieved = flops_per_launch / mean_s / 1e12
    if name.endswith("_splitk2"):
        kernel = f"gemm_nt_splitk_kernel<{name.replace('_splitk2', '')}>"
    elif name.endswith(" persistent"):
        kernel = f"gemm_nt_persistent_kernel<{name.replace(' persistent', '')}>"
    else:
        kernel = f"gemm_nt_kernel<{name.replace(' mx', ', mx')}>"
    return {
        "bound": "mfma",
        "kernel": kernel,
        "achieved": round(achieved, 1),
        "peak": PEAK_FP8_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
        "traffic": recorded_traffic(kernel, shape),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
        "algorithmic_bytes_per_launch": round(e["bytes"] / e["n"]),
        "launches_per_step": e["n"],
        "mean_launch_us": round(mean_s * 1e6, 2),
        "launch_timing": ("HIP events around each launch of this kernel inside the timed region"
                          if timed is not None else "HIP events around each launch (per-linear pass)"),
        "algorithmic_gflop_per_launch": round(flops_per_launch / 1e9, 3),
    }


def bench_object(lin, steps, warmup, fg, torch, trials=TRIALS) -> dict:
    """One linear as a bench object of its own: act-quant + product per step,
    `trials` timed regions of `steps` steps, min and median step time, the
    clock, and the product kernel's roofline."""
    preps, elapsed, per, timed, clock = bench_linears([lin], steps, warmup, fg, torch, trials=trials)
    del preps
    st = trial_stats(elapsed, steps)
    r = per[0]
    return {
        "workload": lin.name,
        "m": lin.m, "n": lin.n, "k": lin.k,
        "kernel": r["kernel"],
        "steps_are": "act-quant (1x128) + block-scaled FP8 GEMM (bf16 out); weight pre-quantized",
        "ms_min": st["ms_per_step_min"],
        "ms_median": st["ms_per_step_median"],
        "tflops_median": round(lin.flops / (st["ms_per_step_median"] * 1e-3) / 1e12, 1),
        "frac_of_fp8_peak": round(lin.flops / (st["ms_per_step_median"] * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
        "quant_us": round(r["quant_us"], 2),
        "gemm_us": round(r["gemm_us"], 2),
        "timing": st,
        "gpu_clock": clock,
        "roofline": roofline_of(per, timed),
    }


# ------------------------------------------------------------------- decode
def bench_decode(fg, torch, ms=(1, 4, 16), shapes=((12288, 4096), (4096, 12288)), sets=8, reps=50, trials=TRIALS):
    """Act-quant + product per call at M = 1, 4, 16; 8 rotating weight sets
    (8 x 50 MB > 256 MB last-level cache) replayed from a HIP graph, and
    eagerly.  M <= 4 runs the fused kernel; M = 16 passes the activation
    workspace, with which the library runs the quantizer and the decode
    product (two launches) at these shapes."""
    import workloads

    out = []
    for m, (n, k) in [(m_, sh) for m_ in ms for sh in shapes]:
        lin = workloads.decode_linear(m, n, k)
        x = dev_bf16(lin.a, torch)
        w = dev_bf16(lin.b, torch)
        qb0, sb0 = fg.quantize_fp8_blocks(w)
        del w
        weights = [(qb0, sb0)] + [(qb0.clone(), sb0.clone()) for _ in range(sets - 1)]
        d = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
        fused = m <= fg.FUSED_FAST_MAX_M  # above it, the workspace path is faster
        act = None if fused else (torch.empty((m, k), dtype=torch.float8_e4m3fn, device="cuda"),
                                  torch.empty((k // 128, fg.padded_rows(m)), dtype=torch.float32, device="cuda"))

        def one_round():
            # act-quant + product (one fused kernel per call for M <= 4)
            for qb, sb in weights:
                fg.fp8_linear_nt(x, (qb, sb), d, act)

        for _ in range(3):
            one_round()
        torch.cuda.synchronize()
        # eager, back-to-back
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            one_round()
        e1.record()
        torch.cuda.synchronize()
        eager_s = e0.elapsed_time(e1) * 1e-3 / (reps * sets)
        # graph replay
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            one_round()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                one_round()
        torch.cuda.synchronize()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        graph_trials = []
        for _ in range(trials):
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            graph_trials.append(e0.elapsed_time(e1) * 1e-3 / (reps * sets))
        graph_s = float(np.median(graph_trials))
        nbytes = quant_bytes(m, k) + gemm_bytes(m, n, k)
        out.append(
            {
                "m": m,
                "n": n,
                "k": k,
                "kernel": fg.describe_linear(m, n, k, act is not None),
                "bytes_per_call": nbytes,
                "graph_us": round(graph_s * 1e6, 3),
                "graph_us_min": round(min(graph_trials) * 1e6, 3),
                "graph_timing": f"median and min of {trials} trials of {reps} replays of {sets} calls",
                "graph_gbs": round(nbytes / graph_s / 1e9, 1),
                "graph_frac_hbm": round(nbytes / graph_s / 1e9 / PEAK_HBM_GBS, 4),
                "eager_us": round(eager_s * 1e6, 3),
                "eager_gbs": round(nbytes / eager_s / 1e9, 1),
                "weight_sets": sets,
            }
        )
        del weights, qb0, sb0, g
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------ quantizer ceiling
def bench_quantize(fg, torch, shapes=((2048, 4096), (2048, 12288), (8192, 8192)), reps=50, trials=TRIALS):
    """quantize_fp8_groups at the prefill activation shapes, beside torch's
    bf16 -> float8_e4m3fn cast of the same tensor (a vendor elementwise kernel
    that moves the same 2 bytes in and 1 byte out per element, without the
    group amax): the rate a read-plus-write stream of that size reaches.
    Inputs rotate over enough buffers (>= 600 MB) that no launch is served
    from the 256 MB last-level cache."""
    out = []
    for m, k in shapes:
        sets = max(2, int(600e6 // (3 * m * k)))
        g = torch.Generator(device="cuda")
        g.manual_seed(m + k)
        xs = [torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16) for _ in range(sets)]
        qs = [fg.quantize_fp8_groups(x) for x in xs]
        casts = [torch.empty((m, k), dtype=torch.float8_e4m3fn, device="cuda") for _ in range(sets)]

        def quant():
            for x, o in zip(xs, qs):
                fg.quantize_fp8_groups(x, out=o)

        def cast():
            for x, c in zip(xs, casts):
                c.copy_(x)

        res = {}
        for name, fn in (("quantize_fp8_groups", quant), ("torch_cast_to_fp8", cast)):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(trials):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(max(1, reps // sets)):
                    fn()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3 / (max(1, reps // sets) * sets))
            res[name] = ts
        qb = quant_bytes(m, k)
        row = {"m": m, "k": k, "bytes": qb, "sets": sets}
        for name, ts in res.items():
            t = float(np.median(ts))
            row[name] = {"us": round(t * 1e6, 3), "us_min": round(min(ts) * 1e6, 3), "gbs": round(qb / t / 1e9, 1),
                         "frac_hbm": round(qb / t / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"quantize {m}x{k}: {row['quantize_fp8_groups']['us']} us; torch cast {row['torch_cast_to_fp8']['us']} us")
        out.append(row)
        del xs, qs, casts
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------ streaming ceiling
def bench_stream(fg, torch, sizes=(50_331_648, 805_306_368), sets=8, reps=50, trials=TRIALS):
    """The plain streaming read (fgfp8_stream_read) at the decode weight's
    size (48 MiB, 8 rotating buffers so that nothing is served from the
    256 MB last-level cache, replayed from a HIP graph as the decode linears
    are) and at 768 MiB: the rate a kernel that only reads contiguous memory
    reaches, the practical ceiling of the HBM-bound calls at that size."""
    out = []
    sink = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    for nbytes in sizes:
        nsets = sets if nbytes < (256 << 20) else 1
        bufs = [torch.ones(nbytes // 4, dtype=torch.int32, device="cuda") for _ in range(nsets)]

        def one_round():
            for b in bufs:
                fg.stream_read(b, sink)

        for _ in range(3):
            one_round()
        torch.cuda.synchronize()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            one_round()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                one_round()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r = reps if nbytes < (256 << 20) else max(reps // 5, 4)
        res = []
        for _ in range(trials):
            e0.record()
            for _ in range(r):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e-3 / (r * nsets))
        t = float(np.median(res))
        out.append({"bytes": nbytes, "buffers": nsets, "us": round(t * 1e6, 3), "us_min": round(min(res) * 1e6, 3),
                    "gbs": round(nbytes / t / 1e9, 1), "frac_hbm": round(nbytes / t / 1e9 / PEAK_HBM_GBS, 4)})
        log(f"stream read {nbytes / 2**20:.0f} MiB: {out[-1]['us']} us, {out[-1]['gbs']} GB/s")
        del bufs, g
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------- CPU oracle
def cpu_baseline(linears, rows=None, cols=None):
    """The oracle (unchanged) on a bounded sample: by default one whole step
    (every row and every output column of each linear, ~10 s on 16 host
    threads); `rows` / `cols` bound it further.  Timed = activation
    quantization + block-scaled product."""
    import oracle
    from threadpoolctl import threadpool_info

    prepared = []
    for lin in linears:
        nc = lin.n if cols is None else min(cols, lin.n)
        qb, sb = oracle.quantize_blocks(lin.b[:nc])  # offline, untimed (as on the GPU side)
        a = lin.a if rows is None else lin.a[:rows]
        prepared.append((a, qb, sb))
    flops = 0
    t0 = time.perf_counter()
    for a, qb, sb in prepared:
        q, sa = oracle.quantize_groups(a)
        oracle.gemm_nt(q, sa, qb, sb)
        flops += 2 * a.shape[0] * qb.shape[0] * a.shape[1]
    dt = time.perf_counter() - t0
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('architecture')}, {i.get('threading_layer')})"
            for i in info if i.get("user_api") == "blas"]
    m = prepared[0][0].shape[0]
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "blas": ", ".join(blas) or None,
        "host_cpus": os.cpu_count(),
        "kind": "oracle",
        "sample": (f"one whole step: {m} rows x all output columns of each of the {len(linears)} linears"
                   if cols is None else f"{m} rows x the first min(N, {cols}) output columns of each of the "
                   f"{len(linears)} linears")
        + f" (quantize_groups + gemm_nt, FP64, numpy+BLAS); {flops / 1e9:.1f} GFLOP in {dt:.1f} s",
        "seconds": round(dt, 2),
    }


# ------------------------------------------------------- counter calibration
COPY_BYTES = 256 << 20


def copy_calibration(args, torch):
    """A plain device-to-device copy of 256 MiB, for scaling the FETCH_SIZE /
    WRITE_SIZE counters: each launch moves exactly COPY_BYTES each way."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"workload": "copy", "bytes_each_way": COPY_BYTES, "launches": args.warmup + args.steps}))


# --------------------------------------------------------------------- main
def main():
    global NO_CLOCK
    args = parse()
    NO_CLOCK = args.no_clock
    if args.gpus != 1:
        print(
            json.dumps(
                {"error": "fgfp8 runs the block-scaled FP8 linear on one MI355X; sharding over several GPUs "
                 "is described in the design notes, not run", "n_gpus": args.gpus}
            )
        )
        sys.exit(2)
    import torch

    import fine_grained_block_fp8_amd as fg
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')}")

    if args.workload == "copy":
        copy_calibration(args, torch)
        return
    if args.workload == "stream":
        print(json.dumps({"workload": "stream_read", "results": bench_stream(fg, torch, trials=args.trials)}))
        return
    if args.workload == "quantize":
        print(json.dumps({"workload": "activation_quantize_vs_cast", "timing": "median and min of the trials; "
                          "launches back to back over rotating inputs, event time per launch",
                          "results": bench_quantize(fg, torch, trials=args.trials)}))
        return
    recipe = {"prefill_ue8m0": "ue8m0", "prefill_mx": "mx"}.get(args.workload, "fp32")
    if args.workload in ("prefill", "prefill_ue8m0", "prefill_mx"):
        linears = workloads.prefill_linears()
        workload = "qwen3_8b_prefill_linears_m2048" + {"ue8m0": "_ue8m0_recipe", "mx": "_mxfp8_recipe"}.get(recipe, "")
    elif args.workload == "decode":
        linears = [workloads.decode_linear(1, 12288, 4096), workloads.decode_linear(1, 4096, 12288)]
        workload = "decode_m1_linears"
    elif args.workload == "square8k":
        linears = [workloads.square_linear(8192, 8192, 8192)]
        workload = "square_8192x8192x8192"
    elif args.workload == "square16k":
        linears = [workloads.square_linear(16384, 16384, 8192)]
        workload = "square_16384x16384x8192"
    elif args.workload == "moe_masked":
        linears = None
        workload = "moe_masked_32experts_1024tok_zipf1.1_top4_k7168_n4096"
    elif args.workload == "moe_layer":
        linears = None
        workload = "moe_layer_32experts_8192tok_zipf1.1_top4_h7168_i2048"
    else:
        linears = None
        workload = "moe_32experts_zipf1.1_top4_k7168_n4096"

    if linears is not None:
        log(f"workload {workload}: " + ", ".join(f"{l.name} [{fg.describe_gemm(l.m, l.n, l.k)}]" for l in linears))
        preps, elapsed, per, timed, clock = bench_linears(linears, args.steps, args.warmup, fg, torch,
                                                            recipe=recipe, trials=args.trials)
        total_flops = sum(l.flops for l in linears)
        trials = trial_stats(elapsed, args.steps)
        ms_per_step = trials["ms_per_step_median"]
        value = total_flops / (ms_per_step * 1e-3) / 1e12
        gemm_s = sum(r["_gemm_s"] for r in per)
        roof = roofline_of(per, timed)
        del preps
    elif args.workload == "moe_masked":
        value, ms_per_step, per, roof, gemm_s, total_flops = bench_masked(args, fg, torch, workloads)
        trials = clock = None
    elif args.workload == "moe_layer":
        value, ms_per_step, per, roof, gemm_s, total_flops = bench_moe_layer(args, fg, torch, workloads)
        trials = clock = None
    else:
        obj = bench_moe(args, fg, torch, workloads)
        value, ms_per_step, per, roof, gemm_s, total_flops = (obj["tflops_useful_median"], obj["ms_median"],
                                                             obj["rows"], obj["roofline"], obj["_gemm_s"],
                                                             obj["_flops"])
        trials, clock = obj["timing"], obj["gpu_clock"]
    torch.cuda.empty_cache()

    extra = {}
    if args.workload == "prefill" and not args.no_extra:
        # The other two shapes the targets name, timed as objects of their own
        # (each: act-quant + product per step, trials, clock, roofline).
        for key, lin in (("square_8192", workloads.square_linear(8192, 8192, 8192)),
                         ("square_16384x16384x8192", workloads.square_linear(16384, 16384, 8192))):
            log(f"{key}: {fg.describe_gemm(lin.m, lin.n, lin.k)}")
            extra[key] = bench_object(lin, args.steps, args.warmup, fg, torch, args.trials)
            del lin
            torch.cuda.empty_cache()
        extra["moe_grouped_zipf32"] = bench_moe(args, fg, torch, workloads)
        for v in extra.values():
            for k in [k for k in v if k.startswith("_") or k == "rows"]:
                del v[k]
        torch.cuda.empty_cache()

    decode = stream = None
    if args.workload in ("prefill", "decode") and not args.no_decode:
        decode = bench_decode(fg, torch, reps=args.decode_reps, trials=args.trials)
        for r in decode:
            log(f"decode M={r['m']} N={r['n']} K={r['k']}: graph {r['graph_us']} us {r['graph_gbs']} GB/s; "
                f"eager {r['eager_us']} us")
        stream = bench_stream(fg, torch, sizes=(50_331_648,), trials=args.trials)[0]
        for r in decode:
            r["frac_of_stream_read_48MiB"] = round(r["graph_gbs"] / stream["gbs"], 4)

    cpu = None
    if args.workload == "prefill" and not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(linears)

    per_out = [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in r.items() if not k.startswith("_")}
               for r in per]
    line = {
        "metric": "FP8 block-scaled GEMM TFLOPS (% dense FP8 peak); decode M=1 GB/s (% HBM)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic (seeded N(0,1) activations with 0.1% x20 outliers, N(0,0.02) weights; no trained weights)",
        "config": {
            "workload": workload,
            "steps_are": STEPS_ARE.get(args.workload, STEPS_ARE["prefill"]),
            "linears": per_out,
            "linears_timing": "per-linear pass before the timed region (three events per linear); "
                              "the timed region records events only around the dominant kernel's launches",
            "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 4),
            "gemm_only_tflops": round(total_flops / gemm_s / 1e12, 2) if gemm_s else None,
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "decode": decode,
        "stream_ceiling": stream,
        "timing": trials,
        "gpu_clock": clock,
        **extra,
    }
    print(json.dumps(line), flush=True)


def bench_moe(args, fg, torch, workloads, steps=None) -> dict:
    """The M-grouped contiguous product on the 32-expert Zipf(1.1) top-4
    layout (K = 7168, N = 4096): one step = act-quant of the padded layout +
    the grouped product; `args.trials` timed regions; TFLOP/s on the useful
    (routed-row) FLOPs, padded FLOPs beside it."""
    steps = steps or args.steps
    g = workloads.moe_grouped()
    x = dev_bf16(g.a, torch)
    q, sa = fg.quantize_fp8_groups(x)
    w = dev_bf16(g.b.reshape(g.num_groups * g.n, g.k), torch)
    g.b = None
    qb, sb = fg.quantize_fp8_blocks(w)
    del w
    qb = qb.view(g.num_groups, g.n, g.k)
    sb = sb.view(g.num_groups, g.n // 128, g.k // 128)
    idx = torch.from_numpy(g.m_indices).cuda()
    d = torch.empty((g.m, g.n), dtype=torch.bfloat16, device="cuda")

    def step(ev=None):
        if ev:
            ev[0].record()
        fg.quantize_fp8_groups(x, out=(q, sa))
        if ev:
            ev[1].record()
        fg.m_grouped_fp8_gemm_nt_contiguous((q, sa), (qb, sb), d, idx)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ahead = GpuAhead(torch)
    probe = [HipEvent(torch) for _ in range(3)]
    host_step = host_enqueue_seconds(lambda: step(probe), torch)
    gpu_step = gpu_step_seconds(step, torch)
    elapsed, gts, qts = [], [], []
    for _ in range(args.trials):
        evs = [[HipEvent(torch) for _ in range(3)] for _ in range(steps)]
        e_first, e_last = HipEvent(torch), HipEvent(torch)
        torch.cuda.synchronize()
        ahead.lead_in(host_step * steps, gpu_step * steps)
        e_first.record()
        for s in range(steps):
            step(evs[s])
        e_last.record()
        torch.cuda.synchronize()
        elapsed.append(e_first.elapsed_time(e_last) * 1e-3)
        gts += [e[1].elapsed_time(e[2]) * 1e-3 for e in evs]
        qts += [e[0].elapsed_time(e[1]) * 1e-3 for e in evs]
    clock = sustained_clock(step, torch, float(np.median(elapsed)) / steps)
    gt, qt = float(np.mean(gts)), float(np.mean(qts))
    st = trial_stats(elapsed, steps)
    flops = g.useful_flops
    padded = 2 * g.m * g.n * g.k
    plan = fg.describe_grouped(g.m, g.n, g.k)
    kernel = ("grouped_gemm_nt_persistent_kernel<" if plan.endswith(" persistent") else "grouped_gemm_nt_kernel<") + \
        plan.split()[0] + ">"
    log(f"moe grouped: ms/step {st['ms_per_step']}; gemm mean {gt * 1e6:.1f} us")
    rows = [{"name": g.name, "m_pad": g.m, "n": g.n, "k": g.k, "groups": g.num_groups, "quant_us": qt * 1e6,
             "gemm_us": gt * 1e6, "gemm_tflops_useful": flops / gt / 1e12, "gemm_tflops_padded": padded / gt / 1e12,
             "_gemm_s": gt}]
    nbytes = (g.m * g.k + 4 * g.m * (g.k // 128) + g.num_groups * (g.n * g.k + 4 * (g.n // 128) * (g.k // 128))
              + 2 * g.m * g.n)
    roof = {"bound": "mfma", "kernel": kernel, "achieved": round(flops / gt / 1e12, 1), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(flops / gt / 1e12 / PEAK_FP8_TFLOPS, 4),
            "traffic": recorded_traffic(kernel, (g.m, g.n, g.k)),
            "algorithmic_gflop_per_launch": round(flops / 1e9, 3),
            "algorithmic_flops_are": "useful: 2 x routed rows x N x K (padding rows excluded)",
            "padded_gflop_per_launch": round(padded / 1e9, 3), "algorithmic_bytes_per_launch": nbytes,
            "mean_launch_us": round(gt * 1e6, 2), "launches": len(gts),
            "launch_timing": "HIP events around each launch of the grouped product inside the timed trials"}
    ms = st["ms_per_step_median"]
    return {
        "workload": g.name, "m_pad": g.m, "routed_rows": int(g.sizes.sum()), "n": g.n, "k": g.k,
        "groups": g.num_groups, "kernel": kernel,
        "steps_are": STEPS_ARE["moe"],
        "ms_min": st["ms_per_step_min"], "ms_median": ms,
        "tflops_useful_median": round(flops / (ms * 1e-3) / 1e12, 1),
        "tflops_padded_median": round(padded / (ms * 1e-3) / 1e12, 1),
        "gemm_us": round(gt * 1e6, 2), "gemm_tflops_useful": round(flops / gt / 1e12, 1),
        "gemm_tflops_padded": round(padded / gt / 1e12, 1), "quant_us": round(qt * 1e6, 2),
        "timing": st, "gpu_clock": clock, "roofline": roof, "rows": rows,
        "_gemm_s": gt, "_flops": flops,
    }


def bench_masked(args, fg, torch, workloads):
    """Decode-time MoE: the masked grouped product over a dispatch buffer
    (32 experts, 1024 tokens routed top-4 by Zipf(1.1), K = 7168, N = 4096);
    one step = quantize the buffer's real rows (the counts stay on the
    device) + the masked product."""
    c = workloads.moe_masked()
    g, mm, n, k = c.num_groups, c.max_m, c.n, c.k
    x = dev_bf16(c.a.reshape(g * mm, k), torch)
    q, sa = fg.quantize_fp8_groups(x)
    w = dev_bf16(c.b.reshape(g * n, k), torch)
    qb, sb = fg.quantize_fp8_blocks(w)
    del w
    qb, sb = qb.view(g, n, k), sb.view(g, n // 128, k // 128)
    masked = torch.from_numpy(c.masked_m.astype(np.int32)).cuda()
    d = torch.empty((g, mm, n), dtype=torch.bfloat16, device="cuda")
    qv, xv = q.view(g, mm, k), x.view(g, mm, k)

    def step(ev=None):
        if ev:
            ev[0].record()
        fg.quantize_fp8_groups_masked(xv, masked, out=(qv, sa))
        if ev:
            ev[1].record()
        fg.m_grouped_fp8_gemm_nt_masked((qv, sa), (qb, sb), d, masked, c.expected_m)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[HipEvent(torch) for _ in range(3)] for _ in range(args.steps)]
    ahead = GpuAhead(torch)
    probe = [HipEvent(torch) for _ in range(3)]
    host_step = host_enqueue_seconds(lambda: step(probe), torch)
    gpu_step = gpu_step_seconds(step, torch)
    e_first, e_last = HipEvent(torch), HipEvent(torch)
    torch.cuda.synchronize()
    ahead.lead_in(host_step * args.steps, gpu_step * args.steps)
    e_first.record()
    for s in range(args.steps):
        step(evs[s])
    e_last.record()
    torch.cuda.synchronize()
    elapsed = e_first.elapsed_time(e_last) * 1e-3
    gt = np.mean([e[1].elapsed_time(e[2]) for e in evs]) * 1e-3
    qt = np.mean([e[0].elapsed_time(e[1]) for e in evs]) * 1e-3
    flops = float(2 * int(c.masked_m.sum()) * n * k)
    kernel = "masked_gemm_nt_kernel (128-row tile chosen from expected_m)"
    per = [{"name": c.name, "max_m": mm, "expected_m": c.expected_m, "rows": int(c.masked_m.sum()), "n": n, "k": k,
            "groups": g, "quant_us": qt * 1e6, "gemm_us": gt * 1e6, "gemm_tflops_useful": flops / gt / 1e12,
            "_gemm_s": gt}]
    # At ~128 rows per expert the product reads every expert's weight once
    # (940 MB) for ~240 GFLOP: ~250 FLOP/B, below the MFMA ridge (~625), so
    # the bound is HBM.  Algorithmic bytes: the weights and weight scales of
    # the experts with rows, their activation rows and scales, their outputs.
    rows = int(c.masked_m.sum())
    active = int((c.masked_m > 0).sum())
    nbytes = active * (n * k + 4 * (n // 128) * (k // 128)) + rows * k + 4 * rows * (k // 128) + 2 * rows * n
    gbs = nbytes / gt / 1e9
    roof = {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "algorithmic_bytes_per_launch": nbytes,
            "useful_tflops": round(flops / gt / 1e12, 1), "mean_launch_us": round(gt * 1e6, 2)}
    return flops * args.steps / elapsed / 1e12, elapsed / args.steps * 1e3, per, roof, gt, flops


def bench_moe_layer(args, fg, torch, workloads):
    """The FP8 MoE layer: one step = route -> gather+quantize -> grouped
    product (gate_up, N = 2I) with SiLU-times-up+quantize in its epilogue
    (two launches with --moe-unfused) -> grouped product (down, N = H) ->
    weighted combine, every buffer sized by the padded-row upper bound so that
    nothing waits for the host.  Value: useful TFLOP/s of the two products
    (routed rows only) over the whole step."""
    c = workloads.moe_layer()
    g, hd, it, t, tk = c.experts, c.hidden, c.inter, c.tokens, c.topk
    x = dev_bf16(c.x, torch)
    idx = torch.from_numpy(c.topk_idx.astype(np.int32)).cuda()
    wts = torch.from_numpy(c.topk_weights).cuda()
    q1 = torch.empty((g, 2 * it, hd), dtype=torch.float8_e4m3fn, device="cuda")
    s1 = torch.empty((g, 2 * it // 128, hd // 128), dtype=torch.float32, device="cuda")
    q2 = torch.empty((g, hd, it), dtype=torch.float8_e4m3fn, device="cuda")
    s2 = torch.empty((g, hd // 128, it // 128), dtype=torch.float32, device="cuda")
    for e in range(g):
        qa, sa = fg.quantize_fp8_blocks(dev_bf16(c.w1[e], torch))
        q1[e].copy_(qa)
        s1[e].copy_(sa)
        qa, sa = fg.quantize_fp8_blocks(dev_bf16(c.w2[e], torch))
        q2[e].copy_(qa)
        s2[e].copy_(sa)
    del qa, sa
    c.w1 = c.w2 = None
    m = fg.moe_max_padded_rows(t, tk, g)
    dev = "cuda"
    route = (torch.empty(g, dtype=torch.int32, device=dev), torch.empty(m, dtype=torch.int32, device=dev),
             torch.empty(m, dtype=torch.int32, device=dev), torch.empty((t, tk), dtype=torch.int32, device=dev),
             torch.empty(max(fg.moe_route_workspace_bytes(t, g), 16), dtype=torch.uint8, device=dev))
    a1 = (torch.empty((m, hd), dtype=torch.float8_e4m3fn, device=dev),
          torch.empty((hd // 128, m), dtype=torch.float32, device=dev))
    h = torch.empty((m, 2 * it), dtype=torch.bfloat16, device=dev)
    a2 = (torch.empty((m, it), dtype=torch.float8_e4m3fn, device=dev),
          torch.empty((it // 128, m), dtype=torch.float32, device=dev))
    y = torch.empty((m, hd), dtype=torch.bfloat16, device=dev)
    out = torch.empty((t, hd), dtype=torch.bfloat16, device=dev)
    fused = not args.moe_unfused
    names = (["route", "gather_quant", "gemm_gate_up_silu_quant", "gemm_down", "combine"] if fused else
             ["route", "gather_quant", "gemm_gate_up", "silu_mul_quant", "gemm_down", "combine"])

    def step(ev=None):
        n_ev = [0]

        def mark():
            if ev:
                ev[n_ev[0]].record()
            n_ev[0] += 1
        mark()
        _counts, m_idx, tok, row_of = fg.moe_route_contiguous(idx, g, out=route)
        mark()
        fg.moe_gather_quantize_tokens(x, row_of, tok, out=a1)
        mark()
        if fused:
            fg.moe_gate_up_silu_quantize(a1, (q1, s1), m_idx, out=a2)
        else:
            fg.m_grouped_fp8_gemm_nt_contiguous(a1, (q1, s1), h, m_idx)
            mark()
            fg.silu_mul_quantize(h, m_idx, out=a2)
        mark()
        fg.m_grouped_fp8_gemm_nt_contiguous(a2, (q2, s2), y, m_idx)
        mark()
        fg.moe_combine(y, row_of, wts, out=out)
        mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[HipEvent(torch) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    ahead = GpuAhead(torch)
    probe = [HipEvent(torch) for _ in range(len(names) + 1)]
    host_step = host_enqueue_seconds(lambda: step(probe), torch)
    gpu_step = gpu_step_seconds(step, torch)
    e_first, e_last = HipEvent(torch), HipEvent(torch)
    torch.cuda.synchronize()
    ahead.lead_in(host_step * args.steps, gpu_step * args.steps)
    e_first.record()
    for s_ in range(args.steps):
        step(evs[s_])
    e_last.record()
    torch.cuda.synchronize()
    elapsed = e_first.elapsed_time(e_last) * 1e-3
    stage = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e-3 for i, n in enumerate(names)}
    pairs = int(c.topk_idx.size)
    f1 = 2.0 * pairs * (2 * it) * hd
    f2 = 2.0 * pairs * hd * it
    flops = f1 + f2
    m_real = padded_rows_of(route[0])
    gu = "gemm_gate_up_silu_quant" if fused else "gemm_gate_up"
    per = [{"name": c.name, "m_pad_max": m, "m_pad": m_real, "pairs": pairs, "hidden": hd, "inter": it, "experts": g,
            "gate_up_fused": fused, **{f"{n}_us": stage[n] * 1e6 for n in names},
            "gate_up_tflops_useful": f1 / stage[gu] / 1e12,
            "down_tflops_useful": f2 / stage["gemm_down"] / 1e12, "_gemm_s": stage[gu] + stage["gemm_down"]}]
    gemm_s = stage[gu] + stage["gemm_down"]
    if fused:
        # the dominant kernel: the gate_up product with its SiLU.mul+quantize epilogue
        roof = {"bound": "mfma", "kernel": "grouped_gemm_silu_kernel<tile128x256_w2x4> (gate_up + SiLU.mul + quantize)",
                "achieved": round(f1 / stage[gu] / 1e12, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(f1 / stage[gu] / 1e12 / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": f1, "mean_launch_us": round(stage[gu] * 1e6, 2)}
    else:
        # both products run m_grouped_fp8_gemm_nt_contiguous: the per-launch average
        plans = sorted({fg.describe_grouped(m, 2 * it, hd), fg.describe_grouped(m, hd, it)})
        roof = {"bound": "mfma", "kernel": "m_grouped_fp8_gemm_nt_contiguous [" + "; ".join(plans) +
                "] (gate_up and down launches averaged)",
                "achieved": round(flops / gemm_s / 1e12, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(flops / gemm_s / 1e12 / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "algorithmic_flops_per_launch": flops / 2, "mean_launch_us": round(gemm_s / 2 * 1e6, 2)}
    return flops * args.steps / elapsed / 1e12, elapsed / args.steps * 1e3, per, roof, gemm_s, flops


def padded_rows_of(counts):
    """Rows the layout really uses: every expert's count rounded up to 128
    (read after the timed region)."""
    return int((((counts.long() + 127) // 128) * 128).sum().item())


if __name__ == "__main__":
    main()
