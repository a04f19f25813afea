"""Throughput of the fused clamped-SwiGLU x probs activation on one MI355X.

A step is one pass of the whole hot path over one batch: the forward kernel, then
the backward kernel (which also reduces grad_probs), on the seeded synthetic
inputs of a workload (default: the 1.1 GB "headline" shape, rows 53760, inter
2048), already resident in HBM. W untimed warm-up steps, then K timed steps
bracketed by device synchronisation.

Order of the legs: the streaming ceilings, the timed steps, each kernel back to back,
the cold launches, the CPU baseline. The ceilings come first so that a device which sat
idle while the inputs were drawn has left its clock ramp before the timed steps.

Printed JSON line (stdout):
  value        whole-job algorithmic GB/s = (fwd + bwd algorithmic bytes) / wall time per
               timed step (ms_per_step; device_ms_per_step is the same from two stream
               events around the timed steps, with none between the kernels)
  fwd, bwd     per-kernel duration over K more steps run right after the timed ones, in
               which each launch records its own start and end into a pair of events
               (the library's timed entry points, hipExtLaunchKernel): the kernel alone;
               average, min, median, max, and the GB/s and HBM fraction the average
               gives (the roofline uses the average; a few slow launches move it, the
               median much less). us_back_to_back: the kernel alone, launched
               back to back (median of five windows of 20 launches between one pair of
               stream events); frac_of_best_ceiling: its GB/s over the best ceiling
               measured at its read:write mix
  roofline     for the dominant kernel (the backward): algorithmic bytes per launch /
               its average duration, against the 8 TB/s MI355X HBM peak; traffic =
               HBM bytes per launch from the committed rocprofv3 counter summary, and
               trace_us the average from the committed rocprofv3 kernel trace, each when
               it was taken on the current kernel source (else null / absent)
  cold         the same kernels one launch at a time after a read of an unrelated 1 GiB
               buffer (evicts the 256 MB Infinity Cache without leaving dirty lines), so
               no input can come from the previous launch's cache state; median and
               minimum of --cold-reps launches (default 30)
  hbm_probe    streaming ceilings at the same bytes: the in-repo probe (1:1 copy, 2:1 and
               3:2 read:write, read-only over three arrays, write-only over two) and,
               sharing no code with the kernels, torch copy_, a bf16
               torch.add and hipMemcpyDtoDAsync. With --op, the probe at each kernel's
               own read:write mix and size, and the kernel's fraction of it
With --op (a MoE operation), the step is that op's kernels in order; kernels.<name>.us is
the kernel alone back to back, timed the same way as its probe (time_windows), and cold_*
as above.
  cpu_baseline the CPU oracle (test infrastructure, untuned) on the same inputs,
               timed on this host's cores (cores = threads used, host_cores = the
               process's CPU affinity)
Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s (fwd, bwd) and % of MI355X HBM peak at 1.1 GB shape"
CSRC = os.path.join(ROOT, "memory_bound_elementwise_amd", "csrc")
KERNEL_SRC = [os.path.join(CSRC, "swiglu_probs.hip"), os.path.join(CSRC, "cdna4_stream.h")]
MOE_SRC = [os.path.join(CSRC, "moe_elementwise.hip"), os.path.join(CSRC, "cdna4_stream.h")]
COUNTERS = os.path.join(ROOT, "profiles", "pmc_swiglu_probs_headline.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(paths=None) -> str:
    """sha256[:16] of the kernel sources' code: comments and whitespace are left out, so
    a counter summary stays valid across edits that change no instruction."""
    h = hashlib.sha256()
    for p in (paths or KERNEL_SRC):
        with open(p) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, key: str = "bwd", path: str = COUNTERS, sources=None):
    """HBM bytes per launch of kernel `key` from a committed counter summary, or None
    when it is missing, for another workload, or taken on other kernel sources."""
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("workload") != workload or d.get("kernel_source_sha256_16") != kernel_source_hash(sources):
        return None
    return d.get(key, {}).get("hbm_bytes_per_launch")


TRACE = os.path.join(ROOT, "profiles", "trace_swiglu_probs_headline.json")


def trace_average(workload: str, key: str = "bwd", path: str = TRACE):
    """Kernel `key`'s durations from the committed rocprofv3 kernel trace of this bench:
    rocprofv3's average over every call and the average over the launches that record
    their own events (the ones fwd.us / bwd.us average here). None when the summary is
    missing, for another workload, or taken on other kernel sources."""
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("workload") != workload or d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    k = d.get(key)
    if not k:
        return None
    return {"trace_us": k.get("average_us"), "trace_us_launch_event_steps": k.get("launch_event_steps_us")}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"



MOE_OPS = {
    "residual_add": "fused MoE residual add (bf16)",
    "router_weight": "router-weight multiply, forward + backward (bf16)",
    "squared_relu": "soft-clamped squared ReLU x probs (bf16)",
    "unpermute": "token-local unpermute in expert order (bf16 in, fp32 out)",
}


DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence


class TimingEvents:
    """HIP events for timing only, on torch's current stream of cuda:0 (the stream the
    kernels are launched on). They are created with hipEventDisableSystemFence: recording
    a default event also makes a system-scope release, whose cache writeback the stream
    waits for, and timing needs only the timestamps (the final device synchronisation
    orders everything). On MI355X that took a fwd+bwd step with two events from 281.6 to
    278.0 us (275.0 with none). torch's Event cannot be given the flag, so this calls
    the HIP runtime torch has loaded."""

    @staticmethod
    def _loaded_runtime() -> str:
        """Path of the HIP runtime already mapped into this process (the one torch uses):
        opening that same file returns the loaded library, never a second copy."""
        with open("/proc/self/maps") as f:
            for line in f:
                fields = line.split()
                if len(fields) >= 6 and os.path.basename(fields[5]).startswith("libamdhip64.so"):
                    return fields[5]
        raise RuntimeError("the HIP runtime is not loaded in this process")

    def __init__(self, count: int, flags: int = DISABLE_SYSTEM_FENCE):
        import ctypes
        import torch
        torch.cuda.init()
        self._ct = ctypes
        self._hip = hip = ctypes.CDLL(self._loaded_runtime())
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                            ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._stream = ctypes.c_void_p(torch.cuda.current_stream(0).cuda_stream)
        self._ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            rc = hip.hipEventCreateWithFlags(ctypes.byref(e), flags)
            if rc != 0:
                self.close()
                raise RuntimeError(f"hipEventCreateWithFlags failed: hipError_t {rc}")
            self._ev.append(e)

    def handle(self, i: int) -> int:
        """The hipEvent_t of event i, for a launch that records into it."""
        return self._ev[i].value

    def record(self, i: int) -> None:
        rc = self._hip.hipEventRecord(self._ev[i], self._stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: hipError_t {rc}")

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds from event i to event j; both must have completed."""
        ms = self._ct.c_float()
        rc = self._hip.hipEventElapsedTime(self._ct.byref(ms), self._ev[i], self._ev[j])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: hipError_t {rc}")
        return float(ms.value)

    def close(self) -> None:
        for e in self._ev:
            self._hip.hipEventDestroy(e)
        self._ev = []


def time_kernels(kernels, steps, warmup, cold_reps):
    """kernels: list of (name, launch), one step being each launched once in order.
    Returns (wall ms per step, device ms per step, {name: ms per launch back to back},
    {name: (median, min) cold ms}) (the last empty when cold_reps is 0).

    The step timing has no event between the kernels: two stream events bracket the
    `steps` timed steps (each event costs the stream several microseconds on MI355X,
    about as long as a small kernel's tail). Each kernel is then timed alone by
    time_windows, the same back-to-back windows the streaming probe is timed with, so
    kernel and probe figures compare like with like. Cold launches are timed one at a
    time, each after a cache-evicting read, between two events."""
    import numpy as np
    import torch
    for _ in range(warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    sev = TimingEvents(2)
    t0 = time.perf_counter()
    sev.record(0)
    for _ in range(steps):
        for _, fn in kernels:
            fn()
    sev.record(1)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    dev_ms = sev.elapsed_ms(0, 1) / steps
    sev.close()
    per = {name: time_windows(fn) for name, fn in kernels}
    cold = {}
    if cold_reps > 0:
        evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
        for name, fn in kernels:
            ts = []
            ev = TimingEvents(2)
            for _ in range(cold_reps):
                evict.sum(dtype=torch.int64)
                ev.record(0)
                fn()
                ev.record(1)
                torch.cuda.synchronize()
                ts.append(ev.elapsed_ms(0, 1))
            ev.close()
            cold[name] = (float(np.median(ts)), float(np.min(ts)))
        del evict
        torch.cuda.empty_cache()  # later buffers (the probe's) get memory of their own
    return wall, dev_ms, per, cold


def time_windows(fn, reps=20, warmup=20, windows=5):
    """Average ms per launch of fn: `warmup` untimed launches, then `windows` windows of
    `reps` back-to-back launches, each window timed with TimingEvents on the launch
    stream; the median window is returned. Right after host-synchronised work one window
    of 20 launches after 3 (or even 20) warm-up launches ran the residual add's 3:1 probe
    at 3.5-5.2 instead of 6.5 TB/s: the device takes a few milliseconds to return to
    full speed, so a single short window can fall inside that."""
    import numpy as np
    import torch
    for _ in range(warmup):
        fn()
    ev = TimingEvents(windows + 1)
    ev.record(0)
    for w in range(windows):
        for _ in range(reps):
            fn()
        ev.record(w + 1)
    torch.cuda.synchronize()
    ms = [ev.elapsed_ms(w, w + 1) / reps for w in range(windows)]
    ev.close()
    return float(np.median(ms))


def time_probe(srcs, dsts, reps=20, warmup=20, windows=5):
    """time_windows of the streaming probe moving srcs -> dsts."""
    from memory_bound_elementwise_amd.hbm_probe import hbm_probe_stream
    return time_windows(lambda: hbm_probe_stream(srcs, dsts), reps, warmup, windows)


def streaming_ceilings(n_elems, dev):
    """The device's streaming ceilings at the activation's byte counts: the in-repo probe
    at 1:1, 2:1 and 3:2 read:write, and, as ceilings that share no code with the kernels,
    torch's own copy_ (1:1) and bf16 add (2:1) and hipMemcpyDtoDAsync (1:1), each over
    arrays of n_elems bf16 elements (as large as one half of x). Every figure is
    time_windows' median window; GB/s counts the bytes each call reads and writes."""
    import ctypes
    import torch
    bufs = [torch.empty(n_elems, dtype=torch.bfloat16, device=dev) for _ in range(5)]
    for b in bufs:
        b.fill_(1)
    i16 = [b.view(torch.int16) for b in bufs]
    nbytes = n_elems * 2
    hip = ctypes.CDLL(TimingEvents._loaded_runtime())
    hip.hipMemcpyDtoDAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream(0).cuda_stream)

    def memcpy():
        rc = hip.hipMemcpyDtoDAsync(bufs[3].data_ptr(), bufs[0].data_ptr(), nbytes, stream)
        if rc != 0:
            raise RuntimeError(f"hipMemcpyDtoDAsync failed: hipError_t {rc}")

    from memory_bound_elementwise_amd.hbm_probe import hbm_probe_fill, hbm_probe_read, hbm_probe_stream
    sink = torch.empty(4, dtype=torch.int32, device=dev)
    cases = [
        ("copy_1r1w", "in-repo probe", lambda: hbm_probe_stream(i16[:1], i16[3:4]), 2),
        ("fwd_like_2r1w", "in-repo probe", lambda: hbm_probe_stream(i16[:2], i16[3:4]), 3),
        ("bwd_like_3r2w", "in-repo probe", lambda: hbm_probe_stream(i16[:3], i16[3:5]), 5),
        # the two ends of the read:write range (the sources hold bf16 1.0, 0x3f80 per
        # half-word, whose XOR over three arrays is never the key)
        ("read_only_3r", "in-repo probe", lambda: hbm_probe_read(i16[:3], 0xFFFFFFFF, sink), 3),
        ("write_only_2w", "in-repo probe", lambda: hbm_probe_fill(i16[3:5], 0x3F803F80), 2),
        ("torch_copy_1r1w", "torch Tensor.copy_", lambda: bufs[3].copy_(bufs[0]), 2),
        ("torch_add_2r1w", "torch.add (bf16)", lambda: torch.add(bufs[0], bufs[1], out=bufs[3]), 3),
        ("hip_memcpy_1r1w", "hipMemcpyDtoDAsync", memcpy, 2),
    ]
    out = {}
    for name, kind, fn, arrays in cases:
        ms = time_windows(fn)
        moved = arrays * nbytes
        out[name] = {"kind": kind, "bytes": moved, "us": round(ms * 1e3, 2),
                     "GB/s": round(moved / (ms * 1e6), 1),
                     "frac_of_peak": round(moved / (ms * 1e6) / HBM_PEAK_GBS, 4)}
        log(f"ceiling {name} ({kind}): {out[name]['GB/s']} GB/s")
    del bufs, i16, sink
    torch.cuda.empty_cache()
    return out


def time_launches(kernels, steps, warmup):
    """kernels: list of (name, launch); launch(events) enqueues one kernel and, given a
    (start, stop) pair of event handles, has the launch itself record the kernel's start
    and end into them (the library's timed entry points).

    `warmup` untimed steps (each kernel once, in order), then the timed region: `steps`
    steps bracketed by device synchronisation, with no event between the kernels (two
    stream events bracket the whole region), giving the wall and the device ms per step.
    Then `steps` more steps in which every launch records its own start and end, giving
    each kernel's durations. Those events cost the stream about 7 us per launch on
    MI355X (a step took 283 against 272 us), so they stay out of the step timing.
    Returns (wall ms per step, device ms per step, {name: [ms per launch]})."""
    import torch
    for _ in range(warmup):
        for _, fn in kernels:
            fn(None)
    torch.cuda.synchronize()
    sev = TimingEvents(2)
    t0 = time.perf_counter()
    sev.record(0)
    for _ in range(steps):
        for _, fn in kernels:
            fn(None)
    sev.record(1)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    dev_ms = sev.elapsed_ms(0, 1) / steps
    sev.close()
    n = len(kernels)
    kev = TimingEvents(2 * n * steps, flags=0)
    for s in range(steps):
        for i, (_, fn) in enumerate(kernels):
            k = 2 * (s * n + i)
            fn((kev.handle(k), kev.handle(k + 1)))
    torch.cuda.synchronize()
    per = {name: [kev.elapsed_ms(2 * (s * n + i), 2 * (s * n + i) + 1) for s in range(steps)]
           for i, (name, _) in enumerate(kernels)}
    kev.close()
    return wall, dev_ms, per


def time_cold(kernels, reps):
    """Each kernel alone, `reps` times, each launch after a read of an unrelated 1 GiB
    buffer (evicts the 256 MB Infinity Cache without leaving dirty lines), timed by the
    launch's own start and end events. (median, min) ms per kernel."""
    import numpy as np
    import torch
    evict = torch.ones(1 << 28, dtype=torch.int32, device="cuda:0")
    cold = {}
    for name, fn in kernels:
        ts = []
        ev = TimingEvents(2, flags=0)
        for _ in range(reps):
            evict.sum(dtype=torch.int64)
            fn((ev.handle(0), ev.handle(1)))
            torch.cuda.synchronize()
            ts.append(ev.elapsed_ms(0, 1))
        ev.close()
        cold[name] = (float(np.median(ts)), float(np.min(ts)))
    del evict
    torch.cuda.empty_cache()
    return cold


# The streaming probe's mix for each MoE kernel: (arrays read, arrays written, bytes per
# array), so that it moves the kernel's algorithmic bytes with its read:write ratio.
def moe_probe_mix(op, inp):
    if op == "residual_add":
        return {"residual_add": (3, 1, inp["expert"].size * 2)}
    if op in ("router_weight", "squared_relu"):
        n = inp["x"].size * 2
        return {"fwd": (1, 1, n), "bwd": (2, 1, n)}
    im, hidden = inp["inverse_map"], inp["expert_output"].shape[1]
    return {"unpermute": (2, 1, im.shape[0] * hidden * 4)}   # gathers about 2x the fp32 output


def bench_moe(args) -> int:
    """One JSON line for one of the MoE elementwise operations (see MOE_OPS)."""
    import numpy as np
    import torch

    import memory_bound_elementwise_amd as mbe
    from memory_bound_elementwise_amd.workloads import make_moe_inputs, moe_algorithmic_bytes

    op = args.op
    dev = torch.device("cuda:0")
    log(f"{op}: drawing inputs")
    inp = make_moe_inputs(op, seed=0)

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    if op == "residual_add":
        e, sh, r = bits(inp["expert"]), bits(inp["shared"]), bits(inp["residual"])
        out = torch.empty_like(r)
        kernels = [("residual_add", lambda: mbe.moe_residual_add(e, sh, r, out))]
        nbytes = {"residual_add": moe_algorithmic_bytes(op, inp)}
        shape = {"tokens": r.shape[0], "hidden": r.shape[1]}
    elif op == "router_weight":
        x, g = bits(inp["x"]), bits(inp["grad_out"])
        p = torch.from_numpy(inp["probs"]).to(dev)
        out, gx = torch.empty_like(x), torch.empty_like(x)
        gp = torch.empty_like(p)
        kernels = [("fwd", lambda: mbe.moe_router_weight_fwd(x, p, out)),
                   ("bwd", lambda: mbe.moe_router_weight_bwd(g, x, p, gx, gp))]
        nbytes = {"fwd": moe_algorithmic_bytes(op, inp, "fwd"), "bwd": moe_algorithmic_bytes(op, inp, "bwd")}
        shape = {"rows": x.shape[0], "hidden": x.shape[1]}
    elif op == "squared_relu":
        x, gy = bits(inp["x"]), bits(inp["grad_y"])
        p = torch.from_numpy(inp["probs"]).to(dev)
        y, gx = torch.empty_like(x), torch.empty_like(x)
        gp = torch.empty_like(p)
        s = inp["clamp_scale"]
        kernels = [("fwd", lambda: mbe.moe_squared_relu_probs_fwd(x, p, y, clamp_scale=s)),
                   ("bwd", lambda: mbe.moe_squared_relu_probs_bwd(x, p, gy, gx, gp, clamp_scale=s))]
        nbytes = {"fwd": moe_algorithmic_bytes(op, inp, "fwd"), "bwd": moe_algorithmic_bytes(op, inp, "bwd")}
        shape = {"rows": x.shape[0], "hidden": x.shape[1], "clamp_scale": inp["clamp_scale"]}
    else:
        eo = bits(inp["expert_output"])
        im = torch.from_numpy(inp["inverse_map"]).to(dev)
        out = torch.empty((im.shape[0], eo.shape[1]), dtype=torch.float32, device=dev)
        kernels = [("unpermute", lambda: mbe.moe_unpermute_expert_order(eo, im, out))]
        nbytes = {"unpermute": moe_algorithmic_bytes(op, inp)}
        shape = {"tokens": im.shape[0], "local_experts": im.shape[1], "hidden": eo.shape[1],
                 "routed_pairs": int((inp["inverse_map"] >= 0).sum())}

    # the probe first: see main() (it also brings an idle device out of its clock ramp)
    probe = None
    if not args.no_probe:
        probe = {}
        for name, (ns, nd, arr) in moe_probe_mix(op, inp).items():
            n16 = arr // 32 * 16  # whole 16-byte vectors, as int16 elements
            bufs = [torch.ones(n16, dtype=torch.int16, device=dev) for _ in range(ns + nd)]
            ms = time_probe(bufs[:ns], bufs[ns:])
            moved = (ns + nd) * n16 * 2
            gbs = moved / (ms * 1e6)
            probe[name] = {"mix": f"{ns}:{nd}", "bytes": moved, "us": round(ms * 1e3, 2),
                           "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
            log(f"{op} probe for {name} ({ns}:{nd}): {probe[name]['GB/s']} GB/s")
            del bufs
        torch.cuda.empty_cache()

    log(f"{op}: warm-up {args.warmup}, timing {args.steps} steps")
    wall, dev_ms, per, cold = time_kernels(kernels, args.steps, args.warmup, args.cold_reps)
    total = sum(nbytes.values())
    value = total / (wall * 1e6)
    kern = {}
    for name, _ in kernels:
        avg = per[name]
        kern[name] = {"algorithmic_bytes": nbytes[name], "us": round(avg * 1e3, 2),
                      "GB/s": round(nbytes[name] / (avg * 1e6), 1),
                      "frac_of_peak": round(nbytes[name] / (avg * 1e6) / HBM_PEAK_GBS, 4)}
        if name in cold:
            med, low = cold[name]
            kern[name]["cold_us"] = round(med * 1e3, 2)
            kern[name]["cold_us_min"] = round(low * 1e3, 2)
            kern[name]["cold_GB/s"] = round(nbytes[name] / (med * 1e6), 1)
        log(f"{op} {name}: {kern[name]}")
    dom = max(nbytes, key=nbytes.get)
    traffic = measured_traffic(op, dom, os.path.join(ROOT, "profiles", f"pmc_moe_{op}.json"), MOE_SRC)

    if probe:
        for name in probe:
            probe[name]["kernel_frac_of_probe"] = round(kern[name]["GB/s"] / probe[name]["GB/s"], 4)
            log(f"{op} {name}: kernel at {probe[name]['kernel_frac_of_probe']:.3f} of its probe")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import oracle.moe as mo
        orc = mo.get()
        threads = oracle.default_threads()
        # the oracle on the whole of the same inputs (each op's full batch runs in about a
        # second on a GPU's share of host cores), repeated up to ~cpu_seconds
        spent, reps, moved = 0.0, 0, 0
        while reps < 1 or (spent < args.cpu_seconds and reps < 50):
            t = time.perf_counter()
            if op == "residual_add":
                orc.residual_add(inp["expert"], inp["shared"], inp["residual"], "bf16", threads=threads)
            elif op == "router_weight":
                orc.router_weight_fwd(inp["x"], "bf16", inp["probs"], "bf16", threads=threads)
                orc.router_weight_bwd(inp["grad_out"], "bf16", inp["x"], "bf16", inp["probs"],
                                      threads=threads)
            elif op == "squared_relu":
                orc.squared_relu_probs(inp["x"], inp["probs"], clamp_scale=inp["clamp_scale"],
                                       threads=threads)
                orc.squared_relu_probs_bwd(inp["x"], inp["probs"], inp["grad_y"],
                                           clamp_scale=inp["clamp_scale"], threads=threads)
            else:
                orc.unpermute(inp["expert_output"], inp["inverse_map"], "f32", threads=threads)
            moved += total
            spent += time.perf_counter() - t
            reps += 1
        cpu = {"value": round(moved / (spent * 1e9), 3), "unit": "GB/s", "cores": threads,
               "host_cores": oracle.host_cores(), "kind": "oracle",
               "sample": (f"the full batch of the same inputs x {reps} reps, {spent:.1f} s, on "
                          f"{threads} threads (OMP_NUM_THREADS caps the host's cores to this GPU's "
                          f"share); {cpu_model()}")}
        log(f"{op}: cpu baseline {cpu['value']} GB/s")

    print(json.dumps({
        "metric": f"achieved HBM GB/s of the {MOE_OPS[op]} and % of MI355X HBM peak",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall, 5), "device_ms_per_step": round(dev_ms, 5),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"moe_{op}", **shape, "io_dtype": "bf16", "seed": 0},
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kern[dom]["frac_of_peak"], "traffic": traffic,
                     "timing": "the kernel alone, launched back to back (median of five windows of "
                               "20 launches, as the probe)"},
        "hbm_probe": probe,
        "cpu_baseline": cpu,
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first; the first ~30 steps of sustained work run through a "
                         "start-up clock transient on MI355X")
    ap.add_argument("--workload", default="headline",
                    choices=["tiny", "mid", "headline", "padded", "edge"])
    ap.add_argument("--op", default="swiglu_probs", choices=["swiglu_probs"] + sorted(MOE_OPS),
                    help="swiglu_probs: the activation fwd+bwd (default); the others: the MoE "
                         "elementwise operations next to it, at the headline MoE shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--cold-reps", type=int, default=30,
                    help="launches of each kernel timed one at a time, each after a cache-evicting "
                         "read; their median and minimum are reported (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent on the oracle baseline")
    ap.add_argument("--fwd-workgroups", type=int, default=0)
    ap.add_argument("--bwd-workgroups", type=int, default=0)
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs on one MI355X and has no multi-GPU "
              f"mode (asked for --gpus {args.gpus}). Rows shard across GPUs with no exchange; "
              f"run one process per GPU instead.", file=sys.stderr)
        return 2

    if args.op != "swiglu_probs":
        return bench_moe(args)

    import numpy as np
    import torch

    from memory_bound_elementwise_amd import load_library, swiglu_probs_bwd, swiglu_probs_fwd
    from memory_bound_elementwise_amd.workloads import WORKLOADS, algorithmic_bytes, make_inputs

    lib = load_library()
    log(f"library {lib._name}")
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} ({props.multi_processor_count} CUs)")
    w = WORKLOADS[args.workload]
    log(f"drawing inputs for {w.name}: rows={w.rows} inter={w.inter}")
    inp = make_inputs(w, seed=0)
    rows, two_inter = inp["x"].shape
    inter = two_inter // 2

    # The ceilings first: besides giving the practical ceiling, their ~0.1 s of streaming
    # brings a device that sat idle while the inputs were drawn out of its clock ramp
    # (after idling, the shader clock needs some 10-30 ms of load to settle; launches
    # timed inside that run up to 20% slow).
    probe = None
    if not args.no_probe:
        probe = streaming_ceilings((rows * inter) // 8 * 8, dev)

    x = torch.from_numpy(inp["x"].view(np.int16)).to(dev)
    gy = torch.from_numpy(inp["grad_y"].view(np.int16)).to(dev)
    probs = torch.from_numpy(inp["probs"]).to(dev)
    n_used = None if inp["n_used"] is None else torch.tensor([inp["n_used"]], dtype=torch.int32, device=dev)
    pm = None if inp["permutation_map"] is None else torch.from_numpy(inp["permutation_map"]).to(dev)
    y = torch.empty((rows, inter), dtype=torch.int16, device=dev)
    gx = torch.empty((rows, two_inter), dtype=torch.int16, device=dev)
    gp = torch.empty((rows,), dtype=torch.float32, device=dev)
    kw = dict(n_used=n_used, permutation_map=pm, zero_padding=inp["zero_padding"])
    L = inp["limit"]
    fwd_bytes = algorithmic_bytes(w, "fwd")
    bwd_bytes = algorithmic_bytes(w, "bwd")
    nbytes = {"fwd": fwd_bytes, "bwd": bwd_bytes}

    kernels = [
        ("fwd", lambda ev: swiglu_probs_fwd(x, probs, y, L, num_workgroups=args.fwd_workgroups, events=ev, **kw)),
        ("bwd", lambda ev: swiglu_probs_bwd(x, probs, gy, gx, gp, L, num_workgroups=args.bwd_workgroups,
                                            events=ev, **kw)),
    ]
    log(f"warm-up {args.warmup} steps, timing {args.steps} steps")
    ms_per_step, dev_ms_per_step, per = time_launches(kernels, args.steps, args.warmup)
    value = (fwd_bytes + bwd_bytes) / (ms_per_step * 1e6)
    res = {}
    for name, _ in kernels:
        t = per[name]
        avg = float(np.mean(t))
        res[name] = {"algorithmic_bytes": nbytes[name], "us": round(avg * 1e3, 2),
                     "us_min": round(min(t) * 1e3, 2), "us_median": round(float(np.median(t)) * 1e3, 2),
                     "us_max": round(max(t) * 1e3, 2),
                     "GB/s": round(nbytes[name] / (avg * 1e6), 1),
                     "frac_of_peak": round(nbytes[name] / (avg * 1e6) / HBM_PEAK_GBS, 4)}
    log(f"fwd {res['fwd']['us']} us ({res['fwd']['GB/s']} GB/s), bwd {res['bwd']['us']} us "
        f"({res['bwd']['GB/s']} GB/s), step {ms_per_step * 1e3:.1f} us ({value:.0f} GB/s)")

    # each kernel alone, back to back: windows of launches between one pair of events
    for name, fn in kernels:
        ms = time_windows(lambda: fn(None))
        res[name]["us_back_to_back"] = round(ms * 1e3, 2)
        if probe:
            mix = "fwd_like_2r1w" if name == "fwd" else "bwd_like_3r2w"
            best = max(probe[m]["GB/s"] for m in probe if m.endswith(mix[-4:]))
            res[name]["frac_of_best_ceiling"] = round(nbytes[name] / (ms * 1e6) / best, 4)
        log(f"{name} back to back: {res[name]['us_back_to_back']} us")

    cold = None
    if args.cold_reps > 0:
        cold_ms = time_cold(kernels, args.cold_reps)
        cold = {"reps": args.cold_reps, "statistic": "median (GB/s from the median)"}
        for name in ("fwd", "bwd"):
            med, low = cold_ms[name]
            cold[f"{name}_us"] = round(med * 1e3, 2)
            cold[f"{name}_us_min"] = round(low * 1e3, 2)
            cold[f"{name}_GB/s"] = round(nbytes[name] / (med * 1e6), 1)
        log(f"cold: fwd {cold['fwd_GB/s']} GB/s, bwd {cold['bwd_GB/s']} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg: the oracle as it stands
        orc = oracle.get()
        threads = oracle.default_threads()
        log(f"cpu baseline: oracle fwd+bwd on the full {w.name} batch, {threads} threads")
        okw = dict(n_used=inp["n_used"], permutation_map=inp["permutation_map"],
                   zero_padding=inp["zero_padding"], threads=threads)
        reps, spent = 0, 0.0
        while reps < 1 or (spent < args.cpu_seconds and reps < 200):
            t = time.perf_counter()
            orc.fwd(inp["x"], inp["probs"], L, **okw)
            orc.bwd(inp["x"], inp["probs"], inp["grad_y"], L, **okw)
            spent += time.perf_counter() - t
            reps += 1
        cpu_step = spent / reps
        cpu = {"value": round((fwd_bytes + bwd_bytes) / (cpu_step * 1e9), 2), "unit": "GB/s",
               "cores": threads, "host_cores": oracle.host_cores(), "kind": "oracle",
               "sample": (f"the full {w.name} batch (fwd then bwd, {fwd_bytes + bwd_bytes} algorithmic "
                          f"bytes) x {reps} reps, {spent:.1f} s total, on {threads} threads "
                          f"(OMP_NUM_THREADS caps the host's cores to this GPU's share); {cpu_model()}"),
               "ms_per_step": round(cpu_step * 1e3, 1)}
        log(f"cpu baseline: {cpu['value']} GB/s")

    traffic = measured_traffic(w.name)
    trace = trace_average(w.name, "bwd")
    roofline = {"bound": "hbm", "kernel": "swiglu_probs_bwd", "achieved": res["bwd"]["GB/s"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": res["bwd"]["frac_of_peak"],
                "traffic": traffic,
                "timing": "each launch records its own start and end (hipExtLaunchKernel events)"}
    if trace is not None:
        roofline.update(trace)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "device_ms_per_step": round(dev_ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": rows, "inter": inter, "limit": L,
                   "n_used": inp["n_used"], "permutation_map": inp["permutation_map"] is not None,
                   "zero_padding": inp["zero_padding"], "io_dtype": "bf16", "probs_dtype": "f32",
                   "math": "fp32", "seed": 0},
        "fwd": res["fwd"],
        "bwd": res["bwd"],
        "roofline": roofline,
        "cold": cold,
        "hbm_probe": probe,
        "cpu_baseline": cpu,
        "context": "pages' only figure: inductor-compiled autograd backward on GB200, ~0.7 ms per "
                   "1.1 GB pass (~1.57 TB/s); another machine and another implementation",
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
