"""Throughput of the fused clamped-SwiGLU x probs activation on one MI355X.

A step is one pass of the whole hot path over one batch: the forward kernel, then
the backward kernel (which also reduces grad_probs), on the seeded synthetic
inputs of a workload (default: the 1.1 GB "headline" shape, rows 53760, inter
2048), already resident in HBM. W untimed warm-up steps, then K timed steps
bracketed by device synchronisation.

Printed JSON line (stdout):
  value        whole-job algorithmic GB/s = (fwd + bwd algorithmic bytes) / step time
  fwd, bwd     per-kernel average duration from HIP events on the launch stream,
               one before the first launch and one after every launch (each launch
               lies between two), and the GB/s and HBM fraction they give
  roofline     for the dominant kernel (the backward): algorithmic bytes per launch /
               its average duration, against the 8 TB/s MI355X HBM peak; traffic =
               HBM bytes per launch from the committed rocprofv3 counter summary when
               it was taken on the current kernel source, else null
  cold         the same kernels timed one launch at a time after a read of an unrelated
               1 GiB buffer (evicts the 256 MB Infinity Cache without leaving dirty
               lines), so no input can come from the previous launch's cache state;
               median and minimum of --cold-reps launches (default 30)
  hbm_probe    plain streaming kernels (1:1 copy, 2:1 and 3:2 read:write) moving the
               same bytes as fwd / bwd: the practical ceiling on this device. With --op,
               the probe at each kernel's own read:write mix and size, and the kernel's
               fraction of it. Median of five windows of 20 back-to-back launches
  cpu_baseline the CPU oracle (test infrastructure, untuned) on the same inputs,
               timed on this host's cores
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


class TimingEvents:
    """HIP events for timing only, on torch's current stream of cuda:0 (the stream the
    kernels are launched on). They are created with hipEventDisableSystemFence: recording
    a default event also makes a system-scope release, whose cache writeback the stream
    waits for, and timing needs only the timestamps (the final device synchronisation
    orders everything). On MI355X that took a fwd+bwd step with two events from 281.6 to
    278.0 us (275.0 with none). torch's Event cannot be given the flag, so this calls
    the HIP runtime torch has loaded."""

    DISABLE_SYSTEM_FENCE = 0x20000000

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

    def __init__(self, count: int):
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
            rc = hip.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE)
            if rc != 0:
                self.close()
                raise RuntimeError(f"hipEventCreateWithFlags failed: hipError_t {rc}")
            self._ev.append(e)

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
    Returns wall ms per step, per-kernel event times (lists, ms) over the timed steps,
    and cold (median, min) ms per kernel (empty when cold_reps is 0).

    One event is recorded before the first launch and one after every launch, on the
    launch stream, so each launch lies between two events and consecutive launches
    share the one between them. Each recorded event costs the stream time (on MI355X,
    with torch's default events, 2 per fwd+bwd step instead of 3 took the step from 283
    to 278 us; with none it was 272 us), so no more are recorded than the per-launch
    durations need, and they are TimingEvents, which skip the system-scope fence."""
    import numpy as np
    import torch
    for _ in range(warmup):
        for _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    n = len(kernels)
    ev = TimingEvents(steps * n + 1)
    t0 = time.perf_counter()
    ev.record(0)
    for s in range(steps):
        for i, (_, fn) in enumerate(kernels):
            fn()
            ev.record(s * n + i + 1)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = {name: [ev.elapsed_ms(s * n + i, s * n + i + 1) for s in range(steps)]
           for i, (name, _) in enumerate(kernels)}
    ev.close()
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
    return wall, per, cold


def time_probe(srcs, dsts, reps=20, warmup=20, windows=5):
    """Average ms per launch of the streaming probe moving srcs -> dsts: `warmup` untimed
    launches, then `windows` windows of `reps` back-to-back launches, each timed with
    TimingEvents on the launch stream; the median window is returned.
    Right after the cold leg's host-synchronised launches, one window of 20 launches
    after 3 (or even 20) warm-up launches ran the residual add's 3:1 probe at 3.5-5.2
    instead of 6.5 TB/s: the device takes a few milliseconds to return to full speed, so
    a single short window can fall inside that."""
    import numpy as np
    import torch
    from memory_bound_elementwise_amd.hbm_probe import hbm_probe_stream
    for _ in range(warmup):
        hbm_probe_stream(srcs, dsts)
    ev = TimingEvents(windows + 1)
    ev.record(0)
    for w in range(windows):
        for _ in range(reps):
            hbm_probe_stream(srcs, dsts)
        ev.record(w + 1)
    torch.cuda.synchronize()
    ms = [ev.elapsed_ms(w, w + 1) / reps for w in range(windows)]
    ev.close()
    return float(np.median(ms))


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

    log(f"{op}: warm-up {args.warmup}, timing {args.steps} steps")
    wall, per, cold = time_kernels(kernels, args.steps, args.warmup, args.cold_reps)
    total = sum(nbytes.values())
    value = total / (wall * 1e6)
    kern = {}
    for name, _ in kernels:
        avg = float(np.mean(per[name]))
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
                           "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                           "kernel_frac_of_probe": round(kern[name]["GB/s"] / gbs, 4)}
            log(f"{op} probe for {name} ({ns}:{nd}): {probe[name]['GB/s']} GB/s; kernel at "
                f"{probe[name]['kernel_frac_of_probe']:.3f} of it")
            del bufs
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle.moe as mo
        orc = mo.get()
        # a bounded sample: the oracle on a leading slice of the same inputs, ~cpu_seconds
        frac = {"residual_add": 1.0, "router_weight": 0.125, "squared_relu": 0.25, "unpermute": 0.25}[op]
        spent, reps, moved = 0.0, 0, 0
        while reps < 1 or (spent < args.cpu_seconds and reps < 50):
            t = time.perf_counter()
            if op == "residual_add":
                orc.residual_add(inp["expert"], inp["shared"], inp["residual"], "bf16")
                moved += total
            elif op == "router_weight":
                n = int(inp["x"].shape[0] * frac)
                orc.router_weight_fwd(inp["x"][:n], "bf16", inp["probs"][:n], "bf16")
                orc.router_weight_bwd(inp["grad_out"][:n], "bf16", inp["x"][:n], "bf16", inp["probs"][:n])
                moved += int(total * n / inp["x"].shape[0])
            elif op == "squared_relu":
                n = int(inp["x"].shape[0] * frac)
                orc.squared_relu_probs(inp["x"][:n], inp["probs"][:n], clamp_scale=inp["clamp_scale"])
                orc.squared_relu_probs_bwd(inp["x"][:n], inp["probs"][:n], inp["grad_y"][:n],
                                           clamp_scale=inp["clamp_scale"])
                moved += int(total * n / inp["x"].shape[0])
            else:
                n = int(inp["inverse_map"].shape[0] * frac)
                orc.unpermute(inp["expert_output"], inp["inverse_map"][:n], "f32")
                moved += int(total * n / inp["inverse_map"].shape[0])
            spent += time.perf_counter() - t
            reps += 1
        cpu = {"value": round(moved / (spent * 1e9), 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{'all' if frac == 1.0 else f'the first {frac:g} of the'} rows of the same "
                         f"inputs x {reps} reps, {spent:.1f} s; {cpu_model()}"}
        log(f"{op}: cpu baseline {cpu['value']} GB/s")

    print(json.dumps({
        "metric": f"achieved HBM GB/s of the {MOE_OPS[op]} and % of MI355X HBM peak",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"moe_{op}", **shape, "io_dtype": "bf16", "seed": 0},
        "kernels": kern,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kern[dom]["GB/s"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kern[dom]["frac_of_peak"], "traffic": traffic},
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

    kernels = [
        ("fwd", lambda: swiglu_probs_fwd(x, probs, y, L, num_workgroups=args.fwd_workgroups, **kw)),
        ("bwd", lambda: swiglu_probs_bwd(x, probs, gy, gx, gp, L, num_workgroups=args.bwd_workgroups, **kw)),
    ]
    log(f"warm-up {args.warmup} steps, timing {args.steps} steps")
    ms_per_step, per, cold_ms = time_kernels(kernels, args.steps, args.warmup, args.cold_reps)
    fwd_ms, bwd_ms = per["fwd"], per["bwd"]
    f_avg, b_avg = float(np.mean(fwd_ms)), float(np.mean(bwd_ms))
    f_gbs, b_gbs = fwd_bytes / (f_avg * 1e6), bwd_bytes / (b_avg * 1e6)
    value = (fwd_bytes + bwd_bytes) / (ms_per_step * 1e6)
    log(f"fwd {f_avg * 1e3:.1f} us ({f_gbs:.0f} GB/s), bwd {b_avg * 1e3:.1f} us ({b_gbs:.0f} GB/s), "
        f"step {ms_per_step * 1e3:.1f} us ({value:.0f} GB/s)")

    cold = None
    if args.cold_reps > 0:
        (cfm, cfl), (cbm, cbl) = cold_ms["fwd"], cold_ms["bwd"]
        cold = {"fwd_us": round(cfm * 1e3, 2), "fwd_us_min": round(cfl * 1e3, 2),
                "fwd_GB/s": round(fwd_bytes / (cfm * 1e6), 1),
                "bwd_us": round(cbm * 1e3, 2), "bwd_us_min": round(cbl * 1e3, 2),
                "bwd_GB/s": round(bwd_bytes / (cbm * 1e6), 1),
                "reps": args.cold_reps, "statistic": "median (GB/s from the median)"}
        log(f"cold: fwd {cold['fwd_GB/s']} GB/s, bwd {cold['bwd_GB/s']} GB/s")

    probe = None
    if not args.no_probe:
        probe = {}
        # same bytes per stream as the kernels: fwd = 2 reads of x/2 + 1 write; bwd = 3 + 2
        nvec_elems = (rows * inter) // 8 * 8
        bufs = [torch.empty(nvec_elems, dtype=torch.int16, device=dev) for _ in range(5)]
        for b in bufs:
            b.fill_(1)
        for name, ns, nd in (("copy_1r1w", 1, 1), ("fwd_like_2r1w", 2, 1), ("bwd_like_3r2w", 3, 2)):
            srcs, dsts = bufs[:ns], bufs[3:3 + nd]
            ms = time_probe(srcs, dsts)
            moved = (ns + nd) * nvec_elems * 2
            probe[name] = {"bytes": moved, "us": round(ms * 1e3, 2),
                           "GB/s": round(moved / (ms * 1e6), 1),
                           "frac_of_peak": round(moved / (ms * 1e6) / HBM_PEAK_GBS, 4)}
            log(f"probe {name}: {probe[name]['GB/s']} GB/s")
        del bufs

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
               "cores": threads, "kind": "oracle",
               "sample": (f"the full {w.name} batch (fwd then bwd, {fwd_bytes + bwd_bytes} algorithmic "
                          f"bytes) x {reps} reps, {spent:.1f} s total; {cpu_model()}"),
               "ms_per_step": round(cpu_step * 1e3, 1)}
        log(f"cpu baseline: {cpu['value']} GB/s")

    traffic = measured_traffic(w.name)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "rows": rows, "inter": inter, "limit": L,
                   "n_used": inp["n_used"], "permutation_map": inp["permutation_map"] is not None,
                   "zero_padding": inp["zero_padding"], "io_dtype": "bf16", "probs_dtype": "f32",
                   "seed": 0},
        "fwd": {"algorithmic_bytes": fwd_bytes, "us": round(f_avg * 1e3, 2),
                "us_min": round(min(fwd_ms) * 1e3, 2), "GB/s": round(f_gbs, 1),
                "frac_of_peak": round(f_gbs / HBM_PEAK_GBS, 4)},
        "bwd": {"algorithmic_bytes": bwd_bytes, "us": round(b_avg * 1e3, 2),
                "us_min": round(min(bwd_ms) * 1e3, 2), "GB/s": round(b_gbs, 1),
                "frac_of_peak": round(b_gbs / HBM_PEAK_GBS, 4)},
        "roofline": {"bound": "hbm", "kernel": "swiglu_probs_bwd_kernel",
                     "achieved": round(b_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(b_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
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
