"""Benchmark of the RAT+ hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--configs 1,2,4]
                    [--graph] [--no-cpu-baseline] [--no-decode-workload] [--calibration-copy MIB]

A step is one pass of the whole hot path over one batch of the headline
prefill workload (default: the largest prefill configuration, the head-wise
hybrid B=2, H=32, hd=128, T=8192 with heads 0-1 dense and heads 2-31 at D=4):
the recurrence scan with fused anchor compaction, the dilated attention over
the anchor cache, and one decode step that appends token T to every
sequence.  Inputs are synthetic (seeded), resident in HBM before the timed
region, and alternate between two copies so no step re-reads the previous
step's data from the 256 MB last-level cache.

Printed: ONE JSON line.  ``value`` is prefill tokens per second of the whole
step, B*T / (wall time of K steps / K), the K steps bracketed by device
synchronisations; the three launches of a step are enqueued one by one
(``--graph``: captured once into a HIP graph per input copy and replayed).
Per-kernel times come from each kernel launched K times back to back between
one pair of HIP events on its launch stream; ``kernels`` holds the headline
workload's, ``configs`` the scan and attention of every prefill workload
(1.5B-like, long prefill with window, head-wise hybrid), each with its
algorithmic bytes and FLOPs and a roofline entry against the roof that binds
it.  Every scan workspace's error word (a bounded wait that gave up) is read
after each pass; a set word turns the line into an error and the exit code
non-zero.  The decode-step time of the metric is measured on the decode
workload (batch 64, 32 heads, context 32768, D=64, W=128, 256 steps) and
reported beside it, as are the decode with top-k block selection, a chunked
prefill (the long-prefill workload in four chunks through the continuation
entry points, against the same sequence in one call), the prefill backward
and one whole RAT+ layer (on the 1.5B-like workload by default).
``roofline`` is for the kernel that takes the most time in the headline
step; ``cpu_baseline`` times the CPU oracle on a bounded sample of the same
work, on all host cores and on one.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
SPIN_CYCLES = 2_000_000         # device-side spin ahead of an event-timed region


def head_list(v):
    """Per-head values, run-length coded: [1]*2 + [4]*30 -> '1x2,4x30'; one value -> '16'."""
    v = [int(x) for x in v]
    runs = []
    for x in v:
        if runs and runs[-1][0] == x:
            runs[-1][1] += 1
        else:
            runs.append([x, 1])
    if len(runs) == 1:
        return str(runs[0][0])
    return ",".join(f"{x}x{n}" for x, n in runs)
MFMA_F32_PEAK_TFLOPS = 157.3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4,
                    help="prefill workload of the headline step (default: the largest, the "
                         "head-wise hybrid B=2 H=32 T=8192)")
    ap.add_argument("--configs", type=lambda v: [int(x) for x in v.split(",") if x],
                    default=[1, 2, 4],
                    help="prefill workloads whose scan and attention are also timed per kernel")
    ap.add_argument("--side-workload", type=int, default=1,
                    help="prefill workload of the backward and layer legs")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step as a captured HIP graph instead of three launches")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode-workload", action="store_true")
    ap.add_argument("--no-topk", action="store_true",
                    help="skip the decode workload with top-k block selection")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the layer measurement (projections around the prefill)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the prefill-backward measurement")
    ap.add_argument("--no-chunked", action="store_true",
                    help="skip the chunked-prefill measurement (long-prefill workload in chunks)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="before the steps, run three plain elementwise copies of MIB MiB "
                         "(reads MIB, writes MIB): the known-size reference that scales "
                         "hardware byte counters (FETCH_SIZE / WRITE_SIZE) to bytes")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method itself must move / compute)
# ---------------------------------------------------------------------------
def keyset_total(T, D, W):
    """sum over t < T of |S(t)| = 1 + min(W,t) + floor(max(0,t-W)/D)."""
    tot = 0
    for t in range(T):
        tot += 1 + min(W, t) + max(0, t - W) // D
    return tot


def scan_bytes(w, es=2):
    # read k, v, g; write hk, hv; write Kc, Vc rows (1/D of positions); ring
    per_head = 0
    for h in range(w.H):
        per_head += w.T * w.hd * es * 5 + (w.T // w.D[h]) * w.hd * es * 2
        per_head += min(w.W[h], w.T) * w.hd * es * 2
    return w.B * per_head + w.B * w.H * w.hd * 4 * 2  # + fp32 final state


def attn_bytes(w, es=2):
    # read q, hk, hv (each once), write o, read each anchor row once, lse
    tot = 0
    for h in range(w.H):
        tot += w.T * w.hd * es * 4 + (w.T // w.D[h]) * w.hd * es * 2 + w.T * 4
    return w.B * tot


def attn_flops(w):
    tot = 0
    cache = {}
    for h in range(w.H):
        key = (w.D[h], w.W[h])
        if key not in cache:
            cache[key] = keyset_total(w.T, *key)
        tot += 4 * w.hd * cache[key]
    return w.B * tot


def backward_bytes(w, es=2):
    # read q, k, v, g, dO, hk, hv, o and lse; write dq, dk, dv, dg
    return w.B * w.H * w.T * (12 * w.hd * es + 4)


def backward_flops(w):
    # per attended key: scores, dP and dq (query side), scores, dP, dV and dK
    # (key side): 7 products of 2*hd flops; the own position is VALU work
    tot = 0
    cache = {}
    for h in range(w.H):
        key = (w.D[h], w.W[h])
        if key not in cache:
            cache[key] = keyset_total(w.T, *key) - w.T  # own positions excluded
        tot += 14 * w.hd * cache[key]
    return w.B * tot


def decode_bytes(B, H, hd, D, W, pos, es=2):
    tot = 0
    for h in range(H):
        rows = max(0, pos - W[h]) // D[h] + min(W[h], pos)
        tot += rows * hd * es * 2              # K and V cache rows
        tot += 4 * hd * es + hd * es           # q, k, v, g in; o out
        tot += 4 * hd * 4                      # fp32 state in and out (k, v)
        tot += (2 * hd * es if W[h] > 0 else 0)  # ring slot
        tot += (2 * hd * es if pos % D[h] == D[h] - 1 else 0)  # anchor row
    return B * tot


def topk_decode_bytes(B, H, hd, D, W, pos, k, es=2, blk=64):
    """Decode-step bytes with top-k block selection: the plain step's, plus
    the eligible blocks' fp32 means, the selected blocks' rows that are not
    anchors (blk - blk/D per block for D dividing blk or a multiple of it),
    and the history row the step appends (plus a mean when pos ends a block)."""
    tot = decode_bytes(B, H, hd, D, W, pos, es) // B
    for h in range(H):
        ne = max(0, pos - W[h]) // blk
        ks = min(k, ne)
        tot += ne * hd * 4                                    # block means
        tot += ks * (blk - blk // D[h] if D[h] <= blk else blk - 1) * hd * es * 2
        tot += 2 * hd * es                                    # history row (k, v)
        tot += (hd * 4 if pos % blk == blk - 1 else 0)        # completed block mean
    return B * tot


# the source files of each profiled kernel (the kernel file, the
# kernel-specific header it includes, and the shared device header)
KERNEL_SOURCES = {
    "scan_kernel": ("scan.hip", "scan_tree.h", "rat_device.h"),
    "attn_prefill_kernel": ("attn_prefill.hip", "attn_tile.h", "rat_device.h"),
    "attn_resident_kernel": ("attn_resident.hip", "attn_tile.h", "rat_device.h"),
}


def kernel_source_hash(*names):
    """sha256[:16] of the named csrc files, concatenated in order."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "dilated_sparse_attention_rat_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel, launch_key):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current sources of the kernel (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        e = d.get(launch_key)
        if not e or e.get("source_sha") != kernel_source_hash(*KERNEL_SOURCES[kernel]):
            return None
        return float(e["bytes_per_launch"])
    except Exception:
        return None


# ---------------------------------------------------------------------------
class ScanError(RuntimeError):
    """A scan's bounded wait gave up (workspace word 2 set): invalid results."""


def roof_for(kind, nbytes, flops, us):
    """Roofline entry of one kernel: the binding roof is the one whose time
    at peak is longer (HBM bytes at 8 TB/s or useful FLOPs at the bf16 MFMA
    peak); the scan is priced on HBM only."""
    t = us * 1e-6
    gbs = nbytes / t / 1e9
    if kind == "scan" or flops is None:
        return dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=gbs / HBM_PEAK_GBS)
    tf = flops / t / 1e12
    if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        return dict(bound="mfma", achieved=tf, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=tf / MFMA_BF16_PEAK_TFLOPS)
    return dict(bound="hbm", achieved=gbs, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=gbs / HBM_PEAK_GBS)


class PrefillRig:
    """Two resident input copies of one prefill workload (so consecutive
    launches never re-read the previous launch's data from the 256 MB
    last-level cache), their outputs, caches and scan workspaces, and the
    launches of the path: scan, attention and one decode step at position T."""

    def __init__(self, rat, synth, torch, wid, decode=True):
        w = synth.WORKLOADS[wid]
        assert w.decode_steps == 0, "a prefill workload"
        self.rat, self.torch, self.w, self.wid = rat, torch, w, wid
        dev = "cuda"
        st = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.es = 2 if w.dtype == "bf16" else 4
        self.B, self.H, self.T, self.hd = w.B, w.H, w.T, w.hd
        self.D, self.W = list(w.D), list(w.W)
        self.T_cap = w.T + 1 if decode else w.T
        B, H, T, hd = self.B, self.H, self.T, self.hd
        x = synth.prefill_inputs(w)
        self.sets = []
        for copy in range(2):
            s = {n: torch.from_numpy(x[n]).to(dev).to(st) for n in "qkvg"}
            s["hk"] = torch.empty_like(s["k"])
            s["hv"] = torch.empty_like(s["v"])
            s["o"] = torch.empty_like(s["q"])
            s["lse"] = torch.empty((B, H, T), dtype=torch.float32, device=dev)
            s["cache"] = rat.alloc_cache(B, H, hd, self.T_cap, self.D, self.W, st, dev)
            s["ws"] = rat.scan_workspace(B, H, T, hd, dev)
            if decode:
                dx = synth.draw((B, H, 1, hd), w.seed + 77, w.qkv_std, w.g_bias, w.dtype)
                s["dec"] = {n: torch.from_numpy(dx[n][:, :, 0]).to(dev).to(st) for n in "qkvg"}
                s["do"] = torch.empty_like(s["dec"]["q"])
                s["dws"] = rat.decode_workspace(B, H, hd, self.T_cap, self.D, self.W, dev)
            self.sets.append(s)
        del x
        self.stream = torch.cuda.current_stream()

    def scan(self, s):
        c = s["cache"]
        self.rat.rat_scan_prefill(s["k"], s["v"], s["g"], self.D, self.W, self.T_cap, c["Kc"],
                                  c["Vc"], c["state_k"], c["state_v"], s["ws"], hk=s["hk"],
                                  hv=s["hv"], k_ring=c["k_ring"], v_ring=c["v_ring"])

    def attn(self, s):
        c = s["cache"]
        self.rat.rat_dilated_attn_prefill(s["q"], s["hk"], s["hv"], c["Kc"], c["Vc"], self.D,
                                          self.W, self.T_cap, s["o"], s["lse"])

    def dec(self, s):
        c, d = s["cache"], s["dec"]
        self.rat.rat_decode_step(d["q"], d["k"], d["v"], d["g"], c["state_k"], c["state_v"],
                                 c["Kc"], c["Vc"], c["k_ring"], c["v_ring"], s["do"], self.D,
                                 self.W, self.T, self.T_cap, workspace=s["dws"])

    def step(self, s, ev=None):
        fns = (self.scan, self.attn, self.dec)
        if ev is not None:
            ev[0].record(self.stream)
        for i, fn in enumerate(fns):
            fn(s)
            if ev is not None:
                ev[i + 1].record(self.stream)

    def check(self, what):
        """Raise ScanError if a scan wait of any launch so far timed out (the
        error word is sticky: it stays set until the workspace is zeroed)."""
        self.torch.cuda.synchronize()
        for s in self.sets:
            if int(s["ws"][2].item()) != 0:
                raise ScanError(f"{self.w.name}: a scan wait timed out during {what}")

    def kernel_ms(self, fn, spin, K, reps=3):
        """Mean time per launch of fn, K launches back to back between one
        pair of HIP events on the launch stream; fastest of reps passes (a
        one-time host stall while queueing, once seen at about 40 ms, would
        otherwise land inside a single pass)."""
        torch = self.torch
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            # keep the GPU busy while the host queues the K launches: one
            # untimed launch of the same kernel when a launch outlasts the
            # host's enqueue time, a device spin for the short decode step
            if spin:
                torch.cuda._sleep(max(SPIN_CYCLES, K * 150_000))
            else:
                fn(self.sets[1])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            for i in range(K):
                fn(self.sets[i % 2])
            e1.record(self.stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / K
            best = ms if best is None else min(best, ms)
        return best

    def kernels(self, K, with_decode=True):
        """Per-kernel times, algorithmic bytes and FLOPs, and roofline entries."""
        w, es = self.w, self.es
        scan_us = self.kernel_ms(self.scan, False, K) * 1e3
        attn_us = self.kernel_ms(self.attn, False, K) * 1e3
        self.check("the per-kernel passes")
        sb, ab, af = scan_bytes(w, es), attn_bytes(w, es), attn_flops(w)
        ks = {
            "scan": dict(us=scan_us, bytes=sb, gbs=sb / scan_us / 1e3, kernel="scan_kernel",
                         roofline=roof_for("scan", sb, None, scan_us)),
            "attention": dict(us=attn_us, bytes=ab, flops=af, gbs=ab / attn_us / 1e3,
                              tflops=af / attn_us / 1e6, kernel=attn_kernel_name(w),
                              roofline=roof_for("attention", ab, af, attn_us)),
        }
        ks["scan"]["roofline"]["traffic"] = traffic_from_profiles("scan_kernel",
                                                                  f"scan_w{self.wid}")
        ks["attention"]["roofline"]["traffic"] = traffic_from_profiles(
            attn_kernel_name(w), f"attn_w{self.wid}")
        ks["attention"]["mfma_frac_useful"] = af / attn_us / 1e6 / MFMA_BF16_PEAK_TFLOPS
        ks["attention"]["hbm_frac"] = ab / attn_us / 1e3 / HBM_PEAK_GBS
        if with_decode:
            dec_us = self.kernel_ms(self.dec, True, K) * 1e3
            db = decode_bytes(self.B, self.H, self.hd, self.D, self.W, self.T, es)
            ks["decode_step"] = dict(us=dec_us, bytes=db, gbs=db / dec_us / 1e3)
        return ks

    def describe(self):
        w = self.w
        return (f"{w.name}: B={w.B} H={w.H} hd={w.hd} T={w.T} D={head_list(w.D)} "
                f"W={head_list(w.W)}")


def bench_prefill_config(rat, synth, torch, wid, K):
    """Scan and attention of one prefill workload, each timed K launches back
    to back; tokens per second of the two kernels."""
    rig = PrefillRig(rat, synth, torch, wid, decode=False)
    for i in range(2):
        rig.scan(rig.sets[i])
        rig.attn(rig.sets[i])
    rig.check("the warm-up")
    ks = rig.kernels(K, with_decode=False)
    tok = rig.B * rig.T
    res = dict(workload=rig.describe(), tok_s_kernels=tok / ((ks["scan"]["us"] + ks["attention"]["us"]) * 1e-6),
               **ks)
    del rig
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the RAT+ hot path "
              "shards over (batch, head) with no exchange, and multi-GPU runs are not "
              "implemented", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dilated_sparse_attention_rat_amd as rat
    from dilated_sparse_attention_rat_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    # the first device spin of a process is not a reliable spin (its kernel
    # is loaded then); issue one here so the spins ahead of timed regions are
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    rat.lib()  # fail loudly if the HIP library is missing

    try:
        line = run(args, rat, synth, torch, np)
    except ScanError as e:
        print(json.dumps({"metric": METRIC, "value": None, "unit": "tok/s", "n_gpus": 1,
                          "error": str(e)}))
        sys.exit(3)
    print(json.dumps(line))


METRIC = "prefill tok/s + decode step µs per RAT+ layer; % of HBM / MFMA bf16 peak"


def run(args, rat, synth, torch, np):
    w = synth.WORKLOADS[args.workload]
    rig = PrefillRig(rat, synth, torch, args.workload)
    B, T = rig.B, rig.T
    sets, stream = rig.sets, rig.stream

    if args.calibration_copy > 0:
        n = args.calibration_copy * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    for i in range(args.warmup):
        rig.step(sets[i % 2])
    rig.check("the warm-up")

    # one graph per input copy: the step's three launches, replayed as a unit
    graphs = None
    if args.graph:
        graphs = []
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                rig.step(s)
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % 2].replay()
        torch.cuda.synchronize()

    # ---- timed passes: K steps each, no instrumentation -------------------
    # Two passes of exactly K steps, each bracketed by device synchronisation;
    # both are reported and the faster one is the headline (a host stall on
    # a shared machine can hold up one pass: one run measured 2.1 ms per step
    # in a pass whose kernels all ran at their usual speed).
    K = args.steps
    walls = []
    # Python's cyclic collector off while steps are queued: a full collection
    # over the interpreter's heap (torch and numpy loaded) stalls the host
    # that launches the steps for tens of ms (a per-step probe saw single
    # launches of 1 and 31 ms among ~0.1 ms ones), which empties the GPU's
    # queue inside a timed pass
    gc.collect()
    gc.disable()
    for _ in range(2):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            if graphs is not None:
                graphs[i % 2].replay()
            else:
                rig.step(sets[i % 2])
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        rig.check("the timed steps")
    wall = min(walls)

    # ---- instrumented pass: K eager steps with HIP events between kernels --
    # (the median over the K steps: one host stall while queueing would
    # otherwise land in the mean of the step it delays)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        rig.step(sets[i % 2], evs[i])
    torch.cuda.synchronize()
    wall_instr = time.perf_counter() - t1
    gc.enable()
    rig.check("the instrumented steps")
    del graphs
    in_step = [float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3 for j in range(3)]

    # ---- per-kernel pass: each kernel K times back to back ----------------
    kernels = rig.kernels(K)
    for name, us in zip(("scan", "attention", "decode_step"), in_step):
        kernels[name]["us_in_step"] = us
    ms_per_step = wall * 1e3 / K
    tok = B * T
    value = tok / (ms_per_step / 1e3)
    t_scan, t_attn = kernels["scan"]["us"], kernels["attention"]["us"]

    # roofline of the kernel that takes the most time in the step
    dom = max(("scan", "attention"), key=lambda k: kernels[k]["us"])
    roof = dict(kernels[dom]["roofline"])
    roof["kernel"] = kernels[dom]["kernel"]
    roof = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "kernel")}
    headline = dict(workload=rig.describe(), tok_s_kernels=tok / ((t_scan + t_attn) * 1e-6),
                    **{k: kernels[k] for k in ("scan", "attention")})
    del rig, sets
    torch.cuda.empty_cache()

    # ---- the other prefill workloads: scan and attention per config --------
    configs = {str(args.workload): headline}
    for wid in args.configs:
        if wid != args.workload:
            configs[str(wid)] = bench_prefill_config(rat, synth, torch, wid, K)

    # ---- decode workload: µs per decode step ------------------------------
    decode_info = None
    if not args.no_decode_workload:
        decode_info = bench_decode_workload(rat, synth, torch, np)
    topk_info = None
    if not args.no_topk:
        topk_info = bench_topk_decode(rat, synth, torch, np)
    chunked_info = None
    if not args.no_chunked:
        chunked_info = bench_chunked(rat, synth, torch, np)
    side = synth.WORKLOADS[args.side_workload]
    backward_info = None
    if not args.no_backward:
        backward_info = bench_backward(rat, synth, torch, np, side)
    layer_info = None
    if not args.no_layer:
        layer_info = bench_layer(rat, synth, torch, np, side)
    torch.cuda.empty_cache()

    # ---- CPU oracle baseline (bounded sample of the same step) -----------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_seconds)

    return {
        "metric": METRIC,
        "value": value,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_passes": [w_ * 1e3 / K for w_ in walls],
        "ms_per_step_instrumented": wall_instr * 1e3 / K,
        "kernel_timing": "kernels.*.us: each kernel K times back to back between one pair of HIP "
                         "events on the launch stream (fastest of 3 such passes); us_in_step: HIP "
                         "events around each launch inside the step, median over the K steps "
                         "(each event pair adds a few us)",
        "launch": "hip graph per step" if args.graph else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{rig_name(w)} (scan + dilated attention prefill + 1 decode step per step)",
            "global_batch": w.B,
            "seq_len": w.T,
            "parallelism": "single GPU",
            "decode_workload": "decode: batch 64, H=32, hd=128, context 32768, D=64, W=128, "
                               "256 steps",
        },
        "prefill_tok_s_kernels_only": tok / ((t_scan + t_attn) * 1e-6),
        "decode_us_per_step": decode_info["us_mean"] if decode_info else None,
        "kernels": kernels,
        "configs": configs,
        "decode_workload": decode_info,
        "topk_decode_workload": topk_info,
        "chunked_prefill": chunked_info,
        "backward": backward_info,
        "layer": layer_info,
        "roofline": roof,
        "cpu_baseline": cpu,
    }


def rig_name(w):
    return (f"{w.name}: B={w.B} H={w.H} hd={w.hd} T={w.T} D={head_list(w.D)} "
            f"W={head_list(w.W)}")


def attn_kernel_name(w) -> str:
    """The attention kernel the library picks for this workload: the
    resident-anchor kernel for bf16 windowless heads whose anchors fit in LDS
    (at most 256 per head), else the streaming kernel."""
    resident = (w.dtype == "bf16" and w.T * w.hd * 2 <= 2 ** 31 - 1
                and all(wh == 0 and (w.T - 1) // d <= 256 for d, wh in zip(w.D, w.W)))
    return "attn_resident_kernel" if resident else "attn_prefill_kernel"


def bench_decode_workload(rat, synth, torch, np):
    w = synth.WORKLOADS[3]
    B, H, T, hd, steps = w.B, w.H, w.T, w.hd, w.decode_steps
    T_cap = w.T_cap
    D, W = list(w.D), list(w.W)
    cache = rat.alloc_cache(B, H, hd, T_cap, D, W, torch.bfloat16, "cuda")
    ws = rat.scan_workspace(1, H, T, hd, "cuda")
    for b in range(B):  # context: cache-only prefill one batch row at a time
        kvg = synth.decode_context_row(w, b)
        rat.rat_scan_prefill(kvg["k"], kvg["v"], kvg["g"], D, W, T_cap, cache["Kc"][b:b + 1],
                             cache["Vc"][b:b + 1], cache["state_k"][b:b + 1],
                             cache["state_v"][b:b + 1], ws, k_ring=cache["k_ring"][b:b + 1],
                             v_ring=cache["v_ring"][b:b + 1])
        del kvg
    torch.cuda.synchronize()
    if int(ws[2].item()) != 0:
        raise ScanError("decode workload: a wait of a context scan timed out")
    inputs = [synth.decode_step_inputs(w, s) for s in range(steps)]
    outs = torch.empty((B, H, hd), dtype=torch.bfloat16, device="cuda")
    dws = rat.decode_workspace(B, H, hd, T_cap, D, W, "cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda._sleep(SPIN_CYCLES)  # the first step queued before its event
    evs[0].record(stream)
    for s in range(steps):
        x = inputs[s]
        rat.rat_decode_step(x["q"], x["k"], x["v"], x["g"], cache["state_k"], cache["state_v"],
                            cache["Kc"], cache["Vc"], cache["k_ring"], cache["v_ring"], outs, D,
                            W, T + s, T_cap, workspace=dws)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([evs[s].elapsed_time(evs[s + 1]) * 1e3 for s in range(steps)])
    nbytes = np.array([decode_bytes(B, H, hd, D, W, T + s) for s in range(steps)], dtype=np.float64)
    gbs = nbytes / (us * 1e-6) / 1e9
    res = dict(us_mean=float(us.mean()), us_max=float(us.max()), us_min=float(us.min()),
               bytes_mean=float(nbytes.mean()), gbs_mean=float(gbs.mean()),
               hbm_frac=float(gbs.mean() / HBM_PEAK_GBS), steps=steps)
    del cache, inputs
    torch.cuda.empty_cache()
    return res


def bench_topk_decode(rat, synth, torch, np, k_sel=8):
    """The decode workload with top-k block selection (k_sel blocks of 64
    positions per query) on top of the dilated key set: the full per-head
    state history [B,H,T_cap,hd] and its fp32 block means are built from the
    same context, then every step is timed with HIP events."""
    w = synth.WORKLOADS[3]
    B, H, T, hd, steps = w.B, w.H, w.T, w.hd, w.decode_steps
    T_cap = w.T_cap
    D, W = list(w.D), list(w.W)
    st = torch.bfloat16
    cache = rat.alloc_cache(B, H, hd, T_cap, D, W, st, "cuda")
    hist = rat.alloc_topk_history(B, H, hd, T_cap, st, "cuda")
    ws = rat.scan_workspace(1, H, T, hd, "cuda")
    hk = torch.empty((1, H, T, hd), dtype=st, device="cuda")
    hv = torch.empty_like(hk)
    for b in range(B):  # context one batch row at a time, then its history
        kvg = synth.decode_context_row(w, b)
        rat.rat_scan_prefill(kvg["k"], kvg["v"], kvg["g"], D, W, T_cap, cache["Kc"][b:b + 1],
                             cache["Vc"][b:b + 1], cache["state_k"][b:b + 1],
                             cache["state_v"][b:b + 1], ws, hk=hk, hv=hv,
                             k_ring=cache["k_ring"][b:b + 1], v_ring=cache["v_ring"][b:b + 1])
        rat.rat_topk_cache_build(hk, hv, hist["hk_hist"][b:b + 1], hist["hv_hist"][b:b + 1],
                                 hist["block_means"][b:b + 1])
        del kvg
    del hk, hv
    torch.cuda.synchronize()
    if int(ws[2].item()) != 0:
        raise ScanError("top-k decode workload: a wait of a context scan timed out")
    inputs = [synth.decode_step_inputs(w, s) for s in range(steps)]
    outs = torch.empty((B, H, hd), dtype=st, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda._sleep(SPIN_CYCLES)  # the first step queued before its event
    evs[0].record(stream)
    for s in range(steps):
        x = inputs[s]
        rat.rat_decode_step_topk(x["q"], x["k"], x["v"], x["g"], cache["state_k"],
                                 cache["state_v"], cache["Kc"], cache["Vc"], cache["k_ring"],
                                 cache["v_ring"], hist["hk_hist"], hist["hv_hist"],
                                 hist["block_means"], outs, D, W, T + s, T_cap, k_sel)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    us = np.array([evs[s].elapsed_time(evs[s + 1]) * 1e3 for s in range(steps)])
    nbytes = np.array([topk_decode_bytes(B, H, hd, D, W, T + s, k_sel) for s in range(steps)],
                      dtype=np.float64)
    gbs = nbytes / (us * 1e-6) / 1e9
    res = dict(k_blocks=k_sel, block=64, us_mean=float(us.mean()), us_max=float(us.max()),
               us_min=float(us.min()), bytes_mean=float(nbytes.mean()),
               gbs_mean=float(gbs.mean()), hbm_frac=float(gbs.mean() / HBM_PEAK_GBS),
               steps=steps)
    del cache, hist, inputs
    torch.cuda.empty_cache()
    return res


def bench_chunked(rat, synth, torch, np, reps=5, nchunks=4):
    """Chunked prefill of the long-prefill workload (T=16384, D=64, W=256):
    the sequence in nchunks equal chunks through the continuation entry
    points (two rings used alternately), against the same sequence in one
    call.  Times are HIP-event medians over reps repetitions."""
    w = synth.WORKLOADS[2]
    B, H, T, hd = w.B, w.H, w.T, w.hd
    D, W = list(w.D), list(w.W)
    x = synth.prefill_inputs(w)
    t = {n: torch.from_numpy(x[n]).to("cuda").to(torch.bfloat16) for n in "qkvg"}
    del x
    Tc = T // nchunks
    ch = [{n: t[n][:, :, i * Tc:(i + 1) * Tc].contiguous() for n in "qkvg"} for i in range(nchunks)]
    c = rat.alloc_cache(B, H, hd, T, D, W, torch.bfloat16, "cuda")
    rings = [(c["k_ring"], c["v_ring"]), (torch.empty_like(c["k_ring"]), torch.empty_like(c["v_ring"]))]
    states = [(c["state_k"], c["state_v"]), (torch.zeros_like(c["state_k"]), torch.zeros_like(c["state_v"]))]
    hk, hv = torch.empty_like(ch[0]["k"]), torch.empty_like(ch[0]["v"])
    o = torch.empty_like(ch[0]["q"])
    ws = rat.scan_workspace(B, H, Tc, hd, "cuda")
    hk_f, hv_f, o_f = torch.empty_like(t["k"]), torch.empty_like(t["v"]), torch.empty_like(t["q"])
    ws_f = rat.scan_workspace(B, H, T, hd, "cuda")
    stream = torch.cuda.current_stream()

    def chunked(ev=None):
        for i in range(nchunks):
            cur, prev = rings[i % 2], rings[1 - i % 2]
            sc, sp = states[i % 2], states[1 - i % 2]
            if ev is not None:
                ev[2 * i].record(stream)
            if i == 0:
                rat.rat_scan_prefill(ch[0]["k"], ch[0]["v"], ch[0]["g"], D, W, T, c["Kc"], c["Vc"],
                                     sc[0], sc[1], ws, hk=hk, hv=hv, k_ring=cur[0], v_ring=cur[1])
                rat.rat_dilated_attn_prefill(ch[0]["q"], hk, hv, c["Kc"], c["Vc"], D, W, T, o)
            else:
                rat.rat_scan_prefill_continue(ch[i]["k"], ch[i]["v"], ch[i]["g"], D, W, T, i * Tc,
                                              sp[0], sp[1], c["Kc"], c["Vc"], sc[0], sc[1], ws,
                                              hk=hk, hv=hv, k_ring_in=prev[0], v_ring_in=prev[1],
                                              k_ring=cur[0], v_ring=cur[1])
                rat.rat_dilated_attn_prefill_continue(ch[i]["q"], hk, hv, c["Kc"], c["Vc"], D, W, T,
                                                      i * Tc, o, k_ring_prev=prev[0],
                                                      v_ring_prev=prev[1])
            if ev is not None:
                ev[2 * i + 1].record(stream)

    def whole():
        rat.rat_scan_prefill(t["k"], t["v"], t["g"], D, W, T, c["Kc"], c["Vc"], c["state_k"],
                             c["state_v"], ws_f, hk=hk_f, hv=hv_f, k_ring=c["k_ring"],
                             v_ring=c["v_ring"])
        rat.rat_dilated_attn_prefill(t["q"], hk_f, hv_f, c["Kc"], c["Vc"], D, W, T, o_f)

    chunked()
    whole()
    torch.cuda.synchronize()
    per_chunk = []
    tot_chunked, tot_whole = [], []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nchunks)]
        # a short device-side spin first, so that every launch of the region
        # is queued before its first event (an idle GPU would otherwise time
        # the host's launch latency into the first chunk)
        torch.cuda._sleep(SPIN_CYCLES)
        chunked(ev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        whole()
        e1.record(stream)
        torch.cuda.synchronize()
        us = [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(nchunks)]
        per_chunk.append(us)
        tot_chunked.append(sum(us))
        tot_whole.append(e0.elapsed_time(e1) * 1e3)
    med = lambda a: float(np.median(a))
    res = dict(workload=f"{w.name}: B={B} H={H} hd={hd} T={T} D={head_list(D)} W={head_list(W)} in {nchunks} "
                        f"chunks of {Tc}",
               us_per_chunk=[med([r[i] for r in per_chunk]) for i in range(nchunks)],
               us_chunked=med(tot_chunked), us_whole=med(tot_whole),
               tok_s_chunked=B * T / (med(tot_chunked) * 1e-6),
               tok_s_whole=B * T / (med(tot_whole) * 1e-6))
    if int(ws[2].item()) != 0 or int(ws_f[2].item()) != 0:
        raise ScanError("chunked prefill: a scan wait timed out")
    del t, ch, c, rings, states, hk, hv, o, hk_f, hv_f, o_f
    torch.cuda.empty_cache()
    return res


def bench_backward(rat, synth, torch, np, w, reps=10):
    """Prefill backward (dq, dk, dv, dg for a random dO) of workload w after
    its forward; HIP-event time of the whole rat_prefill_backward call."""
    x = synth.prefill_inputs(w)
    st = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(x[n]).to("cuda").to(st) for n in "qkvg"}
    del x
    B, H, T, hd = w.B, w.H, w.T, w.hd
    D, W = list(w.D), list(w.W)
    c = rat.alloc_cache(B, H, hd, T, D, W, st, "cuda")
    hk, hv = torch.empty_like(t["k"]), torch.empty_like(t["v"])
    ws = rat.scan_workspace(B, H, T, hd, "cuda")
    rat.rat_scan_prefill(t["k"], t["v"], t["g"], D, W, T, c["Kc"], c["Vc"], c["state_k"],
                         c["state_v"], ws, hk=hk, hv=hv, k_ring=c["k_ring"], v_ring=c["v_ring"])
    o = torch.empty_like(t["q"])
    lse = torch.empty((B, H, T), dtype=torch.float32, device="cuda")
    rat.rat_dilated_attn_prefill(t["q"], hk, hv, c["Kc"], c["Vc"], D, W, T, o, lse)
    torch.cuda.synchronize()
    if int(ws[2].item()) != 0:
        raise ScanError("backward: a wait of the forward scan timed out")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 99)
    dO = torch.randn(t["q"].shape, generator=gen, device="cuda").to(st)
    grads = [torch.empty_like(t["q"]) for _ in range(4)]
    bws = rat.backward_workspace(B, H, T, hd, D, W, "cuda")
    stream = torch.cuda.current_stream()

    def run():
        rat.rat_prefill_backward(t["q"], t["k"], t["v"], t["g"], hk, hv, o, lse, dO, D, W,
                                 *grads, bws)

    run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    if int(bws[2].item()) != 0:
        raise ScanError("backward: a wait of the reverse scan timed out")
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    es = 2 if w.dtype == "bf16" else 4
    nb, nf = backward_bytes(w, es), backward_flops(w)
    med = us[reps // 2]
    res = dict(workload=f"{w.name}: B={B} H={H} hd={hd} T={T} D={head_list(D)} W={head_list(W)}",
               us_median=med, us_min=us[0], bytes=nb, flops=nf, gbs=nb / (med * 1e-6) / 1e9,
               hbm_frac=nb / (med * 1e-6) / 1e9 / HBM_PEAK_GBS,
               tflops=nf / (med * 1e-6) / 1e12,
               mfma_frac_useful=nf / (med * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
               tok_s=B * T / (med * 1e-6))
    del t, c, hk, hv, o, lse, dO, grads, bws
    torch.cuda.empty_cache()
    return res


def bench_layer(rat, synth, torch, np, w, reps=5):
    """One RAT+ layer over the step's prefill workload: d_model = H*hd, random
    projection weights, x ~ N(0, 1).  HIP-event time of rat_layer_prefill."""
    B, H, T, hd = w.B, w.H, w.T, w.hd
    D, W = list(w.D), list(w.W)
    dm = H * hd
    st = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed + 7)

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device="cuda") * std).to(st)

    x = rnd((B, T, dm), 1.0)
    wq, wk, wv = (rnd((dm, dm), w.qkv_std / math.sqrt(dm)) for _ in range(3))
    wg = rnd((dm, dm), 1.0 / math.sqrt(dm))
    wo = rnd((dm, dm), 1.0 / math.sqrt(dm))
    bg = torch.full((dm,), float(w.g_bias), dtype=torch.float32, device="cuda")
    out = torch.empty_like(x)
    cache = rat.alloc_cache(B, H, hd, T, D, W, st, "cuda")
    ws = rat.layer_workspace(rat.binding._dtype_code(x), B, H, T, hd, "cuda")
    stream = torch.cuda.current_stream()

    def run():
        rat.rat_layer_prefill(x, wq, wk, wv, wg, bg, wo, out, D, W, H, hd, T, cache, ws)

    run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    if int(ws[2].item()) != 0:  # the scan workspace heads the layer workspace
        raise ScanError("layer: a scan wait timed out")
    us = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    med = us[reps // 2]
    gemm_flops = 5 * 2 * B * T * dm * dm
    res = dict(workload=f"{w.name} layer: B={B} T={T} d_model={dm} H={H} hd={hd} D={head_list(D)} W={head_list(W)}",
               us_median=med, us_min=us[0], tok_s=B * T / (med * 1e-6),
               gemm_flops=gemm_flops, attn_flops=attn_flops(w),
               tflops_total=(gemm_flops + attn_flops(w)) / (med * 1e-6) / 1e12)
    del x, wq, wk, wv, wg, wo, bg, out, cache, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, target_s):
    """Time the CPU oracle (as it stands) on whole (batch row, head)
    sequences of the headline prefill workload: the scan and the dilated
    attention of one head per thread, repeated over further heads until
    about target_s seconds or the whole workload; then one head on a single
    core.  Each time is scaled to tokens of the full workload by the
    fraction of its attention FLOPs the sample did (heads differ in cost in
    a hybrid)."""
    import numpy as np
    import oracle
    from dilated_sparse_attention_rat_amd import synth
    x = synth.prefill_inputs(w)
    total = attn_flops(w)
    flops_bh = {h: 4 * w.hd * keyset_total(w.T, w.D[h], w.W[h]) for h in range(w.H)}
    # heads in descending cost, so each group of threads runs heads of equal cost
    order = [(b, h) for b in range(w.B) for h in sorted(range(w.H), key=lambda h: -flops_bh[h])]

    def run(pairs):
        for b in sorted({b for b, _ in pairs}):
            hs = [h for bb, h in pairs if bb == b]
            f = {n: x[n][b:b + 1, hs].astype(np.float64) for n in "qkvg"}
            oracle.prefill(f["q"], f["k"], f["v"], f["g"], [w.D[h] for h in hs],
                           [w.W[h] for h in hs], w.scale, w.dtype == "bf16")

    nthr = max(1, oracle.num_threads())
    done, spent, i = [], 0.0, 0
    while i < len(order) and spent < target_s:
        grp = order[i:i + nthr]
        t0 = time.perf_counter()
        run(grp)
        spent += time.perf_counter() - t0
        done += grp
        i += nthr
    frac = sum(flops_bh[h] for _, h in done) / total
    value = w.B * w.T * frac / spent
    # one core, one head of the lightest kind
    one = [min(order, key=lambda bh: flops_bh[bh[1]])]
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        run(one)
        s1 = time.perf_counter() - t0
    finally:
        oracle.set_threads(nthr)
    frac1 = flops_bh[one[0][1]] / total
    heads = sorted({h for _, h in done})
    return dict(value=value, unit="tok/s", cores=nthr, kind="oracle",
                sample=f"oracle prefill (scan + attention, fp64, OpenMP over heads) of "
                       f"{len(done)} of {w.B * w.H} (batch row, head) sequences at T={w.T} "
                       f"(heads {head_list(heads) if len(heads) < 4 else f'{heads[0]}..{heads[-1]}'}), "
                       f"{spent:.1f} s; tokens scaled by the fraction of the workload's attention "
                       "FLOPs done",
                seconds=spent, cpu_model=cpu_model(), nproc=os.cpu_count(),
                single_core=dict(value=w.B * w.T * frac1 / s1, unit="tok/s", cores=1,
                                 seconds=s1,
                                 sample=f"one (batch row, head) sequence (head {one[0][1]}, "
                                        f"D={w.D[one[0][1]]}) on one thread, scaled the same "
                                        "way"),
                topk_decode=cpu_topk_decode())


def cpu_model():
    """The host CPU's model name (first entry of /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_topk_decode(steps=4, k_sel=8):
    """The top-k block decode oracle (numpy fp64, one thread) on one
    (batch row, head) of the decode workload's shape, scaled to a whole step
    of the batch."""
    import numpy as np
    import oracle
    from dilated_sparse_attention_rat_amd import synth
    w = synth.WORKLOADS[3]
    T, hd = w.T, w.hd
    x = synth.random_case(w.seed, 1, 1, T + steps, hd, w.dtype, w.qkv_std, w.g_bias)
    f = {n: x[n].astype(np.float64) for n in "qkvg"}
    hk_u, _ = oracle.scan(f["g"], f["k"])
    hv_u, _ = oracle.scan(f["g"], f["v"])
    hk, hv = oracle.round_bf16(hk_u), oracle.round_bf16(hv_u)
    D, W = np.array(w.D[:1]), np.array(w.W[:1])
    t0 = time.perf_counter()
    for s in range(steps):
        pos = T + s
        oracle.decode_step_topk(f["q"][:, :, pos], f["k"][:, :, pos], f["v"][:, :, pos],
                                f["g"][:, :, pos], hk_u[:, :, pos - 1], hv_u[:, :, pos - 1],
                                hk[:, :, :pos], hv[:, :, :pos], D, W, w.scale, pos, k_sel, True)
    per_bh = (time.perf_counter() - t0) / steps
    return dict(us_per_step=per_bh * w.B * w.H * 1e6, unit="us per decode step", cores=1,
                kind="oracle",
                sample=f"oracle top-k decode (k={k_sel}, numpy fp64) of one (batch row, head) at "
                       f"context {T}, {steps} steps, scaled by the batch's {w.B * w.H} "
                       "(batch row, head) pairs")


if __name__ == "__main__":
    main()
