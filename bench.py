"""Benchmark of the BigBird block-sparse attention forward on one MI355X.

One step = one ``bbsa_forward`` call (all kernels: the gathered-block
attention kernel and the split-K merge of the two global query blocks) over
one batch of the BigBird-base-shaped workload: B=4, H=12, L=4096, d=64,
block=64, r=3, bf16, padded sequences, plan precomputed on the host (a layer
builds its plan once).  Inputs are resident in HBM before timing starts; the
steps rotate over several copies of the inputs (more bytes than the 256 MB
last-level cache) so that no step reads its inputs from cache left by the
previous one.  The JSON line also carries the 10th/50th/90th percentile of
single steps each bracketed by its own events, and the warm-cache step time
(the same input set every step) for comparison.

The other workloads at L >= 4096 (Pegasus-large encoder shape, the 16384-token
and the 32768-token block-128 cases) are timed in the same run with the same
protocol and reported under ``config.other_workloads``.  Before each
workload's warm-up steps a fixed wall time of untimed steps lets the GPU's
clocks ramp up (``--preroll``; its length and step count are in the line).
The roofline fractions are computed from the step time.

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd TFLOP/s (useful) + % MFMA/HBM roofline, L=4096 H=12"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (no sparsity)
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 MFMA
# The kernel and the host code that decides its work decomposition.
KERNEL_SOURCES = ["block_sparse_long_bbsa_amd/csrc/bbsa_forward.hip", "block_sparse_long_bbsa_amd/csrc/bbsa_schedule.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bbsa_attn_bf16_B4_H12_L4096.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def useful_pairs(nb: int, r: int) -> int:
    """Block pairs of one (batch, head) inside the pattern: 2 full rows, rows 1
    and nb-2 with 4 + r blocks, the other nb - 4 middle rows with 5 + r."""
    return 2 * nb + 2 * (4 + r) + (nb - 4) * (5 + r)


def useful_flops(B, H, nb, block, d, r) -> float:
    return 4.0 * block * block * d * useful_pairs(nb, r) * B * H


def algorithmic_bytes(B, H, L, d, nb, r, elt) -> float:
    """Q, K, V read once, O written once, the mask and the plan read once."""
    return 4.0 * B * H * L * d * elt + B * L * 4 + H * (nb - 2) * r * 4


def kernel_source_hash() -> str:
    """Hash of the kernel source with comments, blank lines and indentation
    dropped, so that a counter summary stays valid across comment-only and
    formatting-only edits."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(workload_name: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on this workload and on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash() or t.get("workload") != workload_name:
        return None
    return t.get("hbm_bytes_per_launch")


def host_info():
    """Host cores this process may run on, the CPU model and the BLAS threads."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas = 1
    return cores, model, blas


def cpu_baseline(inp, plan, w, budget_s: float):
    """Time the oracle on a bounded sample: whole (batch, head) slices of the
    same workload, as many as fit in about ``budget_s`` seconds.  The BLAS
    pool is capped at the number of host cores this process may use, so
    ``cores`` is both the host core count and the most threads the oracle
    used."""
    import oracle
    from threadpoolctl import threadpool_limits
    cores, model, blas = host_info()
    flops_per_slice = useful_flops(1, 1, w.nb, w.block, w.d, w.r)
    done, t0 = 0, time.perf_counter()
    with threadpool_limits(cores):
        for b in range(w.B):
            for h in range(w.H):
                oracle.forward(inp["q"][b:b + 1, h:h + 1], inp["k"][b:b + 1, h:h + 1],
                               inp["v"][b:b + 1, h:h + 1], inp["mask"][b:b + 1], plan[h:h + 1], w.block)
                done += 1
                if time.perf_counter() - t0 > budget_s:
                    break
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return {"value": flops_per_slice * done / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": model, "blas_threads": int(min(blas, cores)),
            "sample": f"{done} of {w.B * w.H} (batch, head) slices of {w.name}, float64 dense "
                      f"masked attention, {dt:.1f} s wall"}


def roofline(w, step_ms):
    """Fractions of the MI355X roofs for one step of workload ``w`` taking
    ``step_ms``: useful flops against the dtype's dense MFMA peak, algorithmic
    bytes against HBM; the binding roof is the one with the longer time."""
    elt = 2 if w.dtype == "bf16" else 4
    flops = useful_flops(w.B, w.H, w.nb, w.block, w.d, w.r)
    nbytes = algorithmic_bytes(w.B, w.H, w.L, w.d, w.nb, w.r, elt)
    peak_mfma = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    t_mfma = flops / (peak_mfma * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    sec = step_ms * 1e-3
    mfma_frac = flops / sec / 1e12 / peak_mfma
    hbm_frac = nbytes / sec / 1e9 / PEAK_HBM_GBS
    if t_hbm >= t_mfma:
        rec = {"bound": "hbm", "achieved": round(nbytes / sec / 1e9, 2), "peak": PEAK_HBM_GBS,
               "unit": "GB/s", "frac": round(hbm_frac, 4)}
    else:
        rec = {"bound": "mfma", "achieved": round(flops / sec / 1e12, 2), "peak": peak_mfma,
               "unit": "TFLOP/s", "frac": round(mfma_frac, 4)}
    rec.update({"mfma_frac": round(mfma_frac, 4), "hbm_frac": round(hbm_frac, 4)})
    return rec, flops, nbytes


def executed_pair_fraction(w, mask, plan, bbsa) -> float:
    """Share of the pattern's (64-row query tile, key block) pairs that the
    bf16 kernels execute for this workload's mask: a tile leaves out the key
    blocks whose mask values are all 0 when its list (the kernels' own lists,
    from the library's work map) holds a key of mask 1, except the block at
    list position 0.  The useful flops above count every pattern pair,
    padding included; this is for reporting the work actually done."""
    if w.dtype != "bf16" or mask is None:
        return 1.0
    st, _, rec = bbsa.bbsa_work_map(w.B, w.H, w.L, w.d, w.block, w.r, bbsa.BBSA_BF16, plan)
    if st < 0 or len(rec) == 0:
        return 1.0
    blocks = mask.reshape(w.B, w.nb, w.block)
    padded = (blocks == 0).all(axis=2)          # [B, nb]
    has_one = (blocks == 1).any(axis=2)         # [B, nb]
    total = executed = 0
    for row in rec:
        b = int(row[3]) // w.H
        lst = row[16 + row[8]:16 + row[9]]
        n = len(lst)
        total += n
        if has_one[b, lst].any():
            executed += n - int(padded[b, lst[1:]].sum())
        else:
            executed += n
    return executed / total if total else 1.0


def add_executed(roof, frac):
    """The executed share of the pattern pairs and the MFMA fraction of the
    work actually done (the fractions above count every pattern pair)."""
    roof["executed_pair_fraction"] = round(frac, 4)
    roof["executed_mfma_frac"] = round(roof["mfma_frac"] * frac, 4)


class Runner:
    """Device copies of one workload's inputs and the step that runs on them."""

    def __init__(self, wid, n_sets_arg, torch, bbsa, workloads):
        self.w = w = workloads.WORKLOADS[wid]
        elt = 2 if w.dtype == "bf16" else 4
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        log(f"workload {w.name}: generating inputs")
        self.inp = workloads.make_inputs(wid)
        self.plan = bbsa.bbsa_plan_rand_attn(w.H, w.nb, w.r, w.plan_seed)
        dev = torch.device("cuda:0")
        set_bytes = 4 * w.B * w.H * w.L * w.d * elt
        # Enough copies that one pass over them moves three times the 256 MB
        # last-level cache: no step reads inputs another step left in cache.
        self.n_sets = n_sets_arg or max(1, int(np.ceil(768e6 / set_bytes)))
        base = [torch.from_numpy(self.inp[n]).to(tdt).to(dev) for n in ("q", "k", "v")]
        self.sets = []
        for _ in range(self.n_sets):
            q, k, v = (t.clone() for t in base)
            self.sets.append((q, k, v, torch.empty_like(q)))
        del base
        self.mask = torch.from_numpy(self.inp["mask"]).to(dev) if w.masked else None
        self.ra = torch.from_numpy(self.plan).to(dev)
        self.stream = torch.cuda.current_stream(dev)
        self.bbsa = bbsa
        self.torch = torch

    keep_padded = False   # --keep-padded-blocks: compute every pattern block (for comparison)

    def step(self, i):
        q, k, v, o = self.sets[i % self.n_sets]
        if self.keep_padded:
            self.bbsa.bbsa_forward_ex(q, k, v, self.mask, self.ra, self.w.block, self.w.r, out=o,
                                      stream=self.stream, keep_padded_blocks=True)
        else:
            self.bbsa.bbsa_forward(q, k, v, self.mask, self.ra, self.w.block, self.w.r, out=o,
                                   stream=self.stream)

    def preroll(self, seconds):
        """Untimed steps for a fixed wall time before the warm-up steps: the
        GPU's clocks need tens of milliseconds of sustained work to ramp up."""
        torch = self.torch
        t0, i = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(50):
                self.step(i)
                i += 1
            torch.cuda.synchronize()
        return i

    def timed(self, steps, warmup, same_set=False):
        """Average step time in ms over ``steps`` back-to-back steps, bracketed
        by events on the launch stream (after ``warmup`` untimed steps)."""
        torch = self.torch
        for i in range(warmup):
            self.step(0 if same_set else i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(steps):
            self.step(0 if same_set else i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    def percentiles(self, steps):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(min(steps, 1000))]
        for i, (a, b) in enumerate(ev):
            a.record(self.stream)
            self.step(i)
            b.record(self.stream)
        torch.cuda.synchronize()
        per_step = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        return [round(float(np.percentile(per_step, x)), 2) for x in (10, 50, 90)]

    def kernel_events(self, steps):
        """The library's own events around each kernel: per-launch durations of
        the attention kernel and of the merge kernel (0 when none runs)."""
        bbsa, torch = self.bbsa, self.torch
        bbsa.bbsa_timing_enable(True)
        for i in range(min(steps, 4096)):
            self.step(i)
        torch.cuda.synchronize()
        main_ms, comb_ms, calls = bbsa.bbsa_timing_read()
        bbsa.bbsa_timing_enable(False)
        return main_ms / max(calls, 1) * 1e3, comb_ms / max(calls, 1) * 1e3

    def clock_under_load(self, seconds):
        """Mean graphics clock (MHz) that ``amd-smi metric -c`` reports for the
        GPU while this workload's steps run back to back for ``seconds``
        (untimed), with the number of readings; None when the tool is missing,
        fails or lists more than one GPU."""
        torch = self.torch
        readings, stop = [], threading.Event()

        def sample():
            while not stop.is_set():
                try:
                    res = subprocess.run(["amd-smi", "metric", "-c", "--json"], capture_output=True, text=True,
                                         timeout=10)
                    gpus = json.loads(res.stdout)["gpu_data"]
                    if len(gpus) != 1:
                        return
                    clk = [v["clk"]["value"] for k, v in gpus[0]["clock"].items() if k.startswith("gfx_")]
                    readings.append(sum(clk) / len(clk))
                except (OSError, ValueError, KeyError, TypeError, ZeroDivisionError, subprocess.SubprocessError):
                    return
                stop.wait(0.05)

        th = threading.Thread(target=sample, daemon=True)
        t0, i = time.perf_counter(), 0
        th.start()
        while time.perf_counter() - t0 < seconds:
            for _ in range(64):
                self.step(i)
                i += 1
            torch.cuda.synchronize()
        stop.set()
        th.join(timeout=15)
        if not readings:
            return None
        return {"mhz": round(float(np.mean(readings)), 1), "readings": len(readings),
                "tool": "amd-smi metric -c (mean of the gfx_* clocks)"}

    def close(self):
        self.sets = None
        self.torch.cuda.synchronize()
        self.torch.cuda.empty_cache()


def backward_leg(run, args, torch, bbsa):
    """Time one backward step (the dq kernel, the dk/dv kernel and, for
    split global rows and columns, the merge kernel) on the headline
    workload's inputs, after a forward that saved the output and the row
    log-sum-exp.  Useful flops: 2.5 times the
    forward's (the five products of the gradients; the recompute of the
    scores and the probability gradients in both kernels is not counted)."""
    w = run.w
    q, k, v, _ = run.sets[0]
    dout = torch.randn_like(q)
    keep = Runner.keep_padded
    out, lse, _ = bbsa.bbsa_forward_ex(q, k, v, run.mask, run.ra, w.block, w.r, return_lse=True,
                                       keep_padded_blocks=keep)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    delta = torch.empty_like(lse)

    def step():
        bbsa.bbsa_backward(q, k, v, out, dout, lse, run.mask, run.ra, w.block, w.r, dq=dq, dk=dk, dv=dv,
                           delta=delta, stream=run.stream, keep_padded_blocks=keep)

    t0 = time.perf_counter()
    while time.perf_counter() - t0 < args.preroll:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    n = max(1, args.steps // 4)
    for _ in range(max(1, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(run.stream)
    for _ in range(n):
        step()
    e1.record(run.stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 2.5 * useful_flops(w.B, w.H, w.nb, w.block, w.d, w.r)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"{w.name} backward: step {ms * 1e3:.2f} us; {tf:.1f} useful TFLOP/s; MFMA frac {tf / PEAK_BF16_TFLOPS:.4f}")
    return {"step_us": round(ms * 1e3, 3), "steps": n, "useful_gflop_per_step": round(flops / 1e9, 3),
            "useful_tflops": round(tf, 3),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--workload", type=int, default=2, help="headline workload id 1..5 (default 2)")
    ap.add_argument("--others", default="3,4,5",
                    help="other workload ids timed in the same run ('' for none)")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--preroll", type=float, default=0.3,
                    help="seconds of untimed steps before each workload's warm-up (clock ramp)")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0 = auto)")
    ap.add_argument("--clock-seconds", type=float, default=1.0,
                    help="seconds of untimed steps while amd-smi reads the graphics clock (0: skip)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--keep-padded-blocks", action="store_true",
                    help="compute the key blocks whose keys are all padded (BBSA_FLAG_KEEP_PADDED_BLOCKS)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported "
              "(the operator shards over (batch, head) with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from block_sparse_long_bbsa_amd import bbsa, workloads

    if args.copy_calibration:
        # A plain copy of known size: 256 MiB read + 256 MiB written per dispatch.
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_dispatch": n, "dispatches": 5}), flush=True)
        return

    Runner.keep_padded = args.keep_padded_blocks
    # Headline workload.
    run = Runner(args.workload, args.sets, torch, bbsa, workloads)
    w, n_sets = run.w, run.n_sets
    pre = run.preroll(args.preroll)
    ms = run.timed(args.steps, args.warmup)
    p10, p50, p90 = run.percentiles(args.steps)
    warm_us = run.timed(args.steps, 0, same_set=True) * 1e3
    kern_us, merge_us = run.kernel_events(args.steps)
    roof, flops, nbytes = roofline(w, ms)
    roof["traffic"] = read_traffic(w.name)
    roof["kernel"] = "bbsa_attn_bf16" if w.dtype == "bf16" else "bbsa_attn_f32"
    add_executed(roof, executed_pair_fraction(w, run.inp["mask"] if w.masked and not Runner.keep_padded else None,
                                              run.plan, bbsa))
    # The step is one attention-kernel launch (plus the merge kernel only for
    # rows of more than four key chunks), so the average launch duration over the
    # timed region is the step time; per-launch events (which add their own
    # overhead) are reported beside it.
    roof["kernel_us"] = round(ms * 1e3, 3)
    roof["per_launch_event_us"] = {"attention": round(kern_us, 3), "merge": round(merge_us, 3)}
    # The peaks assume the 2.4 GHz specification clock; the graphics clock
    # that amd-smi reports while the same steps run on (untimed).
    roof["amd_smi_gfx_clock"] = run.clock_under_load(args.clock_seconds) if args.clock_seconds > 0 else None
    value = flops / (ms * 1e-3) / 1e12
    log(f"{w.name}: step {ms * 1e3:.2f} us (p10/p50/p90 {p10}/{p50}/{p90}, warm {warm_us:.1f}); "
        f"{value:.1f} useful TFLOP/s; frac {roof['frac']} ({roof['bound']}); "
        f"MFMA {roof['mfma_frac']} HBM {roof['hbm_frac']}")
    backward = None
    if not args.no_backward and w.dtype == "bf16":
        backward = backward_leg(run, args, torch, bbsa)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(run.inp, run.plan, w, args.cpu_budget)
    run.close()
    del run

    # Other workloads at L >= 4096, same protocol, one JSON entry each.
    others = []
    for tok in [t for t in args.others.split(",") if t.strip()]:
        wid = int(tok)
        if wid == args.workload:
            continue
        r2 = Runner(wid, args.sets, torch, bbsa, workloads)
        r2.preroll(args.preroll)
        ms2 = r2.timed(args.steps, args.warmup)
        rf2, fl2, nb2 = roofline(r2.w, ms2)
        add_executed(rf2, executed_pair_fraction(r2.w, r2.inp["mask"] if r2.w.masked and not Runner.keep_padded
                                                 else None, r2.plan, bbsa))
        v2 = fl2 / (ms2 * 1e-3) / 1e12
        log(f"{r2.w.name}: step {ms2 * 1e3:.2f} us; {v2:.1f} useful TFLOP/s; frac {rf2['frac']} "
            f"({rf2['bound']}); MFMA {rf2['mfma_frac']} HBM {rf2['hbm_frac']}")
        others.append({"workload": r2.w.name, "step_us": round(ms2 * 1e3, 3),
                       "useful_tflops": round(v2, 3), "useful_gflop_per_step": round(fl2 / 1e9, 3),
                       "algorithmic_mb_per_step": round(nb2 / 1e6, 3), "roofline": rf2})
        r2.close()
        del r2

    rec = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "block": w.block,
                   "r": w.r, "useful_gflop_per_step": round(flops / 1e9, 3),
                   "algorithmic_mb_per_step": round(nbytes / 1e6, 3), "input_sets": n_sets,
                   "step_us_p10_p50_p90": [p10, p50, p90],
                   "warm_step_us": round(warm_us, 2),
                   "preroll": {"seconds": args.preroll, "steps": pre},
                   "parallelism": "none (1 GPU)",
                   "keep_padded_blocks": bool(args.keep_padded_blocks),
                   "other_workloads": others,
                   "backward": backward},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
