#!/usr/bin/env python3
"""Benchmark of block-causal ReLU linear attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c2|c3|c4|c5]
                    [--c4-mode stream|oneshot] [--rotate R] [--settle S] [--no-cpu-baseline]

A step is one pass of the whole path (state build -> scan -> apply) over one
batch of the workload's synthetic input, with inputs resident in HBM.  R
copies of the inputs and outputs rotate so that consecutive steps do not hit
in the 256 MB Infinity Cache.  About S seconds of untimed steps let the
clocks settle, then W untimed steps, then K timed steps between two device
synchronisations; one JSON line on stdout.

Also:
  --copy-calibration           time a plain device copy of known size (run it
                               under rocprofv3 --pmc to calibrate byte counters)
  --summarize-counters F W CF CW
                               fold rocprofv3 --pmc CSVs (FETCH_SIZE run F,
                               WRITE_SIZE run W, and the same two counters
                               over --copy-calibration runs CF, CW) into
                               profiles/counters_<config>.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block linear-attn tokens·heads/s + achieved HBM GB/s vs MI355X peak"
UNIT = "tokens·heads/s"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
SOURCE = os.path.join(ROOT, "block_causal_linear_relu_amd", "csrc", "svla.hip")
KERNEL_SLOTS = {"build": (0, 1), "scan": (2, 3), "apply": (4, 5)}
COPY_BYTES = 1 << 29            # 512 MiB read + 512 MiB written


def source_hash() -> str:
    return hashlib.sha256(open(SOURCE, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--c4-mode", default="stream", choices=["stream", "oneshot"])
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup (clock settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------
class Workload:
    """Device buffers (R rotating sets) and the call for one step."""

    def __init__(self, name: str, rotate: int, c4_mode: str):
        import torch
        import block_causal_linear_relu_amd as svla
        from workloads import CONFIGS, make_inputs

        self.torch, self.svla = torch, svla
        self.cfg = cfg = CONFIGS[name]
        self.name = name
        self.stream_mode = name == "c4" and c4_mode == "stream"
        x = make_inputs(cfg)
        self.x = x
        dev = torch.device("cuda:0")
        bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
        Q, K, V = bf(x["Q"]), bf(x["K"]), bf(x["V"])
        self.g = None if x["g"] is None else torch.from_numpy(x["g"]).to(dev)
        B, H, N, d = Q.shape
        self.B, self.H, self.N, self.d, self.nb, self.n = B, H, N, d, cfg.nb, cfg.n
        self.sets = []
        for r in range(rotate):
            if self.stream_mode:
                n = cfg.n
                blocks = [tuple(t[:, :, s * n:(s + 1) * n].contiguous() for t in (Q, K, V))
                          for s in range(cfg.nb)]
                outs = [torch.empty_like(blocks[0][0]) for _ in range(cfg.nb)]
                S = torch.zeros((B, H, d, d), device=dev)
                z = torch.zeros((B, H, d), device=dev)
                self.sets.append((blocks, outs, S, z))
            else:
                q, k, v = (Q, K, V) if r == 0 else (Q.clone(), K.clone(), V.clone())
                self.sets.append((q, k, v, torch.empty_like(q)))
        del Q, K, V
        if self.stream_mode:
            self.ws = torch.empty(svla.workspace_size("block_step", torch.bfloat16, B, H, 1,
                                                      cfg.n, d), dtype=torch.uint8, device=dev)
            self.frames = cfg.n // (cfg.rope.grid_h * cfg.rope.grid_w)
            self.ropes = [cfg.rope.with_t0(self.frames * s) for s in range(cfg.nb)]
        else:
            op = "noncausal" if cfg.nb == 1 else "block_causal"
            self.ws = torch.empty(svla.workspace_size(op, torch.bfloat16, B, H, cfg.nb, cfg.n, d),
                                  dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N

    def launches_per_step(self) -> int:
        return self.nb if self.stream_mode else 1

    def algorithmic_bytes(self) -> dict:
        """Bytes the method must move (Q, K, V read once, O written once; the
        carried state read and written once per streaming step)."""
        e = 2
        t = self.B * self.H * self.N * self.d * e
        per_launch = {"build": 2 * t, "apply": 2 * t, "scan": 0}
        state = self.B * self.H * (self.d * self.d + self.d) * 4
        if self.stream_mode:
            per_launch = {k: v // self.nb for k, v in per_launch.items()}
            per_launch["scan"] = 2 * state
            path = 4 * t + 2 * state * self.nb
        else:
            path = 4 * t
        return {"per_launch": per_launch, "path": path}

    def stream_pass(self, r: int):
        """The 80 block steps of one video; the state starts from zero."""
        blocks, outs, S, z = self.sets[r]
        for s in range(self.nb):
            q, k, v = blocks[s]
            self.svla.block_step(q, k, v, S if s else None, z if s else None, S_out=S, z_out=z,
                                 rope=self.ropes[s], out=outs[s], workspace=self.ws)

    def capture(self):
        """Streaming mode: capture each set's pass in a HIP graph (the 240
        launches of a pass would otherwise be bound by host launch cost)."""
        torch = self.torch
        self.graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for r in range(len(self.sets)):
                self.stream_pass(r)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for r in range(len(self.sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.stream_pass(r)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def step(self, i: int):
        svla = self.svla
        if self.stream_mode:
            r = i % len(self.sets)
            if getattr(self, "graphs", None):
                self.graphs[r].replay()
            else:
                self.stream_pass(r)
        else:
            q, k, v, o = self.sets[i % len(self.sets)]
            if self.nb == 1:
                svla.noncausal(q, k, v, out=o, workspace=self.ws)
            else:
                svla.block_causal(q, k, v, self.nb, g=self.g, rope=self.cfg.rope, out=o,
                                  workspace=self.ws)

    def describe_plan(self) -> dict:
        """The library's launch plan for one call of this workload."""
        torch = self.torch
        if self.stream_mode:
            return self.svla.describe("block_step", torch.bfloat16, self.B, self.H, 1, self.n,
                                      self.d, rope=self.ropes[0])
        op = "noncausal" if self.nb == 1 else "block_causal"
        return self.svla.describe(op, torch.bfloat16, self.B, self.H, self.nb, self.n, self.d,
                                  rope=self.cfg.rope)

    def describe(self) -> dict:
        c = self.cfg
        d = {"workload": "%s: %s" % (c.name, c.description), "B": c.B, "H": c.H, "N": c.N,
             "d": c.d, "blocks": c.nb, "block_tokens": c.n, "input_dtype": c.dtype,
             "rope": c.rope is not None, "gated": c.gated, "rotating_input_sets": len(self.sets)}
        if c.name == "c4":
            d["c4_mode"] = ("80 sequential block steps (HIP graph per pass)" if self.stream_mode
                            else "one-shot call over the 80 blocks")
        return d


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------
def settle(w: Workload, seconds: float) -> int:
    """Run the step, untimed, for about `seconds` of wall time so the GPU
    leaves its idle clock state before the warmup steps (a fresh process's
    first few hundred milliseconds of work run measurably slower)."""
    torch = w.torch
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            w.step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_steps(w: Workload, steps: int, warmup: int) -> float:
    torch = w.torch
    for i in range(warmup):
        w.step(i)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps):
        w.step(i)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps       # ms per step


def time_kernels(w: Workload, steps: int) -> dict:
    """Average duration (ms) per launch of each kernel, from HIP events the
    library records between its own launches, on the launch stream."""
    torch, svla = w.torch, w.svla
    per_step = w.launches_per_step()
    total = {k: 0.0 for k in KERNEL_SLOTS}
    count = 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    svla.set_timing_events(ev)
    try:
        for i in range(steps):
            if w.stream_mode:
                # eager, one block step at a time, so the 6 events describe one launch set
                blocks, outs, S, z = w.sets[i % len(w.sets)]
                for s in range(w.nb):
                    q, k, v = blocks[s]
                    svla.block_step(q, k, v, S if s else None, z if s else None, S_out=S,
                                    z_out=z, rope=w.ropes[s], out=outs[s], workspace=w.ws)
                    torch.cuda.synchronize()
                    for name, (a, b) in KERNEL_SLOTS.items():
                        total[name] += ev[a].elapsed_time(ev[b])
                    count += 1
            else:
                w.step(i)
                torch.cuda.synchronize()
                for name, (a, b) in KERNEL_SLOTS.items():
                    total[name] += ev[a].elapsed_time(ev[b])
                count += 1
    finally:
        svla.set_timing_events(None)
    assert count == steps * per_step
    return {k: v / count for k, v in total.items()}


def cpu_baseline(w: Workload, budget_s: float = 10.0) -> dict:
    """The fp64 oracle, as it stands, on the host cores: the full workload,
    repeated until about `budget_s` seconds of wall time have passed."""
    import numpy as np
    import oracle

    x = w.x
    Q, K, V = (np.ascontiguousarray(x[k], dtype=np.float64) for k in "QKV")
    threads = len(os.sched_getaffinity(0))
    reps, secs, used = 0, 0.0, threads
    kw = dict(g=x["g"], rope=w.cfg.rope, eps=x["eps"], threads=threads)
    while secs < budget_s and reps < 1000:
        r = oracle.forward(Q, K, V, w.cfg.nb, **kw)
        secs += r["seconds"]
        used = r["threads"]
        reps += 1
    return {"value": reps * w.tokens_heads / secs, "unit": UNIT, "cores": used,
            "kind": "oracle",
            "sample": "%d full run(s) of %s (%d tokens x %d heads x batch %d, fp64, one-shot "
                      "over all %d blocks), %.1f s on %d host threads"
                      % (reps, w.name, w.N, w.H, w.B, w.cfg.nb, secs, used)}


def load_traffic(config: str, kernel: str, launches_per_step: int):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when the summary is missing or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % config)
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("source_sha256") != source_hash():
        return None
    k = c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_dispatch")


# ---------------------------------------------------------------------------
# rocprofv3 counter summaries
# ---------------------------------------------------------------------------
def _pmc_rows(path):
    files = [path] if os.path.isfile(path) else glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no counter_collection.csv under %s" % path)
    return rows


def _per_kernel(rows, counter):
    """Mean counter value per dispatch, grouped by a short kernel name."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        name = r.get("Kernel_Name", "").replace("(anonymous namespace)::", "")
        short = name.split("(")[0].strip()
        disp = r.get("Dispatch_Id")
        acc.setdefault(short, {}).setdefault(disp, 0.0)
        acc[short][disp] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, config):
    fetch = _per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = _per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")
    cf = _per_kernel(_pmc_rows(copy_fetch_dir), "FETCH_SIZE")
    cw = _per_kernel(_pmc_rows(copy_write_dir), "WRITE_SIZE")
    # the calibration run's copy kernel: the one with the largest fetch
    copy_name = max(cf, key=cf.get)
    f_factor = COPY_BYTES / (cf[copy_name] * 1024.0)
    w_factor = COPY_BYTES / (cw[copy_name] * 1024.0)
    out = {"source_sha256": source_hash(), "config": config,
           "copy_kernel": copy_name, "copy_bytes": COPY_BYTES,
           "fetch_factor": f_factor, "write_factor": w_factor, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if not k.startswith("void svla") and "svla" not in k:
            continue
        fb = fetch.get(k, 0.0) * 1024.0 * f_factor
        wb = write.get(k, 0.0) * 1024.0 * w_factor
        out["kernels"][k] = {"fetch_kib": fetch.get(k), "write_kib": write.get(k),
                             "hbm_bytes_per_dispatch": fb + wb}
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % config)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def copy_calibration():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 3}))


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, config=args.config)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only (the path shards by (batch, head) with no "
              "communication, so N GPUs run N independent calls); --gpus %d is not supported"
              % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    w = Workload(args.config, args.rotate, args.c4_mode)
    if w.stream_mode:
        w.capture()
    settled = settle(w, args.settle) if args.settle > 0 else 0
    ms = time_steps(w, args.steps, args.warmup)
    plan = w.describe_plan()
    used = {k["slot"] for k in plan["kernels"]}
    # a call that folds the scan into the apply launches no scan kernel
    kern = {k: v for k, v in time_kernels(w, max(5, min(args.steps, 50))).items() if k in used}
    ab = w.algorithmic_bytes()
    dominant = max(("build", "apply"), key=lambda k: kern[k])
    dur_s = kern[dominant] * 1e-3
    achieved = ab["per_launch"][dominant] / dur_s / 1e9
    kernel_full = {k["slot"]: k["name"] for k in plan["kernels"]}[dominant]
    traffic = load_traffic(args.config, kernel_full, w.launches_per_step())
    path_gbps = ab["path"] / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": w.tokens_heads / (ms * 1e-3),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settled,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16-rounded; shapes of the pages' video workloads)",
        "config": w.describe(),
        "roofline": {"bound": "hbm", "kernel": kernel_full, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": ab["per_launch"][dominant],
                     "avg_launch_ms": kern[dominant]},
        "path": {"algorithmic_bytes_per_step": ab["path"], "achieved_GBps": path_gbps,
                 "frac_of_peak": path_gbps / HBM_PEAK_GBPS,
                 "kernel_ms_per_launch": kern, "launches_per_step": w.launches_per_step(),
                 "plan": plan},
        "source_sha256": source_hash(),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
