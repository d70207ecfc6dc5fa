#!/usr/bin/env python3
"""Benchmark of block-causal ReLU linear attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4|c2|c3|c5|t3|t4]
                    [--c4-mode both|stream|oneshot] [--inplace] [--stream] [--dtype fp8]
                    [--backward] [--anchor] [--rotate R] [--settle S] [--no-cpu-baseline]

A step is one pass of the whole path over one batch of the workload's
synthetic input, with the inputs resident in HBM.  R copies of the inputs and
outputs rotate so that consecutive steps do not hit in the 256 MB Infinity
Cache.  About S seconds of untimed steps let the clocks settle, then W untimed
steps, then K timed steps between two device synchronisations; one JSON line
on stdout.

The default workload is the minute-long 480p stream (B1 H70 d32, 80 blocks of
1170 tokens, 3D RoPE), the largest one: a step is the 80 sequential
`svla_block_step` calls of one video (replayed from a HIP graph), with the
state committed into the other of two state buffers (the one-launch step;
--inplace commits in place, the two-kernel step).  `value` is that stream's
tokens*heads/s.  With --c4-mode both (the default) the same 80 blocks are also
timed as one `svla_block_causal` call and reported under "c4_oneshot".

Also:
  --ceiling                    time a plain device copy and a read-only
                               reduction of 2 GiB (the achievable HBM rates)
  --copy-calibration           a plain device copy of known size (run it under
                               rocprofv3 --pmc to calibrate byte counters)
  --summarize-counters F W CF CW --tag T
                               fold rocprofv3 --pmc CSVs (FETCH_SIZE run F,
                               WRITE_SIZE run W, and the same two counters
                               over --copy-calibration runs CF, CW) into
                               profiles/counters_<T>.json
  --summarize-mfma M --tag T   fold a rocprofv3 --pmc run of the matrix-core
                               counters into profiles/mfma_<T>.json
  --summarize-kernels CSV --tag T
                               profiles/kernels_<workload>.md from a rocprofv3
                               --kernel-trace --stats kernel_stats.csv
  --summarize-tables           the traffic and matrix-core tables in profiles/
                               from the current source's summaries
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, published
GATE_FRAC = 0.60                # the minute-long and 720p shapes' target fraction of peak HBM
SOURCE = os.path.join(ROOT, "block_causal_linear_relu_amd", "csrc", "svla.hip")
KERNEL_SLOTS = {"build": (0, 1), "scan": (2, 3), "apply": (4, 5), "step": (6, 7), "conv": (8, 9),
                "bwd_query": (10, 11), "bwd_scan": (12, 13), "bwd_key": (14, 15)}
BWD_METRIC = "block-causal linear-attn backward tokens·heads/s + achieved HBM GB/s vs MI355X peak"
ANCHOR_METRIC = "block-causal softmax anchor tokens·heads/s + achieved TFLOP/s vs MI355X bf16 MFMA peak"
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
CONV_METRIC = "causal temporal conv frames·positions·channels/s + achieved HBM GB/s vs MI355X peak"
CONV_UNIT = "frames·positions·channels/s"
COPY_BYTES = 1 << 29            # 512 MiB read + 512 MiB written
# one rocprofv3 --pmc pass (3 SQ counters underneath, 1 GRBM): MfmaUtil =
# 100 * sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMDs); MfmaFlopsBF16 =
# 512 * SQ_INSTS_VALU_MFMA_MOPS_BF16; VALUBusy = 100 * sum SQ_ACTIVE_INST_VALU /
# CUs / GRBM_GUI_ACTIVE (the box's own derived-counter definitions)
MFMA_COUNTERS = ("MfmaUtil", "MfmaFlopsBF16", "VALUBusy", "GRBM_GUI_ACTIVE")


def source_hash() -> str:
    return hashlib.sha256(open(SOURCE, "rb").read()).hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=["c2", "c3", "c4", "c5", "t3", "t4"])
    ap.add_argument("--c4-mode", default="both", choices=["both", "stream", "oneshot"])
    ap.add_argument("--stream", action="store_true",
                    help="c3, c5: time the workload as one svla_block_step per block (the gated "
                         "d = 128 block step for c5) instead of one call")
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp8"],
                    help="input type of Q, K, V (fp8: OCP E4M3, d = 32 workloads; O stays bf16)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (block-causal training) of the workload")
    ap.add_argument("--anchor", action="store_true",
                    help="time the 2.0 hybrid's softmax anchor layer on the gated 720p shape (c5)")
    ap.add_argument("--inplace", action="store_true",
                    help="streaming: commit the state in place (the two-kernel step)")
    ap.add_argument("--rotate", type=int, default=4)
    ap.add_argument("--settle", type=float, default=0.5,
                    help="seconds of untimed steps before the warmup (clock settling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ceiling", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-counters", nargs=4,
                    metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    ap.add_argument("--summarize-mfma", metavar="DIR")
    ap.add_argument("--summarize-kernels", metavar="KERNEL_STATS_CSV",
                    help="write profiles/kernels_<workload>.md for --tag from a rocprofv3 --stats CSV")
    ap.add_argument("--summarize-tables", action="store_true",
                    help="rewrite the traffic and matrix-core tables in profiles/ from the summaries")
    ap.add_argument("--tag", help="name of the summary written by --summarize-*")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------
class Workload:
    """Device buffers (R rotating sets) and the call for one step.

    mode: "oneshot" (one call over all blocks; the non-causal call for a
    one-block workload), "stream" (one svla_block_step per block, the state
    double-buffered) or "stream_inplace" (the state committed in place)."""

    def __init__(self, name: str, rotate: int, mode: str, x=None, dtype: str = "bf16"):
        import torch
        import block_causal_linear_relu_amd as svla
        from workloads import CONFIGS, make_inputs, scaled_config

        self.torch, self.svla = torch, svla
        self.cfg = cfg = scaled_config(CONFIGS[name], dtype=dtype) if dtype != "bf16" else CONFIGS[name]
        self.tdt = torch.float8_e4m3fn if cfg.dtype == "fp8" else torch.bfloat16
        self.name = name
        self.mode = mode
        self.stream_mode = mode != "oneshot"
        x = make_inputs(cfg) if x is None else x
        self.x = x
        dev = torch.device("cuda:0")
        if cfg.dtype == "fp8":
            bf = lambda k: torch.from_numpy(x[k + "_bits"]).to(dev).view(torch.float8_e4m3fn)
        else:
            bf = lambda k: torch.from_numpy(x[k]).to(dev).to(torch.bfloat16)
        Q, K, V = bf("Q"), bf("K"), bf("V")
        self.g = None if x["g"] is None else torch.from_numpy(x["g"]).to(dev)
        B, H, N, d = Q.shape
        self.B, self.H, self.N, self.d, self.nb, self.n = B, H, N, d, cfg.nb, cfg.n
        self.sets = []
        nbuf = 2 if mode == "stream" else 1
        for r in range(rotate):
            if self.stream_mode:
                n = cfg.n
                blocks = [tuple(t[:, :, s * n:(s + 1) * n].contiguous() for t in (Q, K, V))
                          for s in range(cfg.nb)]
                outs = [torch.empty(blocks[0][0].shape, dtype=torch.bfloat16, device=dev)
                        for _ in range(cfg.nb)]
                states = [(torch.zeros((B, H, d, d), device=dev), torch.zeros((B, H, d), device=dev))
                          for _ in range(nbuf)]
                self.sets.append((blocks, outs, states))
            else:
                q, k, v = (Q, K, V) if r == 0 else (Q.clone(), K.clone(), V.clone())
                self.sets.append((q, k, v, torch.empty(q.shape, dtype=torch.bfloat16, device=dev)))
        del Q, K, V
        if self.stream_mode:
            self.ws = torch.empty(svla.workspace_size("block_step", self.tdt, B, H, 1,
                                                      cfg.n, d), dtype=torch.uint8, device=dev)
            self.frames = cfg.n // (cfg.rope.grid_h * cfg.rope.grid_w) if cfg.rope else 0
            self.ropes = [cfg.rope.with_t0(self.frames * s) if cfg.rope else None
                          for s in range(cfg.nb)]
            self.gs = [None if self.g is None else self.g[:, :, s].contiguous()
                       for s in range(cfg.nb)]
        else:
            op = "noncausal" if cfg.nb == 1 else "block_causal"
            self.ws = torch.empty(svla.workspace_size(op, self.tdt, B, H, cfg.nb, cfg.n, d),
                                  dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N

    def launches_per_step(self) -> int:
        return self.nb if self.stream_mode else 1

    def algorithmic_bytes(self) -> dict:
        """Bytes the method must move (Q, K, V read once, O written once; the
        carried state read and written once per streaming step).  Per launch
        of each kernel: the state build K and V, the read-out Q and O, the
        one-launch step all four plus the state; the scan nothing."""
        e = 1 if self.cfg.dtype == "fp8" else 2
        t = self.B * self.H * self.N * self.d * e          # one input tensor
        o = self.B * self.H * self.N * self.d * 2          # O (bf16)
        state = self.B * self.H * (self.d * self.d + self.d) * 4
        per_launch = {"build": 2 * t, "apply": t + o, "scan": 0, "step": 3 * t + o}
        if self.stream_mode:
            per_launch = {k: v // self.nb for k, v in per_launch.items()}
            per_launch["step"] += 2 * state
            path = 3 * t + o + 2 * state * self.nb
        else:
            path = 3 * t + o
        return {"per_launch": per_launch, "path": path}

    def block_step(self, r: int, s: int):
        """Block s of rotating set r; the state starts from zero at block 0."""
        blocks, outs, states = self.sets[r]
        S, z = states[s % len(states)]
        S_next, z_next = states[(s + 1) % len(states)]
        q, k, v = blocks[s]
        self.svla.block_step(q, k, v, S if s else None, z if s else None, S_out=S_next,
                             z_out=z_next, g=self.gs[s], rope=self.ropes[s], out=outs[s],
                             workspace=self.ws)

    def stream_pass(self, r: int):
        for s in range(self.nb):
            self.block_step(r, s)

    def capture(self):
        """Streaming: capture each set's pass in a HIP graph (the launches of a
        pass would otherwise be bound by host launch cost)."""
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
        r = i % len(self.sets)
        if self.stream_mode:
            if getattr(self, "graphs", None):
                self.graphs[r].replay()
            else:
                self.stream_pass(r)
        else:
            q, k, v, o = self.sets[r]
            if self.nb == 1:
                svla.noncausal(q, k, v, out=o, workspace=self.ws)
            else:
                svla.block_causal(q, k, v, self.nb, g=self.g, rope=self.cfg.rope, out=o,
                                  workspace=self.ws)

    def plan(self) -> dict:
        """The library's launch plan for one call of this workload, as taken."""
        torch = self.torch
        if self.stream_mode:
            p = self.svla.describe("block_step", self.tdt, self.B, self.H, 1, self.n,
                                   self.d, rope=self.ropes[0])
            if self.mode == "stream_inplace" and p.get("fused"):
                p["kernels"] = p["in_place_kernels"]
                p["fused"] = False
            return p
        op = "noncausal" if self.nb == 1 else "block_causal"
        return self.svla.describe(op, self.tdt, self.B, self.H, self.nb, self.n, self.d,
                                  rope=self.cfg.rope)

    def describe(self) -> dict:
        c = self.cfg
        d = {"workload": "%s: %s" % (c.name, c.description), "B": c.B, "H": c.H, "N": c.N,
             "d": c.d, "blocks": c.nb, "block_tokens": c.n, "input_dtype": c.dtype,
             "rope": c.rope is not None, "gated": c.gated, "rotating_input_sets": len(self.sets)}
        if self.mode == "stream":
            d["mode"] = ("%d sequential block steps per step (one HIP graph per pass), the state "
                         "committed into the other of two buffers" % c.nb)
        elif self.mode == "stream_inplace":
            d["mode"] = ("%d sequential block steps per step (one HIP graph per pass), the state "
                         "committed in place" % c.nb)
        else:
            d["mode"] = "one call over all %d blocks" % c.nb
        return d


class ConvWorkload:
    """The FFN's temporal convolution, causal across blocks: one call over the
    whole clip, or (streaming) one call per block of F frames with the cache
    carried in two buffers."""

    def __init__(self, name: str, rotate: int):
        import torch
        import block_causal_linear_relu_amd as svla
        from workloads import CONV_CONFIGS, make_conv_inputs

        self.torch, self.svla = torch, svla
        self.cfg = cfg = CONV_CONFIGS[name]
        self.name = name
        self.mode = "stream" if cfg.streaming else "oneshot"
        self.stream_mode = cfg.streaming
        self.x = x = make_conv_inputs(cfg)
        dev = torch.device("cuda:0")
        X = torch.from_numpy(x["X"]).to(dev).to(torch.bfloat16)
        self.w = torch.from_numpy(x["w"]).to(dev)
        self.b = torch.from_numpy(x["bias"]).to(dev)
        self.cache0 = torch.from_numpy(x["cache"]).to(dev).to(torch.bfloat16)
        self.nb, self.F = cfg.nb, cfg.F
        self.sets = []
        for r in range(rotate):
            Xr = X if r == 0 else X.clone()
            if self.stream_mode:
                blocks = [Xr[:, s * cfg.F:(s + 1) * cfg.F].contiguous() for s in range(cfg.nb)]
                outs = [torch.empty_like(blocks[0]) for _ in range(cfg.nb)]
                caches = [self.cache0.clone(), torch.empty_like(self.cache0)]
                self.sets.append((blocks, outs, caches))
            else:
                self.sets.append((Xr, torch.empty_like(Xr)))
        torch.cuda.synchronize()

    @property
    def tokens_heads(self) -> int:              # elements: frames x positions x channels
        c = self.cfg
        return c.B * c.T * c.P * c.C

    def launches_per_step(self) -> int:
        return self.nb if self.stream_mode else 1

    def algorithmic_bytes(self) -> dict:
        """X read once, Y written once (bf16); the cache frame read (and, when
        streaming, written) once per call."""
        c = self.cfg
        t = c.B * c.T * c.P * c.C * 2
        frame = c.B * c.P * c.C * 2
        if self.stream_mode:
            per = 2 * t // c.nb + 2 * frame
            return {"per_launch": {"conv": per}, "path": per * c.nb}
        return {"per_launch": {"conv": 2 * t + frame}, "path": 2 * t + frame}

    def block_step(self, r: int, s: int):
        blocks, outs, caches = self.sets[r]
        self.svla.temporal_conv(blocks[s], self.w, self.F, bias=self.b, cache_in=caches[s % 2],
                                cache_out=caches[(s + 1) % 2], out=outs[s])

    def stream_pass(self, r: int):
        for s in range(self.nb):
            self.block_step(r, s)

    capture = Workload.capture

    def step(self, i: int):
        r = i % len(self.sets)
        if self.stream_mode:
            if getattr(self, "graphs", None):
                self.graphs[r].replay()
            else:
                self.stream_pass(r)
        else:
            X, Y = self.sets[r]
            self.svla.temporal_conv(X, self.w, self.F, bias=self.b, cache_in=self.cache0, out=Y)

    def plan(self) -> dict:
        # the kernel's name as profilers report it (bf16, the library's default chunk length)
        return {"kernels": [{"slot": "conv", "name": "void svla_temporal_conv_k<2, 4>"}]}

    def describe(self) -> dict:
        c = self.cfg
        return {"workload": "%s: %s" % (c.name, c.description), "B": c.B, "frames": c.T,
                "frames_per_block": c.F, "positions": c.P, "channels": c.C, "input_dtype": c.dtype,
                "mode": ("%d block steps per step (one HIP graph per pass), the cache in two "
                         "buffers" % c.nb) if c.streaming else "one call over all %d blocks" % c.nb,
                "rotating_input_sets": len(self.sets)}


class BackwardWorkload:
    """The backward pass of one block-causal call over the whole workload:
    Q, K, V, dO in, dQ, dK, dV (and, gated, dg) out; R rotating sets."""

    def __init__(self, name: str, rotate: int, x=None):
        import torch
        import block_causal_linear_relu_amd as svla
        from workloads import CONFIGS, make_grad_output, make_inputs

        self.torch, self.svla = torch, svla
        self.cfg = cfg = CONFIGS[name]
        self.name, self.mode, self.stream_mode = name, "backward", False
        self.x = x = make_inputs(cfg) if x is None else x
        self.dO = dO = make_grad_output(x, 1000 + cfg.seed)
        dev = torch.device("cuda:0")
        t = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16)
        base = [t(x["Q"]), t(x["K"]), t(x["V"]), t(dO)]
        self.g = None if x["g"] is None else torch.from_numpy(x["g"]).to(dev)
        B, H, N, d = base[0].shape
        self.B, self.H, self.N, self.d, self.nb, self.n = B, H, N, d, cfg.nb, cfg.n
        self.sets = []
        for r in range(rotate):
            ins = base if r == 0 else [a.clone() for a in base]
            outs = {k: torch.empty_like(base[0]) for k in ("dQ", "dK", "dV")}
            if self.g is not None:
                outs["dg"] = torch.empty((B, H, cfg.nb), dtype=torch.float32, device=dev)
            self.sets.append((ins, outs))
        self.ws = torch.empty(svla.workspace_size("backward", torch.bfloat16, B, H, cfg.nb, cfg.n, d),
                              dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N

    def launches_per_step(self) -> int:
        return 1

    def algorithmic(self) -> dict:
        """Per launch of each kernel: HBM bytes the method must move and
        matrix flops (multiply-adds x 2) it must do.  Rebuild: K, V read,
        d^2 products per token.  Query side: Q, dO read, dQ written; three d x d
        products per token (S^T p~, S dnum, p~ dnum^T).  Key side: K, V read,
        dK, dV written; two (G^T a~, G v).  The scans: the d x d states only."""
        t = self.B * self.H * self.N * self.d * 2
        fl = 2 * self.B * self.H * self.N * self.d * self.d
        return {"bytes": {"build": 2 * t, "bwd_query": 3 * t, "bwd_key": 4 * t, "scan": 0, "bwd_scan": 0},
                "flops": {"build": fl, "bwd_query": 3 * fl, "bwd_key": 2 * fl, "scan": 0, "bwd_scan": 0},
                "path_bytes": 9 * t, "path_flops": 6 * fl}

    def block_step(self, r: int, s: int):
        self.step(r)

    def step(self, i: int):
        ins, outs = self.sets[i % len(self.sets)]
        q, k, v, dO = ins
        self.svla.block_causal_backward(q, k, v, dO, self.nb, g=self.g, rope=self.cfg.rope,
                                        eps=self.cfg.eps, workspace=self.ws, out=outs)

    def describe(self) -> dict:
        c = self.cfg
        return {"workload": "%s backward: %s" % (c.name, c.description), "B": c.B, "H": c.H,
                "N": c.N, "d": c.d, "blocks": c.nb, "block_tokens": c.n, "input_dtype": c.dtype,
                "rope": c.rope is not None, "gated": c.gated,
                "mode": "one backward call over all %d blocks (state rebuild, query side, reverse "
                        "scan, key side)" % c.nb, "rotating_input_sets": len(self.sets)}


def backward_cpu_baseline(w: BackwardWorkload, budget_s: float = 10.0) -> dict:
    """The numpy fp64 backward oracle on the host, head by head over the
    workload's heads until about `budget_s` seconds have passed."""
    from oracle.backward import backward
    x = w.x
    heads, secs = 0, 0.0
    while secs < budget_s and heads < w.B * w.H:
        b, h = divmod(heads, w.H)
        sl = lambda a: None if a is None else a[b:b + 1, h:h + 1]
        t = time.perf_counter()
        backward(sl(x["Q"]), sl(x["K"]), sl(x["V"]), w.nb, sl(w.dO), g=sl(x["g"]), rope=w.cfg.rope,
                 eps=x["eps"])
        secs += time.perf_counter() - t
        heads += 1
    return {"value": heads * w.N / secs, "unit": UNIT, "cores": 1, "kind": "oracle",
            "sample": "%d of %d (batch, head) slices of %s backward (numpy fp64), %.1f s"
                      % (heads, w.B * w.H, w.name, secs)}


def measure_backward(w: BackwardWorkload, args, settle_s: float) -> dict:
    settled = settle(w, settle_s) if settle_s > 0 else 0
    t = time_steps(w, args.steps, args.warmup)
    kern = time_kernels(w, max(5, min(args.steps, 50)))
    kern = {k: v for k, v in kern.items() if k in ("build", "scan", "bwd_query", "bwd_scan", "bwd_key")}
    al = w.algorithmic()
    per = {}
    for k in ("bwd_query", "bwd_key", "build"):
        dur = kern[k] * 1e-3
        tf = al["flops"][k] / dur / 1e12
        gb = al["bytes"][k] / dur / 1e9
        per[k] = {"avg_launch_ms": kern[k], "TFLOPs": tf, "GBps": gb, "frac_hbm": gb / HBM_PEAK_GBPS,
                  "flops_per_launch": al["flops"][k], "bytes_per_launch": al["bytes"][k]}
    names = {"bwd_query": "svla_bwd_query<%d, 2, %s>", "bwd_key": "svla_bwd_key<%d, 2, %s>"}
    r = "true" if w.cfg.rope else "false"
    # bf16 inputs at d = 32 run the products on the bf16 matrix cores (hi + lo
    # operands), far below their peak: both sides are bound by HBM, and the
    # line reports the slower one against 8 TB/s
    dom = max(("bwd_query", "bwd_key"), key=lambda k: per[k]["avg_launch_ms"])
    q = per[dom]
    kname = "void " + names[dom] % (w.d, r)
    ms = t["mean_ms"]
    return {
        "settle_steps": settled, "ms_per_step": ms, "value": w.tokens_heads / (ms * 1e-3),
        "timing": {k: t[k] for k in ("median_ms", "p10_ms", "p90_ms")},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": q["GBps"], "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": q["frac_hbm"],
                     "traffic": load_traffic(w.name + "_bwd", kname),
                     "algorithmic_bytes_per_launch": q["bytes_per_launch"],
                     "avg_launch_ms": q["avg_launch_ms"]},
        "kernels": per,
        "path": {"algorithmic_bytes_per_step": al["path_bytes"], "algorithmic_flops_per_step": al["path_flops"],
                 "achieved_GBps": al["path_bytes"] / (ms * 1e-3) / 1e9,
                 "achieved_TFLOPs": al["path_flops"] / (ms * 1e-3) / 1e12,
                 "kernel_ms_per_launch": kern},
        "mfma": load_mfma(w.name + "_bwd", kname),
    }


class AnchorWorkload:
    """One block-causal softmax anchor layer over a whole clip (queries of all
    nb blocks against all their keys), R rotating input sets."""

    def __init__(self, name: str, rotate: int):
        import numpy as np
        import torch
        import block_causal_linear_relu_amd as svla
        from workloads import CONFIGS, make_inputs

        self.torch, self.svla = torch, svla
        self.cfg = cfg = CONFIGS[name]
        self.name, self.mode, self.stream_mode = name, "anchor", False
        self.x = x = make_inputs(cfg)
        dev = torch.device("cuda:0")
        base = [torch.from_numpy(x[k]).to(dev).to(torch.bfloat16) for k in "QKV"]
        B, H, N, d = base[0].shape
        self.B, self.H, self.N, self.d, self.nb, self.n = B, H, N, d, cfg.nb, cfg.n
        self.sets = []
        for r in range(rotate):
            ins = base if r == 0 else [t.clone() for t in base]
            self.sets.append((ins, torch.empty_like(base[0])))
        torch.cuda.synchronize()

    @property
    def tokens_heads(self) -> int:
        return self.B * self.H * self.N

    def flops(self) -> int:
        """Matrix flops of the block-causal layer: block c's n queries against
        (c + 1) n keys, q.k and the weighted sum of v, 2 d flops each."""
        n, nb, d = self.n, self.nb, self.d
        return self.B * self.H * 4 * d * n * n * nb * (nb + 1) // 2

    def bytes(self) -> int:
        return self.B * self.H * self.N * self.d * 2 * 4       # Q, K, V read once, O written once

    def step(self, i: int):
        (q, k, v), o = self.sets[i % len(self.sets)]
        self.svla.softmax_attention(q, k, v, self.nb, out=o)

    def describe(self) -> dict:
        c = self.cfg
        return {"workload": "%s anchor: block-causal softmax attention on the shape of %s" % (c.name, c.description),
                "B": c.B, "H": c.H, "N": c.N, "d": c.d, "blocks": c.nb, "block_tokens": c.n,
                "input_dtype": "bf16", "scale": "1/sqrt(d)", "mode": "one call over all %d blocks" % c.nb,
                "rotating_input_sets": len(self.sets)}


def anchor_cpu_baseline(w: AnchorWorkload, budget_s: float = 10.0) -> dict:
    """The numpy fp64 softmax oracle on the host, head by head, until about
    `budget_s` seconds have passed."""
    from oracle.softmax import softmax_attention
    x = w.x
    heads, secs = 0, 0.0
    while secs < budget_s and heads < w.B * w.H:
        b, h = divmod(heads, w.H)
        sl = lambda a: a[b:b + 1, h:h + 1]
        t = time.perf_counter()
        softmax_attention(sl(x["Q"]), sl(x["K"]), sl(x["V"]), w.nb)
        secs += time.perf_counter() - t
        heads += 1
    return {"value": heads * w.N / secs, "unit": UNIT, "cores": len(os.sched_getaffinity(0)),
            "kind": "oracle",
            "sample": "%d of %d (batch, head) slices of the %s anchor (numpy fp64; its matrix products "
                      "use the BLAS threads), %.1f s" % (heads, w.B * w.H, w.name, secs)}


def conv_cpu_baseline(w: ConvWorkload, budget_s: float = 10.0) -> dict:
    """The numpy fp64 oracle of the temporal convolution on the host, repeated
    over the full workload until about `budget_s` seconds have passed."""
    from oracle.tconv import temporal_conv
    x = w.x
    reps, secs = 0, 0.0
    while secs < budget_s and reps < 1000:
        t = time.perf_counter()
        temporal_conv(x["X"], x["w"], x["F"], bias=x["bias"], cache_in=x["cache"])
        secs += time.perf_counter() - t
        reps += 1
    return {"value": reps * w.tokens_heads / secs, "unit": CONV_UNIT, "cores": 1, "kind": "oracle",
            "sample": "%d full run(s) of %s (numpy fp64, one call over all %d blocks), %.1f s"
                      % (reps, w.name, w.nb, secs)}


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


def _pct(xs, p):
    xs = sorted(xs)
    k = (len(xs) - 1) * p / 100.0
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def time_steps(w: Workload, steps: int, warmup: int) -> dict:
    """K steps between two device synchronisations, an event before each step
    and one after the last: the mean over the whole bracket, and the median,
    p10 and p90 of the single steps (ms)."""
    torch = w.torch
    for i in range(warmup):
        w.step(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i].record()
        w.step(i)
    ev[steps].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return {"mean_ms": ev[0].elapsed_time(ev[steps]) / steps, "median_ms": _pct(per, 50),
            "p10_ms": _pct(per, 10), "p90_ms": _pct(per, 90)}


def time_kernels(w: Workload, steps: int) -> dict:
    """Average duration (ms) per launch of each kernel, from HIP events the
    library records around its own launches, on the launch stream."""
    torch, svla = w.torch, w.svla
    total = {k: 0.0 for k in KERNEL_SLOTS}
    count = 0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * len(KERNEL_SLOTS))]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    svla.set_timing_events(ev)
    try:
        for i in range(steps):
            if w.stream_mode:
                # eager, one block step at a time, so the events describe one launch set
                for s in range(w.nb):
                    w.block_step(i % len(w.sets), s)
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
    assert count == steps * w.launches_per_step()
    return {k: v / count for k, v in total.items()}


def cpu_baseline(w: Workload, budget_s: float = 10.0, single_thread: bool = False) -> dict:
    """The fp64 oracle, as it stands, on the host cores: the full workload,
    repeated until about `budget_s` seconds of wall time have passed.  With
    single_thread, also one thread on a bounded sample of heads."""
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
    out = {"value": reps * w.tokens_heads / secs, "unit": UNIT, "cores": used,
           "kind": "oracle", "affinity_cores": threads,
           "sample": "%d full run(s) of %s (%d tokens x %d heads x batch %d, fp64, one call "
                     "over all %d blocks), %.1f s on %d host threads"
                     % (reps, w.name, w.N, w.H, w.B, w.cfg.nb, secs, used)}
    if single_thread:
        hs = slice(0, max(1, w.H // 7))
        sub = lambda a: None if a is None else np.ascontiguousarray(a[:, hs])
        r = oracle.forward(sub(Q), sub(K), sub(V), w.cfg.nb, g=sub(x["g"]), rope=w.cfg.rope,
                           eps=x["eps"], threads=1)
        th = w.B * (hs.stop - hs.start) * w.N
        out["single_thread"] = {"value": th / r["seconds"], "unit": UNIT, "cores": r["threads"],
                                "sample": "%d of %d heads of %s on one thread, %.1f s"
                                          % (hs.stop - hs.start, w.H, w.name, r["seconds"])}
    return out


def _load_summary(prefix: str, tag: str):
    path = os.path.join(ROOT, "profiles", "%s_%s.json" % (prefix, tag))
    if not os.path.exists(path):
        return None
    c = json.load(open(path))
    if c.get("source_sha256") != source_hash():
        return None          # the kernels changed since the counters were taken
    return c


def load_traffic(tag: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when the summary is missing or the kernels changed since."""
    c = _load_summary("counters", tag)
    k = None if c is None else c.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_dispatch")


def load_mfma(tag: str, kernel: str):
    c = _load_summary("mfma", tag)
    return None if c is None else c.get("kernels", {}).get(kernel)


def measure(w: Workload, args, settle_s: float) -> dict:
    """Timing of K steps, per-kernel times, roofline of the dominant kernel."""
    if w.stream_mode:
        w.capture()
    settled = settle(w, settle_s) if settle_s > 0 else 0
    t = time_steps(w, args.steps, args.warmup)
    plan = w.plan()
    used = {k["slot"] for k in plan["kernels"]}
    # a call that folds the scan into the apply launches no scan kernel
    kern = {k: v for k, v in time_kernels(w, max(5, min(args.steps, 50))).items() if k in used}
    kern_eager = None
    if w.stream_mode and used == {"step"}:
        # the one-launch step is the only kernel of the timed graph replays:
        # its average launch duration is the timed region over the launches
        # in it (gaps between launches included).  The eager events, one step
        # at a time after a device synchronisation, start each kernel on an
        # idle GPU and read about 1 us longer; they are kept for reference.
        kern_eager = dict(kern)
        kern = {"step": t["mean_ms"] / w.launches_per_step()}
    ab = w.algorithmic_bytes()
    dominant = max((k for k in ("build", "apply", "step", "conv") if k in kern), key=lambda k: kern[k])
    dur_s = kern[dominant] * 1e-3
    achieved = ab["per_launch"][dominant] / dur_s / 1e9
    kernel_full = {k["slot"]: k["name"] for k in plan["kernels"]}[dominant]
    stream_tag = w.name == "c4" or (w.stream_mode and w.name in ("c3", "c5"))
    tag = w.name + ("_" + w.mode if stream_tag else "") + ("_fp8" if w.cfg.dtype == "fp8" else "")
    ms = t["mean_ms"]
    path_gbps = ab["path"] / (ms * 1e-3) / 1e9
    mf = load_mfma(tag, kernel_full)
    return {
        "settle_steps": settled, "ms_per_step": ms, "value": w.tokens_heads / (ms * 1e-3),
        "timing": {k: t[k] for k in ("median_ms", "p10_ms", "p90_ms")},
        "roofline": {"bound": "hbm", "kernel": kernel_full, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": load_traffic(tag, kernel_full),
                     "algorithmic_bytes_per_launch": ab["per_launch"][dominant],
                     "avg_launch_ms": kern[dominant]},
        "path": {"algorithmic_bytes_per_step": ab["path"], "achieved_GBps": path_gbps,
                 "frac_of_peak": path_gbps / HBM_PEAK_GBPS,
                 "kernel_ms_per_launch": kern, "launches_per_step": w.launches_per_step(),
                 "plan": plan},
        "eager_event_ms_per_launch": kern_eager,
        "mfma": mf,
        "counter_tag": tag,
    }


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


def summarize_counters(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, tag):
    fetch = _per_kernel(_pmc_rows(fetch_dir), "FETCH_SIZE")
    write = _per_kernel(_pmc_rows(write_dir), "WRITE_SIZE")
    cf = _per_kernel(_pmc_rows(copy_fetch_dir), "FETCH_SIZE")
    cw = _per_kernel(_pmc_rows(copy_write_dir), "WRITE_SIZE")
    # the calibration run's copy kernel: the one with the largest fetch
    copy_name = max(cf, key=cf.get)
    f_factor = COPY_BYTES / (cf[copy_name] * 1024.0)
    w_factor = COPY_BYTES / (cw[copy_name] * 1024.0)
    out = {"source_sha256": source_hash(), "tag": tag,
           "copy_kernel": copy_name, "copy_bytes": COPY_BYTES,
           "fetch_factor": f_factor, "write_factor": w_factor, "kernels": {}}
    for k in sorted(set(fetch) | set(write)):
        if "svla" not in k:
            continue
        fb = fetch.get(k, 0.0) * 1024.0 * f_factor
        wb = write.get(k, 0.0) * 1024.0 * w_factor
        out["kernels"][k] = {"fetch_kib": fetch.get(k), "write_kib": write.get(k),
                             "hbm_bytes_per_dispatch": fb + wb}
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % tag)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def summarize_mfma(mdir, tag):
    """Matrix-core and vector-ALU use per dispatch from one rocprofv3 --pmc
    pass of MFMA_COUNTERS: MFMA busy percent of the SIMD cycles, bf16 MFMA
    flops, VALU busy percent, and the dispatch's GPU-active cycles."""
    rows = _pmc_rows(mdir)
    vals = {c: _per_kernel(rows, c) for c in MFMA_COUNTERS}
    out = {"source_sha256": source_hash(), "tag": tag, "counters": list(MFMA_COUNTERS),
           "kernels": {}}
    for k in sorted(vals["GRBM_GUI_ACTIVE"]):
        if "svla" not in k:
            continue
        ent = {c: vals[c].get(k) for c in MFMA_COUNTERS}
        ent["mfma_busy_frac"] = None if ent["MfmaUtil"] is None else ent["MfmaUtil"] / 100.0
        ent["valu_busy_frac"] = None if ent["VALUBusy"] is None else ent["VALUBusy"] / 100.0
        out["kernels"][k] = ent
    path = os.path.join(ROOT, "profiles", "mfma_%s.json" % tag)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


# profile summaries: tag -> (kernel table file, workload title, bench options)
PROFILE_TAGS = {
    "c4_stream": ("kernels_c4_minute_rope_stream.md", "c4 minute-long streaming (80 one-launch block steps of B1 H70 1170 tokens d32, bf16, RoPE, HIP graph)", "--config c4 --c4-mode stream"),
    "c4_oneshot": ("kernels_c4_minute_rope_oneshot.md", "c4 minute-long one shot (B1 H70, 80 blocks x 1170 tokens d32, bf16, RoPE)", "--config c4 --c4-mode oneshot"),
    "c3": ("kernels_c3_720p_block_causal.md", "c3 720p block-causal (B1 H70, 7 blocks x 2640 tokens d32, bf16)", "--config c3"),
    "c3_stream": ("kernels_c3_720p_block_steps.md", "c3 720p as 7 block steps (B1 H70, 2640 tokens d32, bf16, one-launch step, HIP graph)", "--config c3 --stream"),
    "c3_bwd": ("kernels_c3_720p_backward.md", "c3 720p backward (B1 H70, 7 blocks x 2640 tokens d32, bf16 in and out)", "--config c3 --backward"),
    "c2": ("kernels_c2_480p_noncausal.md", "c2 480p non-causal (B2 H70, 8190 tokens d32, bf16)", "--config c2"),
    "c5": ("kernels_c5_gated_d128.md", "c5 2.0-style gated (B1 H20, 8 blocks x 1760 tokens d128, bf16)", "--config c5"),
    "c5_stream": ("kernels_c5_gated_d128_stream.md", "c5 2.0-style gated as 8 block steps (B1 H20, 1760 tokens d128, bf16, gate per step, HIP graph)", "--config c5 --stream"),
    "t3": ("kernels_t3_720p_temporal_conv.md", "t3 720p temporal convolution (B1, 7 blocks x 3 frames, 22x40 positions, 2240 channels, bf16)", "--config t3"),
    "t4": ("kernels_t4_minute_temporal_conv_stream.md", "t4 minute-long temporal convolution (80 block steps of 3 frames, 15x26 positions, 2240 channels, bf16, cache carried)", "--config t4"),
    "c4_stream_fp8": ("kernels_c4_minute_rope_stream_fp8.md", "c4 minute-long streaming with fp8 (E4M3) Q, K, V (80 one-launch block steps, bf16 O, RoPE, HIP graph)", "--config c4 --c4-mode stream --dtype fp8"),
    "c3_fp8": ("kernels_c3_720p_block_causal_fp8.md", "c3 720p block-causal with fp8 (E4M3) Q, K, V (bf16 O)", "--config c3 --dtype fp8"),
}


def summarize_kernels(stats_csv, tag):
    """profiles/kernels_<workload>.md from a rocprofv3 --kernel-trace --stats
    kernel_stats.csv of `python bench.py <options of tag> --steps 5 --warmup 2
    --no-cpu-baseline`: the six kernels with the most GPU time."""
    fn, title, opts = PROFILE_TAGS[tag]
    rows = list(csv.DictReader(open(stats_csv)))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0

    def short(n):
        n = n.replace("(anonymous namespace)::", "")
        return n if len(n) <= 90 else n[:87] + "..."
    out = ["# rocprofv3 kernel statistics: " + title, "",
           "Library source sha256 prefix: `%s` (block_causal_linear_relu_amd/csrc/svla.hip)." % source_hash(), "",
           "Command (run from the repository root; `<out>` is a scratch directory), then this table with "
           "`python bench.py --summarize-kernels <out>/kt_kernel_stats.csv --tag %s`:" % tag, "", "```",
           "rocprofv3 --kernel-trace --stats -d <out> -o kt --output-format csv -- python -u bench.py %s "
           "--steps 5 --warmup 2 --no-cpu-baseline" % opts, "```", "",
           "The bench process also runs its clock-settling steps, the warm-up steps, the per-kernel event "
           "loop and the input set-up copies; every libsvla kernel of every step is listed.", "",
           "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows[:6]:
        out.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f%% |" % (
            short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, 100 * float(r["TotalDurationNs"]) / tot))
    with open(os.path.join(ROOT, "profiles", fn), "w") as fh:
        fh.write("\n".join(out) + "\n")


def summarize_tables():
    """profiles/hbm_traffic_counters.md and profiles/mfma_utilisation.md from
    the counter summaries of the current source (counters_<tag>.json,
    mfma_<tag>.json); a summary of other kernels is left out."""
    h = source_hash()
    fetch_f = write_f = None
    traffic = ["| tag | bench option | kernel | fetch (KiB) | write (KiB) | HBM bytes per launch |",
               "|---|---|---|---|---|---|"]
    mfma = ["| tag | kernel | MfmaUtil (%) | VALUBusy (%) | bf16 MFMA flops per launch |", "|---|---|---|---|---|"]
    for tag, (_, _, opts) in PROFILE_TAGS.items():
        c = _load_summary("counters", tag)
        if c is not None:
            fetch_f, write_f = c["fetch_factor"], c["write_factor"]
            for k, v in c["kernels"].items():
                traffic.append("| %s | `%s` | `%s` | %.0f | %.0f | %.2f MB |" % (
                    tag, opts, k, v["fetch_kib"] or 0, v["write_kib"] or 0, v["hbm_bytes_per_dispatch"] / 1e6))
        m = _load_summary("mfma", tag)
        if m is not None:
            for k, v in m["kernels"].items():
                mfma.append("| %s | `%s` | %.1f | %.1f | %.3g |" % (
                    tag, k, v["MfmaUtil"] or 0, v["VALUBusy"] or 0, v["MfmaFlopsBF16"] or 0))
    pmc = "--steps 2 --warmup 1 --settle 0 --no-cpu-baseline"
    t = ["# HBM traffic per kernel launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
         "Each counter was collected in a run of its own (run from the repository root; `<out>` is a "
         "scratch directory; `<args>` is the workload's bench option in the table below):", "", "```",
         "rocprofv3 --pmc FETCH_SIZE -d <out>/<tag>/f -o f --output-format csv -- python -u bench.py <args> " + pmc,
         "rocprofv3 --pmc WRITE_SIZE -d <out>/<tag>/w -o w --output-format csv -- python -u bench.py <args> " + pmc,
         "rocprofv3 --pmc FETCH_SIZE -d <out>/copy/f -o f --output-format csv -- python -u bench.py --copy-calibration",
         "rocprofv3 --pmc WRITE_SIZE -d <out>/copy/w -o w --output-format csv -- python -u bench.py --copy-calibration",
         "python bench.py --summarize-counters <out>/<tag>/f <out>/<tag>/w <out>/copy/f <out>/copy/w --tag <tag>",
         "python bench.py --summarize-tables", "```", ""]
    if fetch_f is not None:
        t += ["Calibration: a plain device copy of 512 MiB (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = "
              "%.3f x and WRITE_SIZE = %.3f x its size in KiB, so fetch KiB x 1024 x %.3f and write KiB x "
              "1024 x %.3f are bytes." % (1 / fetch_f, 1 / write_f, fetch_f, write_f), ""]
    t += ["Library source sha256 prefix: `%s`." % h, ""] + traffic
    mm = ["# Matrix-core and vector-ALU utilisation per kernel (rocprofv3 derived counters)", "",
          "One `--pmc` pass per workload (run from the repository root):", "", "```",
          "rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 VALUBusy GRBM_GUI_ACTIVE -d <out>/<tag>/m -o m "
          "--output-format csv -- python -u bench.py <args> " + pmc,
          "python bench.py --summarize-mfma <out>/<tag>/m --tag <tag>", "python bench.py --summarize-tables", "```", "",
          "MfmaUtil = 100 x sum SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs): the share of the "
          "kernel's time the matrix cores were busy. MfmaFlopsBF16 = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 per "
          "dispatch (bf16 matrix flops, the backward's bf16 hi + lo products included; fp32 products are not "
          "counted there). VALUBusy: the share of time the vector ALUs issued.", "",
          "Library source sha256 prefix: `%s`." % h, ""] + mfma
    with open(os.path.join(ROOT, "profiles", "hbm_traffic_counters.md"), "w") as fh:
        fh.write("\n".join(t) + "\n")
    with open(os.path.join(ROOT, "profiles", "mfma_utilisation.md"), "w") as fh:
        fh.write("\n".join(mm) + "\n")


def copy_calibration():
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "dispatches": 3}))


def ceiling(reps: int = 20):
    """Achievable HBM rates on this GPU, from the library's bandwidth probes
    (svla_hbm_probe: 16-byte non-temporal buffer loads, 2048 workgroups each
    streaming one contiguous MiB): a read of 2 GiB and a copy of 2 GiB (reads +
    writes), each the median of `reps` event-timed runs over four rotating
    buffers (8 GiB, far past the 256 MB Infinity Cache)."""
    import ctypes
    import torch
    import block_causal_linear_relu_amd as svla
    lib = svla.library()
    nbytes, wgs = 2 << 30, 2048
    src = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda:0") for _ in range(4)]
    dst = [torch.empty_like(s) for s in src]
    sink = torch.zeros(wgs, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def probe(mode, i):
        st = lib.svla_hbm_probe(mode, ctypes.c_void_p(src[i % 4].data_ptr()),
                                ctypes.c_void_p(dst[i % 4].data_ptr()), nbytes,
                                ctypes.c_void_p(sink.data_ptr()), wgs, stream)
        if st != 0:
            raise RuntimeError("svla_hbm_probe failed: %d" % st)

    def med(fn):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        ts = []
        for i in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(i)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return _pct(ts, 50)

    t_read = med(lambda i: probe(0, i))
    t_copy = med(lambda i: probe(1, i))
    t_torch = med(lambda i: dst[i % 4].copy_(src[i % 4]))
    res = {"read_GBps": nbytes / (t_read * 1e-3) / 1e9, "copy_GBps": 2 * nbytes / (t_copy * 1e-3) / 1e9,
           "torch_copy_GBps": 2 * nbytes / (t_torch * 1e-3) / 1e9,
           "read_ms": t_read, "copy_ms": t_copy, "bytes": nbytes, "peak_GBps": HBM_PEAK_GBPS}
    res["read_frac"] = res["read_GBps"] / HBM_PEAK_GBPS
    res["copy_frac"] = res["copy_GBps"] / HBM_PEAK_GBPS
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, tag=args.tag or args.config)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, tag=args.tag or args.config)
        return
    if args.summarize_kernels:
        summarize_kernels(args.summarize_kernels, args.tag)
        return
    if args.summarize_tables:
        summarize_tables()
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
    if args.ceiling:
        ceiling()
        return

    if args.anchor:
        aw = AnchorWorkload("c5" if args.config == "c4" else args.config, args.rotate)
        settled = settle(aw, args.settle) if args.settle > 0 else 0
        t = time_steps(aw, args.steps, args.warmup)
        ms = t["mean_ms"]
        tf = aw.flops() / (ms * 1e-3) / 1e12
        line = {"metric": ANCHOR_METRIC, "value": aw.tokens_heads / (ms * 1e-3), "unit": UNIT, "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "settle_steps": settled, "ms_per_step": ms,
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded N(0,1) Q, K, V, bf16-rounded)", "config": aw.describe(),
                "timing": {k: t[k] for k in ("median_ms", "p10_ms", "p90_ms")},
                "roofline": {"bound": "mfma", "kernel": "void svla_softmax_fwd<%d>" % aw.d, "achieved": tf,
                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_MFMA_PEAK_TFLOPS,
                             "traffic": None, "algorithmic_flops_per_launch": aw.flops(),
                             "avg_launch_ms": ms, "hbm_GBps": aw.bytes() / (ms * 1e-3) / 1e9},
                "source": "block_causal_linear_relu_amd/csrc/svla_softmax.hip",
                "cpu_baseline": None if args.no_cpu_baseline else anchor_cpu_baseline(aw)}
        print(json.dumps(line), flush=True)
        return
    if args.backward:
        if args.config not in ("c3", "c2") or args.dtype != "bf16":
            print("bench.py: --backward times the bf16 d = 32 training shapes (c3, c2)", file=sys.stderr)
            sys.exit(2)
        bw = BackwardWorkload(args.config, args.rotate)
        m = measure_backward(bw, args, args.settle)
        line = {"metric": BWD_METRIC, "value": m["value"], "unit": UNIT, "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "settle_steps": m["settle_steps"],
                "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16 (fp32 arithmetic)",
                "data": "synthetic (seeded N(0,1) Q, K, V, dO, bf16-rounded)",
                "config": bw.describe(), "timing": m["timing"], "roofline": m["roofline"],
                "kernels": m["kernels"], "path": m["path"], "mfma": m["mfma"],
                "source_sha256": source_hash(),
                "cpu_baseline": None if args.no_cpu_baseline else backward_cpu_baseline(bw)}
        print(json.dumps(line), flush=True)
        return
    if args.config.startswith("t"):
        cw = ConvWorkload(args.config, args.rotate)
        m = measure(cw, args, args.settle)
        line = {"metric": CONV_METRIC, "value": m["value"], "unit": CONV_UNIT, "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "settle_steps": m["settle_steps"],
                "ms_per_step": m["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "bf16",
                "data": "synthetic (seeded N(0,1), bf16-rounded; random fp32 taps and bias)",
                "config": cw.describe(), "timing": m["timing"], "roofline": m["roofline"],
                "path": m["path"], "source_sha256": source_hash(),
                "cpu_baseline": None if args.no_cpu_baseline else conv_cpu_baseline(cw)}
        print(json.dumps(line), flush=True)
        return
    from workloads import CONFIGS, make_inputs, scaled_config
    if args.dtype == "fp8" and CONFIGS[args.config].d != 32:
        print("bench.py: fp8 inputs are for the d = 32 workloads", file=sys.stderr)
        sys.exit(2)
    if args.stream and args.config not in ("c3", "c5"):
        print("bench.py: --stream is for c3 and c5 (c4 takes --c4-mode; c2 is one block)",
              file=sys.stderr)
        sys.exit(2)
    x = make_inputs(scaled_config(CONFIGS[args.config], dtype=args.dtype))
    c4 = args.config == "c4"
    stream_mode = "stream_inplace" if args.inplace else "stream"
    primary = stream_mode if ((c4 and args.c4_mode in ("both", "stream")) or
                              (args.stream and args.config in ("c3", "c5"))) else "oneshot"
    w = Workload(args.config, args.rotate, primary, x=x, dtype=args.dtype)
    m = measure(w, args, args.settle)
    line = {
        "metric": METRIC,
        "value": m["value"],
        "unit": UNIT,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": m["settle_steps"],
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic (seeded N(0,1), %s-rounded; shapes of the pages' video workloads)"
                % ("OCP-E4M3" if args.dtype == "fp8" else "bf16"),
        "config": w.describe(),
        "timing": m["timing"],
        "roofline": m["roofline"],
        "path": m["path"],
        "mfma": m["mfma"],
        "source_sha256": source_hash(),
    }
    if m["eager_event_ms_per_launch"]:
        line["path"]["eager_event_ms_per_launch"] = m["eager_event_ms_per_launch"]
    if c4 and args.c4_mode == "both":
        del w
        torch.cuda.empty_cache()
        w1 = Workload(args.config, args.rotate, "oneshot", x=x, dtype=args.dtype)
        m1 = measure(w1, args, 0.1)
        line["c4_oneshot"] = {k: m1[k] for k in ("value", "ms_per_step", "timing", "roofline",
                                                 "path", "mfma")}
        line["c4_oneshot"]["config"] = w1.describe()
        w = w1
    if c4 or args.config == "c3":
        fr = {"stream": line["path"]["frac_of_peak"]} if primary != "oneshot" else {}
        if "c4_oneshot" in line:
            fr["oneshot"] = line["c4_oneshot"]["path"]["frac_of_peak"]
        elif primary == "oneshot":
            fr["oneshot"] = line["path"]["frac_of_peak"]
        carried = "stream" if fr.get("stream", 0.0) >= GATE_FRAC else "oneshot" if "oneshot" in fr else "stream"
        line["gate"] = {"target_frac_of_peak": GATE_FRAC, "path_frac": fr, "carried_by": carried,
                        "met": fr.get(carried, 0.0) >= GATE_FRAC}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, single_thread=args.config == "c3")
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
