#!/usr/bin/env python3
"""Benchmark of the batch-size-1 MoE decode-step weight stream on one MI355X.

One step = 42 independent full-shape MoE layers (router over 512 experts, top-8 + shared expert,
MXFP4 gate_up/down with SwiGLU, hidden 2560, intermediate 768; each layer with its own seeded
weights and its own seeded token vector) run in stream order, followed by the FP8 LM head
(157,184 x 2,560), at M = 1 token. Inputs are resident in HBM before timing starts. The value is
whole-step algorithmic bytes / step time.

The 42 layers of a step run as ONE persistent launch (moe_layers_mxfp4: each layer's router,
top-K, experts and combine inside one grid; no x-dependent work of layer l+1 starts before layer
l's output is written); the FP8 head follows on the same stream. HIP events bracket both
launches in every timed step, which gives the live per-launch durations for the roofline entry.
(Feeding layer l's output to layer l+1 instead is not used: without the attention block's
residual and normalisation, seeded random SwiGLU layers grow the activations by orders of
magnitude per layer, and within a few layers they overflow.)

Also reported (in "breakdown"): one layer cold-cache at M = 1 (natural and Zipf-concentrated
routing), the three M = 4 verification regimes and their cost ratio over M = 1, the FP8 and bf16
heads cold-cache, the decode step at M = 4, the device's streaming-read ceiling, and FP8-vs-bf16
head top-1/top-10 agreement.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
N_LAYERS = 42
K_TOP = 8


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--layers", type=int, default=N_LAYERS, help="MoE layers per step (42 for the real step)")
    p.add_argument("--no-breakdown", action="store_true", help="skip the per-configuration breakdown")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--agreement", type=int, default=1000, help="x vectors for FP8-vs-bf16 head agreement")
    p.add_argument("--profile", action="store_true",
                   help="a short fixed sequence for hardware-counter runs (rocprofv3 --pmc): per kernel two "
                        "launches, in this order: copy probe, 42-layer launch at M=1, FP8 head M=1, bf16 head "
                        "M=1, one cold layer at M=1, 42-layer launch at M=4, FP8 head verification M=4; no JSON")
    return p.parse_args()


# ------------------------------------------------------------------------------------ bytes
def expert_bytes(H=2560, I=768):
    return 2 * I * (H // 2 + H // 32) + H * (I // 2 + I // 32)


def layer_bytes(union, M, E=512, H=2560, I=768, shared=1):
    """Algorithmic bytes of one MoE layer: router rows, the union's experts + shared, x and y (bf16)."""
    return E * H * 2 + (union + shared) * expert_bytes(H, I) + 2 * M * H * 2


def head_bytes(M, V=157184, H=2560, fp8=True):
    w = V * H + V * 4 if fp8 else V * H * 2
    return w + M * H * 2 + M * V * 4


# ------------------------------------------------------------------------------------ helpers
def _bf16(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class Flusher:
    """Evicts L2 and the Infinity Cache between timed iterations by streaming a 1 GiB buffer
    through the read probe (a read flush leaves no dirty lines to write back during the next
    measured launch)."""

    def __init__(self, qws, dev):
        import torch
        self.qws = qws
        self.buf = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        self.sink = torch.empty(4096, dtype=torch.int32, device=dev)

    def __call__(self):
        self.qws.probe_read(self.buf, self.sink, 4096)


def time_cold(fn, dev, iters=100, warm=10, flush=None):
    """Median / p10 / p90 microseconds of fn() between HIP events, flushing caches before each
    (outside the event pair): 10 warm-up calls, then 100 timed."""
    import torch
    for _ in range(warm):
        fn()
    ts = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        if flush:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize(dev)
    ts = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    return {"median_us": ts[len(ts) // 2], "p10_us": ts[len(ts) // 10], "p90_us": ts[(9 * len(ts)) // 10]}


class MoeLayer:
    """Device-resident inputs and outputs of one MoE layer, runnable through the fused one-launch
    entry point or through the two-call path (router kernel, then the expert kernels)."""

    def __init__(self, qws, seed, layer, M, dev, bias=None, bank=None, packed=None, x=None, keep_canonical=True,
                 n_routed=512):
        import torch
        import synth
        shape = synth.LayerShape(n_routed=n_routed)
        self.E = n_routed
        # canonical bank: the two-call path; task-major copy: the fused path. Layers that only run
        # fused drop the canonical bank once packed (a 42-layer step then holds ~70 GB, not ~137)
        self.bank_t = bank
        if self.bank_t is None and (packed is None or keep_canonical):
            self.bank_t = synth.expert_bank_torch(seed, layer, shape, device=dev)
        self.bank = None if self.bank_t is None else qws.ExpertBank.from_dict(self.bank_t, shape.n_routed, True)
        self.packed = packed if packed is not None else qws.moe_pack_mxfp4(self.bank)
        if not keep_canonical:
            self.bank_t, self.bank = None, None
        self.wr = _bf16(synth.router_weights(seed, layer, shape.n_routed), dev)
        self.x = x if x is not None else _bf16(synth.token_vectors(seed, layer, M), dev)
        self.bias = None if bias is None else torch.from_numpy(bias).to(dev)
        self.fused = qws.MoeLayer(self.x, self.wr, self.packed, K_TOP, bias=self.bias, want_f32=False)
        self.idx, self.w, self.y = self.fused.topk_idx, self.fused.topk_w, self.fused.y_bf16
        self.M = M
        self.qws = qws

    def run(self, ws):
        self.qws.moe_layer_mxfp4(self.fused, workspace=ws)

    def run_two_call(self, ws_route, ws_exp):
        q = self.qws
        q.moe_route_topk(self.x, self.wr, K_TOP, self.bias, topk_idx=self.idx, topk_w=self.w, workspace=ws_route)
        q.moe_expert_gemv_mxfp4(self.bank, self.x, self.idx, self.w, y_bf16=self.y, workspace=ws_exp, want_f32=False)

    def union(self):
        return len({int(e) for e in self.idx.cpu().reshape(-1).tolist()})


def probe_ceiling(qws, dev, probe="probe_read"):
    """Best read rate over a few grid sizes for 4 GiB: `probe_read` (ordinary grid-strided loads)
    or `probe_read_nt` (non-temporal loads, one contiguous share per workgroup)."""
    import torch
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    fn = getattr(qws, probe)
    best = {}
    for blocks in (1024, 2048, 4096, 8192):
        r = time_cold(lambda: fn(buf, sink, blocks), dev, iters=10, warm=2)
        best[blocks] = buf.numel() / (r["median_us"] * 1e-6) / 1e9
    del buf
    b = max(best, key=best.get)
    return {"GBps": round(best[b], 1), "blocks": b, "bytes": 4 << 30}


# ------------------------------------------------------------------------------------ decode step
def speculation_model(t1_ms, t4_ms, draft_step_ms, drafts=3, accepts=(1.0, 2.68, 3.90, 4.0)):
    """Decode throughput of speculative decoding priced from measured step times (the pages report
    accept length and verification-cost ratio so that readers can price the trade: runbyai.xyz
    signal/190 on the four-position window, Netics post on the 3.90 / 2.68 accept lengths). A round
    drafts `drafts` tokens (each a draft step at M = 1) and verifies drafts + 1 positions in one
    step of cost t4; it emits `accept` tokens on average. Plain decoding emits one token per t1."""
    round_ms = t4_ms + drafts * draft_step_ms
    return {"t_decode_ms": round(t1_ms, 4), "t_verify_ms": round(t4_ms, 4),
            "verify_cost_ratio": round(t4_ms / t1_ms, 3), "draft_step_ms": round(draft_step_ms, 4),
            "round_ms": round(round_ms, 4), "break_even_accept": round(round_ms / t1_ms, 3),
            "plain_tokens_per_s": round(1e3 / t1_ms, 1),
            "by_accept": {f"{a:.2f}": {"tokens_per_s": round(a * 1e3 / round_ms, 1),
                                       "speedup": round(a * t1_ms / round_ms, 3)} for a in accepts}}


class DecodeStep:
    """42 independent MoE layers in one persistent launch (moe_layers_mxfp4), then the FP8 head
    (at M > 1 with the greedy verification epilogue: a verification round's target pass)."""

    def __init__(self, qws, M, dev, n_layers, head, packed=None):
        import torch
        import synth
        self.qws, self.M, self.dev = qws, M, dev
        self.w4a8 = False   # True: the layers run moe_layers_w4a8 (MXFP8 activations)
        log(f"building {n_layers} layers (M={M})")
        self.layers = []
        for l in range(n_layers):
            self.layers.append(MoeLayer(qws, 0, l, M, dev, packed=None if packed is None else packed[l],
                                        keep_canonical=False))
        self.seq = qws.MoeLayers([L.fused for L in self.layers])
        self.ws = qws.moe_layer_workspace(M, K_TOP, 512, 2560, 768, dev)
        self.xh = _bf16(synth.token_vectors(0, 1000, M), dev)
        self.head = head
        self.logits = torch.empty((M, head.rows), dtype=torch.float32, device=dev)
        if M > 1:
            self.vws = qws.verify_workspace(M, dev)
            self.draft = torch.arange(1, M, dtype=torch.int32, device=dev)
            self.vout = qws.lmhead_verify_greedy_fp8(head, self.xh, self.draft, self.vws, logits=self.logits)

    def layers_call(self):
        self.seq.run(self.ws, w4a8=self.w4a8)

    def head_call(self):
        if self.M == 1:
            self.qws.lmhead_gemv_fp8(self.head, self.xh, out=self.logits)
        else:
            self.qws.lmhead_verify_greedy_fp8(self.head, self.xh, self.draft, self.vws, logits=self.logits,
                                              out=self.vout)

    def bytes(self):
        return sum(layer_bytes(L.union(), self.M) for L in self.layers) + head_bytes(self.M)

    def errors(self):
        return self.qws.moe_workspace_errors(self.ws, self.M, K_TOP, 512, 768)

    def timed(self, steps, warmup):
        import torch
        for _ in range(warmup):
            self.layers_call()
            self.head_call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        torch.cuda.synchronize(self.dev)
        t0 = time.perf_counter()
        for a, b, c in ev:
            a.record()
            self.layers_call()
            b.record()
            self.head_call()
            c.record()
        torch.cuda.synchronize(self.dev)
        wall = (time.perf_counter() - t0) / steps
        moe_us = sorted(a.elapsed_time(b) * 1e3 for a, b, _ in ev)
        head_us = sorted(b.elapsed_time(c) * 1e3 for _, b, c in ev)
        gpu_ms = sum(a.elapsed_time(c) for a, _, c in ev) / steps
        return {"wall_ms": wall * 1e3, "gpu_ms": gpu_ms, "moe_us_mean": sum(moe_us) / len(moe_us),
                "head_us_mean": sum(head_us) / len(head_us), "head_us_median": head_us[len(head_us) // 2]}

    def timed_flushed(self, steps, flush):
        """The same step with the caches flushed before each one, outside its event pair: no byte
        of the step (router rows, experts, head) can be served from the L2 or the Infinity Cache
        left warm by the previous step."""
        import torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for a, b, c in ev:
            flush()
            a.record()
            self.layers_call()
            b.record()
            self.head_call()
            c.record()
        torch.cuda.synchronize(self.dev)
        step_ms = sorted(a.elapsed_time(c) for a, _, c in ev)
        moe_us = sorted(a.elapsed_time(b) * 1e3 for a, b, _ in ev)
        return {"step_ms_median": step_ms[len(step_ms) // 2], "moe_us_median": moe_us[len(moe_us) // 2]}


# ------------------------------------------------------------------------------------ traffic
def source_sha256(kernel_src) -> str:
    """sha256 of a kernel's source file, or of several concatenated in the order given."""
    h = hashlib.sha256()
    for f in ([kernel_src] if isinstance(kernel_src, str) else kernel_src):
        h.update(open(os.path.join(ROOT, "quantized_weight_streaming_amd", "csrc", f), "rb").read())
    return h.hexdigest()


# the fused MoE kernel: its device code and the host file that packs the records it reads
MOE_SRC = ("moe_fused_kernel.hpp", "moe_fused.hip")


def traffic_for(kernel_src, name: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, if it was
    taken on the current source of the kernel (else None)."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    sha = source_sha256(kernel_src)
    if kv.get("source_sha256") != sha:
        return None
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------------------------ CPU baseline
def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(step_bytes_m1, n_layer_sample=2, head_rows=8192, repeats=3):
    """The oracle as it stands, on a bounded sample of the M = 1 step (n_layer_sample MoE layers and
    head_rows FP8 head rows), extrapolated to one step: the median of `repeats` runs with all the
    cores this process may use, and the same sample on one thread. Input generation is excluded."""
    import numpy as np
    import synth
    from oracle import lmhead as OL
    from oracle import moe as OM
    from threadpoolctl import threadpool_info, threadpool_limits
    cores = len(os.sched_getaffinity(0))
    shape = synth.LayerShape()
    layers = []
    for l in range(n_layer_sample):
        x = synth.token_vectors(0, l, 1)
        wr = synth.router_weights(0, l, 512)
        idx0, _, _ = OM.route(x, wr, 8)
        experts = {e: synth.expert_np(0, l, e, shape) for e in set(idx0.reshape(-1).tolist()) | {512}}
        layers.append((x, wr, experts))
    wh = synth.head_chunk(0, 0, head_rows)
    codes, scales = OL.fp8_rowquant(wh)
    xh = synth.token_vectors(0, 1000, 1)

    def one_step_s():
        t_layers = []
        for x, wr, experts in layers:
            t0 = time.perf_counter()
            idx, w, _ = OM.route(x, wr, 8)
            OM.moe_layer(x, idx, w, experts, 512)
            t_layers.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        OL.lmhead_fp8(codes, scales, xh)
        t_head = time.perf_counter() - t0
        return N_LAYERS * (sum(t_layers) / len(t_layers)) + (157184 / head_rows) * t_head

    with threadpool_limits(limits=cores):
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        runs = sorted(one_step_s() for _ in range(repeats))
    with threadpool_limits(limits=1):
        one = one_step_s()
    t_step = runs[len(runs) // 2]
    return {"value": round(step_bytes_m1 / t_step / 1e9, 3), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "step_s": round(t_step, 3), "step_s_runs": [round(r, 3) for r in runs],
            "value_1_thread": round(step_bytes_m1 / one / 1e9, 3), "step_s_1_thread": round(one, 3),
            "cpu_model": _cpu_model(), "numpy": np.__version__, "blas_threads": int(blas),
            "sample": f"numpy fp64 oracle on {n_layer_sample} of the 42 MoE layers (route + dequantise the activated "
                      f"experts + SwiGLU + combine) and {head_rows} of 157,184 FP8 head rows at M=1, extrapolated to "
                      f"one step; median of {repeats} runs on the process's {cores} cores (BLAS threads {blas}; "
                      "elementwise numpy runs on one thread), and one run on one thread; input generation excluded"}


def profile_sequence(qws, dev, n_layers):
    """Two launches of each kernel whose HBM traffic the counters measure, in a fixed order, with the
    caches flushed before each launch (the counter summaries under profiles/ name the dispatches by
    this order)."""
    import torch
    import synth
    flush = Flusher(qws, dev)
    cp_src = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    wh_t = _bf16(synth.head_weights(0), dev)
    head_bf16 = qws.lmhead_bf16(wh_t)
    head8 = qws.lmhead_quantize_fp8(wh_t)
    step = DecodeStep(qws, 1, dev, n_layers, head8)
    step4 = DecodeStep(qws, 4, dev, n_layers, head8, packed=[L.packed for L in step.layers])
    one = qws.MoeLayers([step.layers[0].fused])
    ws1 = qws.moe_layer_workspace(1, K_TOP, 512, 2560, 768, dev)
    seq = [("probe_copy", lambda: qws.probe_copy(cp_src, cp_dst, 4096)),
           ("moe_layers_m1", step.layers_call),
           ("head_fp8_m1", lambda: qws.lmhead_gemv_fp8(head8, step.xh, out=step.logits)),
           ("head_bf16_m1", lambda: qws.lmhead_gemv_bf16(head_bf16, step.xh, out=step.logits)),
           ("moe_layer_m1_single", lambda: one.run(ws1)),
           ("moe_layers_m4", step4.layers_call),
           ("verify_greedy_m4", step4.head_call)]
    for name, fn in seq:
        for _ in range(2):
            flush()
            torch.cuda.synchronize(dev)
            fn()
            torch.cuda.synchronize(dev)
        log("profile", name, "done")
    print("profile sequence:", ", ".join(f"{n} x2" for n, _ in seq), flush=True)


# ------------------------------------------------------------------------------------ main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): this benchmark "
              "measures the single-GPU decode step; there is no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_weight_streaming_amd as qws
    import synth

    dev = torch.device("cuda:0")
    qws.lib()
    qws.selfcheck(dev)
    log("selfcheck ok")
    if args.profile:
        profile_sequence(qws, dev, args.layers)
        return

    # LM head: bf16 weights generated on the host, quantised online to FP8 on the device (one-off)
    t0 = time.perf_counter()
    wh = synth.head_weights(0)
    wh_t = _bf16(wh, dev)
    log(f"head generated in {time.perf_counter() - t0:.1f}s")
    head_bf16 = qws.lmhead_bf16(wh_t)
    head8 = qws.lmhead_quantize_fp8(wh_t)
    flush = Flusher(qws, dev)
    quant_us = time_cold(lambda: qws.lmhead_quantize_fp8(wh_t, codes=head8.w, row_scale=head8.row_scale), dev,
                         iters=5, warm=1, flush=flush)["median_us"]

    step = DecodeStep(qws, 1, dev, args.layers, head8)
    step.layers_call()
    torch.cuda.synchronize(dev)
    sb = step.bytes()
    log(f"decode step M=1: {args.layers} layers, {sb / 1e9:.3f} GB per step; timing {args.steps} steps")
    r = step.timed(args.steps, args.warmup)
    value = sb / (r["wall_ms"] * 1e-3) / 1e9
    # the dominant kernel of the step is the 42-layer MoE launch; the FP8 head follows in "breakdown"
    moe_bytes = sb - head_bytes(1)
    moe_gbs = moe_bytes / (r["moe_us_mean"] * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": f"qws_moe::moe_layers_kernel<1, false, false> ({args.layers} MoE layers, one launch)",
                "achieved": round(moe_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(moe_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for(MOE_SRC, "moe_layers_kernel"),
                "algorithmic_bytes_per_launch": moe_bytes, "launch_us_mean": round(r["moe_us_mean"], 2)}
    head_launch_bytes = head_bytes(1)
    head_gbs = head_launch_bytes / (r["head_us_mean"] * 1e-6) / 1e9
    roofline_head = {"bound": "hbm", "kernel": "head_fp8_kernel<1, 0> (FP8 LM head GEMV, 157184x2560)",
                     "achieved": round(head_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(head_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_for("head_fp8.hpp", "head_fp8_kernel"),
                     "algorithmic_bytes_per_launch": head_launch_bytes, "launch_us_mean": round(r["head_us_mean"], 2)}

    breakdown = {"decode_step_m1": {"ms_wall": round(r["wall_ms"], 4), "ms_gpu_events": round(r["gpu_ms"], 4),
                                    "bytes": sb, "GBps": round(value, 1),
                                    "moe_layers_us": round(r["moe_us_mean"], 2),
                                    "moe_us_per_layer": round(r["moe_us_mean"] / args.layers, 3),
                                    "moe_layers_GBps": round(moe_bytes / (r["moe_us_mean"] * 1e-6) / 1e9, 1),
                                    "head_us_median": round(r["head_us_median"], 2),
                                    "unions": [L.union() for L in step.layers[:4]],
                                    "in_kernel_wait_timeouts": step.errors()},
                 "roofline_lmhead_fp8": roofline_head,
                 "lmhead_quantize_fp8_us": round(quant_us, 1)}

    # the same step with every cache flushed before each step (outside the events): nothing of one
    # step (router rows, experts, head) is left in the L2 or the Infinity Cache for the next
    rf = step.timed_flushed(args.steps, flush)
    breakdown["decode_step_m1_flushed"] = {"ms_median": round(rf["step_ms_median"], 4),
                                           "moe_us_per_layer": round(rf["moe_us_median"] / args.layers, 3),
                                           "GBps": round(sb / (rf["step_ms_median"] * 1e-3) / 1e9, 1),
                                           "back_to_back_ms": round(r["gpu_ms"], 4)}
    log("decode_step_m1_flushed", breakdown["decode_step_m1_flushed"])
    # the same step with MXFP8 activations in the MoE layers (W4A8)
    step.w4a8 = True
    rw8 = step.timed(args.steps, args.warmup)
    step.w4a8 = False
    breakdown["decode_step_m1_w4a8"] = {"ms_wall": round(rw8["wall_ms"], 4), "GBps": round(sb / (rw8["wall_ms"] * 1e-3) / 1e9, 1),
                                        "moe_us_per_layer": round(rw8["moe_us_mean"] / args.layers, 3),
                                        "bf16_activations_moe_us_per_layer": round(r["moe_us_mean"] / args.layers, 3),
                                        "in_kernel_wait_timeouts": step.errors()}
    log("decode_step_m1_w4a8", breakdown["decode_step_m1_w4a8"])

    if not args.no_breakdown:
        breakdown["probe_read_ceiling"] = probe_ceiling(qws, dev)
        log("probe", breakdown["probe_read_ceiling"])
        breakdown["probe_read_nt_ceiling"] = probe_ceiling(qws, dev, "probe_read_nt")
        log("probe nt", breakdown["probe_read_nt_ceiling"])
        wsf = {1: qws.moe_layer_workspace(1, K_TOP, 512, 2560, 768, dev),
               4: qws.moe_layer_workspace(4, K_TOP, 512, 2560, 768, dev)}
        wsr1 = qws.route_workspace(1, 512, dev)
        wse1 = qws.expert_workspace(1, K_TOP, 2560, 768, dev)
        lay = {}
        L0 = step.layers[0]
        lay["moe_layer_m1_seed0"] = MoeLayer(qws, 0, 0, 1, dev, packed=L0.packed)   # canonical again: two-call path
        bank1 = synth.expert_bank_torch(1, 0, synth.LayerShape(), device=dev)
        lay["moe_layer_m1_seed1_zipf"] = MoeLayer(qws, 1, 0, 1, dev, bias=synth.zipf_bias(1, 0, 512), bank=bank1)
        # the reduced layer: 64 routed experts + shared (one expert-parallel shard's bank at 8 GPUs)
        bank64 = synth.expert_bank_torch(0, 0, synth.LayerShape(n_routed=64), device=dev)
        lay["moe_layer_m1_e64"] = MoeLayer(qws, 0, 0, 1, dev, bank=bank64, keep_canonical=False, n_routed=64)
        for reg in synth.REGIMES:
            sets = synth.regime_sets(0, 0, reg, 4, 512)
            lay[f"moe_layer_m4_{reg}"] = MoeLayer(qws, 0, 0, 4, dev, bias=synth.regime_bias(sets, 512), packed=L0.packed,
                                                 keep_canonical=False)
        wsf64 = qws.moe_layer_workspace(1, K_TOP, 64, 2560, 768, dev)
        for name, Lr in lay.items():
            ws_ = wsf64 if Lr.E == 64 else wsf[Lr.M]
            t = time_cold(lambda: Lr.run(ws_), dev, flush=flush)
            u = Lr.union()
            b = layer_bytes(u, Lr.M, E=Lr.E)
            t.update({"union": u, "bytes": b, "GBps": round(b / (t["median_us"] * 1e-6) / 1e9, 1)})
            t["frac_of_peak"] = round(t["GBps"] / PEAK_HBM_GBS, 4)
            t["frac_of_nt_probe"] = round(t["GBps"] / breakdown["probe_read_nt_ceiling"]["GBps"], 4)
            if name == "moe_layer_m1_seed0":
                t["traffic"] = traffic_for(MOE_SRC, "moe_layers_kernel_single_layer")
            breakdown[name] = t
            log(name, t)
        L2 = lay["moe_layer_m1_seed0"]
        t = time_cold(lambda: L2.run_two_call(wsr1, wse1), dev, flush=flush)
        breakdown["moe_layer_m1_seed0_two_call_path"] = {"median_us": t["median_us"]}
        # the same layers with MXFP8 activations (W4A8: moe_layer_w4a8), cold
        for name in ("moe_layer_m1_seed0", "moe_layer_m4_disjoint"):
            Lw = lay[name]
            t = time_cold(lambda: qws.moe_layer_w4a8(Lw.fused, workspace=wsf[Lw.M]), dev, flush=flush)
            nb = breakdown[name]["bytes"]
            t.update({"bytes": nb, "GBps": round(nb / (t["median_us"] * 1e-6) / 1e9, 1),
                      "bf16_activations_median_us": round(breakdown[name]["median_us"], 2)})
            breakdown[name + "_w4a8"] = t
            log(name + "_w4a8", t)
        t1 = breakdown["moe_layer_m1_seed0"]["median_us"]
        breakdown["verify_cost_ratio"] = {reg: round(breakdown[f"moe_layer_m4_{reg}"]["median_us"] / t1, 3)
                                          for reg in synth.REGIMES}
        breakdown["verify_cost_ratio_byte_ideal"] = {
            reg: round(layer_bytes(breakdown[f"moe_layer_m4_{reg}"]["union"], 4) / layer_bytes(K_TOP, 1), 3)
            for reg in synth.REGIMES}
        xh = step.xh
        # a verification window of four positions: the head GEMV alone, and with the greedy
        # epilogue fused (targets, accepted prefix of three synthetic drafts; logits still written)
        x4 = _bf16(synth.token_vectors(0, 1001, 4), dev)
        lg4 = torch.empty((4, head8.rows), dtype=torch.float32, device=dev)
        ws_v = qws.verify_workspace(4, dev)
        draft = torch.tensor([1, 2, 3], dtype=torch.int32, device=dev)
        vout = qws.lmhead_verify_greedy_fp8(head8, x4, draft, ws_v, logits=lg4)
        # the sampled run's settings (temperature 0.6, top_k 29, top_p 0.95) with seeded uniforms
        u4 = torch.tensor(np.random.default_rng(1002).random(4), dtype=torch.float32, device=dev)
        sout = qws.lmhead_verify_sample_fp8(head8, x4, draft, u4, ws_v, logits=lg4)
        head_traffic = {"lmhead_fp8_m1": ("head_fp8.hpp", "head_fp8_kernel"),
                        "lmhead_bf16_m1": ("lmhead.hip", "gemv_bf16_kernel"),
                        "lmhead_verify_greedy_fp8_m4": ("head_fp8.hpp", "head_fp8_kernel_verify_m4")}
        for name, fn, nb in (("lmhead_fp8_m1", lambda: qws.lmhead_gemv_fp8(head8, xh, out=step.logits), head_bytes(1)),
                             ("lmhead_bf16_m1", lambda: qws.lmhead_gemv_bf16(head_bf16, xh, out=step.logits),
                              head_bytes(1, fp8=False)),
                             ("lmhead_fp8_m4", lambda: qws.lmhead_gemv_fp8(head8, x4, out=lg4), head_bytes(4)),
                             ("lmhead_verify_greedy_fp8_m4",
                              lambda: qws.lmhead_verify_greedy_fp8(head8, x4, draft, ws_v, logits=lg4, out=vout),
                              head_bytes(4)),
                             ("lmhead_verify_sample_fp8_m4",
                              lambda: qws.lmhead_verify_sample_fp8(head8, x4, draft, u4, ws_v, out=sout),
                              head_bytes(4))):
            t = time_cold(fn, dev, flush=flush)
            t.update({"bytes": nb, "GBps": round(nb / (t["median_us"] * 1e-6) / 1e9, 1)})
            t["frac_of_peak"] = round(t["GBps"] / PEAK_HBM_GBS, 4)
            t["frac_of_nt_probe"] = round(t["GBps"] / breakdown["probe_read_nt_ceiling"]["GBps"], 4)
            if name in head_traffic:
                t["traffic"] = traffic_for(*head_traffic[name])
            breakdown[name] = t
            log(name, t)
        # run-time specialisation (hipRTC): first call into an empty cache (compile + load), cold
        # kernel times against the template build, then a first call served by the disk cache
        import shutil
        import tempfile
        rtc_dir = tempfile.mkdtemp(prefix="qws_rtc_")
        qws.rtc_reset()
        rtc = {}
        for m_, xx, lg in ((1, xh, step.logits), (4, x4, lg4)):
            t0 = time.perf_counter()
            qws.lmhead_gemv_fp8_rtc(head8, xx, out=lg, cache_dir=rtc_dir)
            torch.cuda.synchronize(dev)
            first = (time.perf_counter() - t0) * 1e3
            tr = time_cold(lambda: qws.lmhead_gemv_fp8_rtc(head8, xx, out=lg, cache_dir=rtc_dir), dev, flush=flush)
            tt = time_cold(lambda: qws.lmhead_gemv_fp8(head8, xx, out=lg), dev, flush=flush)
            rtc[f"m{m_}"] = {"first_call_ms": round(first, 1), "rtc_median_us": round(tr["median_us"], 2),
                             "template_median_us": round(tt["median_us"], 2)}
        st = qws.rtc_stats()
        rtc["compiles"], rtc["compile_ms_total"] = st["compiles"], round(st["compile_ms"], 1)
        qws.rtc_reset()
        t0 = time.perf_counter()
        qws.lmhead_gemv_fp8_rtc(head8, x4, out=lg4, cache_dir=rtc_dir)
        torch.cuda.synchronize(dev)
        rtc["disk_cache_first_call_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        breakdown["lmhead_fp8_rtc"] = rtc
        log("lmhead_fp8_rtc", rtc)
        # the fused MoE kernel compiled at run time for the layer shape: the 42-layer launch of the
        # decode step (M = 1), first call into an empty cache, then back-to-back launches against
        # the template build, then a first call served by the disk cache
        qws.rtc_reset()
        mrtc = {}
        for w8 in (False, True):
            tag = "w4a8" if w8 else "bf16"
            t0 = time.perf_counter()
            step.seq.run(step.ws, w4a8=w8, rtc=True, cache_dir=rtc_dir)
            torch.cuda.synchronize(dev)
            mrtc[f"{tag}_first_call_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
            for name_, use in (("template", False), ("rtc", True)):
                for _ in range(3):
                    step.seq.run(step.ws, w4a8=w8, rtc=use, cache_dir=rtc_dir)
                evr = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
                for a_, b_ in evr:
                    a_.record()
                    step.seq.run(step.ws, w4a8=w8, rtc=use, cache_dir=rtc_dir)
                    b_.record()
                torch.cuda.synchronize(dev)
                tr = sorted(a_.elapsed_time(b_) * 1e3 for a_, b_ in evr)
                mrtc[f"{tag}_{name_}_us_per_layer"] = round(tr[len(tr) // 2] / args.layers, 3)
        st = qws.rtc_stats()
        mrtc["compiles"], mrtc["compile_ms_total"] = st["compiles"], round(st["compile_ms"], 1)
        qws.rtc_reset()
        t0 = time.perf_counter()
        step.seq.run(step.ws, rtc=True, cache_dir=rtc_dir)
        torch.cuda.synchronize(dev)
        mrtc["disk_cache_first_call_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        mrtc["in_kernel_wait_timeouts"] = step.errors()
        shutil.rmtree(rtc_dir, ignore_errors=True)
        breakdown["moe_layers_m1_rtc"] = mrtc
        log("moe_layers_m1_rtc", mrtc)
        # the same M = 1 step captured once in a HIP graph (the 42-layer launch and the head) and
        # replayed: the host's per-step launch work leaves the loop
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step.layers_call()
            step.head_call()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize(dev)
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        breakdown["decode_step_m1_graph"] = {"ms_wall": round(gms, 4), "GBps": round(sb / (gms * 1e-3) / 1e9, 1),
                                             "in_kernel_wait_timeouts": step.errors()}
        log("decode_step_m1_graph", breakdown["decode_step_m1_graph"])
        del graph
        # chained layers (x of layer l+1 = layer l's bf16 y, one launch) against the same layers
        # launched as independent layers. Without the model's normalisation between layers |y| grows
        # ~40x per layer with these weights and is NaN after ~5 layers (every logit then ties), so
        # the comparison uses the first 4 layers, whose values stay finite.
        nch = 4
        chain = []
        for l, L in enumerate(step.layers[:nch]):
            chain.append(qws.MoeLayer(L.x if l == 0 else chain[-1].y_bf16, L.wr, L.packed, K_TOP, want_f32=False))
        cmp = {}
        for name, seq4 in (("chained", qws.MoeLayers(chain)), ("independent", qws.MoeLayers([L.fused for L in step.layers[:nch]]))):
            for _ in range(3):
                seq4.run(step.ws)
            evc = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
            for a, b in evc:
                a.record()
                seq4.run(step.ws)
                b.record()
            torch.cuda.synchronize(dev)
            tc = sorted(a.elapsed_time(b) * 1e3 for a, b in evc)
            cmp[name] = {"us_median": round(tc[len(tc) // 2], 2), "us_per_layer": round(tc[len(tc) // 2] / nch, 3)}
        cmp["finite"] = bool(all(torch.isfinite(L.y_bf16.float()).all() for L in chain))
        cmp["in_kernel_wait_timeouts"] = step.errors()
        breakdown["moe_layers_m1_chained_4"] = cmp
        log("moe_layers_m1_chained_4", cmp)
        del chain
        # decode step at M = 4 (natural routing), sharing the M = 1 step's expert banks
        step4 = DecodeStep(qws, 4, dev, args.layers, head8, packed=[L.packed for L in step.layers])
        step4.layers_call()
        torch.cuda.synchronize(dev)
        r4 = step4.timed(max(5, args.steps // 2), 2)
        b4 = step4.bytes()
        breakdown["decode_step_m4"] = {"ms_wall": round(r4["wall_ms"], 4), "bytes": b4,
                                       "moe_us_per_layer": round(r4["moe_us_mean"] / args.layers, 3),
                                       "GBps": round(b4 / (r4["wall_ms"] * 1e-3) / 1e9, 1),
                                       "mean_union": round(float(np.mean([L.union() for L in step4.layers])), 2),
                                       "moe_layers_traffic": traffic_for(MOE_SRC, "moe_layers_kernel_m4"),
                                       "moe_layers_algorithmic_bytes": b4 - head_bytes(4)}
        log("decode_step_m4", breakdown["decode_step_m4"])
        step4.w4a8 = True
        r48 = step4.timed(max(5, args.steps // 2), 2)
        breakdown["decode_step_m4_w4a8"] = {"ms_wall": round(r48["wall_ms"], 4),
                                            "moe_us_per_layer": round(r48["moe_us_mean"] / args.layers, 3),
                                            "GBps": round(b4 / (r48["wall_ms"] * 1e-3) / 1e9, 1),
                                            "in_kernel_wait_timeouts": step4.errors()}
        log("decode_step_m4_w4a8", breakdown["decode_step_m4_w4a8"])
        del step4
        # speculation priced from these steps: a draft step taken as one MoE layer plus the shared
        # head at M = 1 (the draft is the model's one extra NEXTN layer; attention is not modelled)
        draft_ms = (r["moe_us_mean"] / args.layers + r["head_us_mean"]) / 1e3
        breakdown["speculation"] = speculation_model(r["wall_ms"], r4["wall_ms"], draft_ms)
        log("speculation", breakdown["speculation"])
        # FP8 vs bf16 head agreement over seeded x vectors (a measurement, not parity)
        if args.agreement:
            topk1, topk10, in10 = 0, 0.0, 0
            n = args.agreement
            xs = synth.token_vectors(7, 0, n)
            lb = torch.empty((4, 157184), dtype=torch.float32, device=dev)
            l8 = torch.empty((4, 157184), dtype=torch.float32, device=dev)
            for i in range(0, n, 4):
                xb = _bf16(xs[i:i + 4], dev)
                qws.lmhead_gemv_fp8(head8, xb, out=l8[:xb.shape[0]])
                qws.lmhead_gemv_bf16(head_bf16, xb, out=lb[:xb.shape[0]])
                t8 = torch.topk(l8[:xb.shape[0]], 10, dim=1).indices
                tb = torch.topk(lb[:xb.shape[0]], 10, dim=1).indices
                topk1 += int((t8[:, 0] == tb[:, 0]).sum())
                in10 += int((t8[:, :1] == tb).any(dim=1).sum())
                for j in range(xb.shape[0]):
                    topk10 += len(set(t8[j].tolist()) & set(tb[j].tolist())) / 10
            breakdown["fp8_vs_bf16_head_agreement"] = {"n_x": n, "top1": round(topk1 / n, 4),
                                                       "top10_overlap": round(topk10 / n, 4),
                                                       "top1_in_bf16_top10": round(in10 / n, 4)}
            log("agreement", breakdown["fp8_vs_bf16_head_agreement"])

    # a plain device copy of known size (probe_copy_kernel, 256 MiB read + 256 MiB written): the
    # scale for rocprofv3 FETCH_SIZE / WRITE_SIZE readings of the kernels above
    cp_src = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    qws.probe_copy(cp_src, cp_dst, 4096)
    torch.cuda.synchronize(dev)
    del cp_src, cp_dst

    cpu = None
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(sb)

    out = {"metric": "HBM GB/s & % of peak; us per MoE layer (M=1, M=4); FP8 LM-head us",
           "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(r["wall_ms"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "fp32-accumulate (bf16 activations x MXFP4/FP8-dequantised weights)",
           "data": "synthetic: seeded MXFP4 bytes, bf16 N(0,0.02^2) router/head weights, bf16 N(0,1) tokens",
           "config": {"workload": f"decode step: {args.layers} independent MoE layers (512 routed + 1 shared, top-8, "
                                  "hidden 2560, inter 768, MXFP4) + FP8 E4M3 LM head 157184x2560, M=1",
                      "layers": args.layers, "M": 1, "bytes_per_step": sb},
           "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
           "roofline": roofline, "cpu_baseline": cpu, "breakdown": breakdown}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
