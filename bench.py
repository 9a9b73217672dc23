"""Benchmark of the sparse MoE layer on one MI355X.

Headline workload: prefill of 4,096 tokens through 48 stacked MoE layers with
3-bit experts (hidden 2048, 512 experts, top-10 with renormalised softmax,
expert intermediate 704, one shared expert of 704, 32-weight blocks with fp16
scales, uniform routing), with the residual + RMSNorm + bf16 glue between
layers.  One step = one pass of all 48 layers over the 4,096 tokens (route,
permute, expert FFN, shared expert, combine, glue at every layer); `value` is
tokens per second through the whole stack.  `--steps` steps are timed after
`--warmup` untimed ones, each bracketed by HIP events (median and range
reported); the same steps are also timed as replays of one captured graph.
The roofline is that of the stack's dominant kernel, the grouped gate/up
GEMM (MFMA-bound), timed on the stack's own per-layer inputs.

Secondary workloads, each built from its own seeds and reported with its own
roofline and an oracle CPU baseline on a bounded sample:
  decode1   single-token decode walking 48 resident 2-bit layers (HBM)
  decode16  16 tokens through a 48-layer 2-bit stack (HBM)
  verify4   the verify window (a token + 3 drafts) through a 48-layer stack;
            also with the opt-in route tail skip (speed and output shift)
  prefill   32,768 tokens through one 2-bit layer (MFMA, Zipf-skewed routing)
  four_bit  the 4-bit block variant (4,096-token layer; single-token decode)
plus a kernel probe (the decode GEMV kernels alone over every expert of a
layer), labelled as such.

Output: one JSON line.  --gpus N with N > 1 exits: one GPU only.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bit_quantized_expert_amd as M  # noqa: E402
from bit_quantized_expert_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16 MFMA
METRIC = "MoE-layer tokens/s (decode & prefill) + % of HBM BW / MFMA peak on 1 MI355X"


# ----------------------------------------------------------------------------- sizes and work

def matrix_bytes(rows, k, qbits) -> int:
    return rows * k * qbits // 8 + (rows * k // 32) * 2


def expert_bytes(s) -> int:
    return 2 * matrix_bytes(s.inter, s.hidden, s.qbits) + matrix_bytes(s.hidden, s.inter, s.qbits)


def shared_bytes(s) -> int:
    if not s.shared_inter:
        return 0
    return 2 * matrix_bytes(s.shared_inter, s.hidden, s.qbits) + matrix_bytes(s.hidden, s.shared_inter, s.qbits)


def router_bytes(s) -> int:
    return s.n_experts * s.hidden * 2


def ffn_flops(s, T) -> tuple[int, int]:
    """Algorithmic flops of the gate/up and down projections for T tokens
    (routed pairs plus the shared expert)."""
    P = T * s.top_k
    gu = 2 * s.hidden * 2 * (P * s.inter + T * s.shared_inter)
    dn = 2 * s.hidden * (P * s.inter + T * s.shared_inter)
    return gu, dn


def layer_flops(s, T) -> int:
    gu, dn = ffn_flops(s, T)
    return gu + dn + 2 * T * s.hidden * s.n_experts


def stats(ms) -> dict:
    a = np.asarray(ms, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(a.min()), "max": float(a.max()), "n": int(a.size)}


# ----------------------------------------------------------------------------- device layers

def build_layers(wl, n_layers, device, log):
    """n_layers resident layers of a workload (quantised with the library:
    moe_quantize into the canonical layout, moe_repack into the arena)."""
    layers = []
    s = wl.shape
    t0 = time.time()
    for l in range(n_layers):
        w_r, bias = synth.router(wl, l, device)
        arena = M.QArena(s.n_experts, s.hidden, s.inter, s.qbits, device)
        for lo in range(0, s.n_experts, 256):
            sl = slice(lo, min(s.n_experts, lo + 256))
            for m, w in enumerate(synth.expert_weights(wl, l, device, experts=sl)):
                arena.quantize_from(m, w, experts=sl)
        sarena = None
        sw = synth.shared_weights(wl, l, device)
        if sw is not None:
            sarena = M.QArena(1, s.hidden, s.shared_inter, s.qbits, device)
            for m, w in enumerate(sw):
                sarena.quantize_from(m, w[None])
        layers.append(M.QLayer(w_r, bias, arena, sarena))
        if (l + 1) % 16 == 0 or l + 1 == n_layers:
            torch.cuda.synchronize()
            log(f"{wl.name}: built {l + 1}/{n_layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return layers


def release():
    """Synchronise and hand cached device memory back to the driver (callers
    drop their references first)."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def event_steps(fn, steps, warmup):
    """warmup untimed calls, then `steps` calls each between HIP events on the
    current stream; synchronised before and after.  Returns (per-step ms,
    wall seconds of the timed region)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)], wall


class FfnState:
    """Inputs of moe_expert_ffn for one token batch on one layer: routing,
    permutation and a workspace holding the plan, the activations and h."""

    def __init__(self, s, T, device, algo, shape=None):
        self.s = shape or s
        self.algo = algo
        s = self.s
        self.T = T
        P = T * s.top_k
        self.ws = M.alloc_workspace(s, T, device=device)
        self.idx = torch.empty(T, s.top_k, dtype=torch.int32, device=device)
        self.w = torch.empty(T, s.top_k, device=device)
        self.counts = torch.empty(s.n_experts, dtype=torch.int32, device=device)
        self.offsets = torch.empty(s.n_experts + 1, dtype=torch.int32, device=device)
        self.sp = torch.empty(P, dtype=torch.int32, device=device)
        self.pp = torch.empty(P, dtype=torch.int32, device=device)
        self.y = torch.empty(P, s.hidden, device=device)
        self.so = torch.empty(T, s.hidden, device=device) if s.shared_inter else None

    def prepare(self, x, layer):
        M.route(x, layer, self.s, self.idx, self.w, ws=self.ws)
        M.permute(self.idx, self.T, self.s, self.counts, self.offsets, self.sp, self.pp, self.ws)
        self.run(x, layer, 0)

    def run(self, x, layer, flags):
        M.expert_ffn(x, layer, self.s, self.offsets, self.sp, self.y, self.so, algo=self.algo, ws=self.ws,
                     flags=flags)


def time_phase(states, xs, layers, skip, reps):
    """One projection kernel launched alone through moe_expert_ffn
    (REUSE_PLAN | skip), once per state back to back in one captured graph,
    replayed `reps` times between HIP events on the capturing stream.
    Returns the per-replay average per launch (ms), a list."""
    flags = M.FFN_REUSE_PLAN | skip
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st, x, layer in zip(states, xs, layers):
            st.run(x, layer, flags)
    g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    del g
    return [ev[i].elapsed_time(ev[i + 1]) / len(states) for i in range(reps)]


# ----------------------------------------------------------------------------- traffic counters

TRAFFIC_FILES = {
    "grouped_gateup_prefill3": ("grouped_gateup_prefill3_traffic.txt", ("ffn_grouped.hip", "common.h", "launch.h")),
}


def source_digest(files) -> str:
    """SHA-256 of kernel sources with // comments and blank lines removed (a
    comment edit does not change the code the counters measured)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "bit_quantized_expert_amd", "csrc", f)) as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    runs (scaled by the copy-kernel calibration), or None when the kernel
    sources changed since the counters were taken."""
    fname, files = TRAFFIC_FILES[key]
    try:
        kv = {}
        for line in open(os.path.join(ROOT, "profiles", fname)):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if source_digest(files) != kv["source_sha256"]:
            return None
        return (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) +
                float(kv["write_kib"]) * float(kv["write_scale"])) * 1024
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- stacks

class Stack:
    """T tokens through the resident layers with the residual + RMSNorm +
    bf16 glue, as plain launches or as one captured graph."""

    def __init__(self, wl, layers, dev, flags=0):
        s = wl.shape
        self.wl, self.s, self.layers, self.T, self.flags = wl, s, layers, wl.tokens, flags
        self.x0 = synth.tokens(wl, dev).float()
        self.r = torch.empty(self.T, s.hidden, device=dev)
        self.a = torch.empty(self.T, s.hidden, dtype=torch.bfloat16, device=dev)
        self.ws = M.alloc_workspace(s, self.T, device=dev)
        self.idx = torch.empty(len(layers), self.T, s.top_k, dtype=torch.int32, device=dev)
        self.acts = None
        self.graph = None

    def step(self, record=None):
        self.r.copy_(self.x0)
        M.rmsnorm_bf16(self.r, self.a)
        for l, layer in enumerate(self.layers):
            if record is not None and l in record:
                record[l] = self.a.clone()
            M.layer_forward(self.a, layer, self.s, residual=self.r, next_in=self.a, topk_idx=self.idx[l], ws=self.ws,
                            flags=self.flags)

    def capture(self):
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.step()

    def replay(self):
        self.graph.replay()


def stack_bench(wl, dev, log, steps, warmup, n_layers=48, kernel_layers=None, algo_label=""):
    """Time a stack workload (plain launches and graph replay), and return its
    layers' per-layer inputs on `kernel_layers` for kernel timing."""
    layers = build_layers(wl, n_layers, dev, log)
    st = Stack(wl, layers, dev)
    record = {l: None for l in (kernel_layers or [])}
    st.step(record=record)
    torch.cuda.synchronize()
    r_eager = st.r.clone()
    plain_ms, plain_wall = event_steps(st.step, steps, warmup)
    st.capture()
    graph_ms, graph_wall = event_steps(st.replay, steps, warmup)
    same = bool(torch.equal(st.r, r_eager))
    if not same:
        raise SystemExit(f"{wl.name}: graph replay differs from the eager stack")
    uniq = [int(torch.unique(st.idx[l]).numel()) for l in range(n_layers)]
    log(f"{wl.name} stack: plain {np.median(plain_ms):.3f} ms/step, graph {np.median(graph_ms):.3f} ms/step "
        f"({wl.tokens / np.median(graph_ms) * 1e3:.0f} tok/s), unique experts/layer {np.mean(uniq):.1f}")
    return layers, st, record, {"plain": plain_ms, "plain_wall": plain_wall, "graph": graph_ms,
                                "graph_wall": graph_wall, "uniq": uniq}


def kernel_timing(wl, layers, record, dev, reps, log, label):
    """The grouped (or GEMV) gate/up and down kernels launched alone on the
    recorded per-layer inputs of a stack, walking those layers."""
    s = wl.shape
    ls = sorted(record)
    algo = "grouped" if wl.tokens > 16 else "gemv"
    states, xs, lays = [], [], []
    for l in ls:
        stt = FfnState(s, wl.tokens, dev, algo)
        stt.prepare(record[l], layers[l])
        states.append(stt)
        xs.append(record[l])
        lays.append(layers[l])
    torch.cuda.synchronize()
    gu = time_phase(states, xs, lays, M.FFN_SKIP_DOWN, reps)
    dn = time_phase(states, xs, lays, M.FFN_SKIP_GATEUP, reps)
    counts = torch.stack([stt.counts for stt in states]).cpu().numpy()
    del states
    torch.cuda.empty_cache()
    log(f"{label}: gate/up alone {np.median(gu) * 1e3:.1f} us, down alone {np.median(dn) * 1e3:.1f} us "
        f"(layers {ls[0]}..{ls[-1]})")
    return gu, dn, counts


# ----------------------------------------------------------------------------- CPU baseline (oracle)

def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_oracle_sample(wl, layer_ids, x, dev, stack=True):
    """The oracle on a bounded sample: token rows x (float64) through the
    layers `layer_ids` of the workload, with the stack glue (RMSNorm + bf16
    before each layer, residual after) when `stack`, else each layer on its
    own row of x.  float64 numpy.  Timed: the glue, routing, the dequantisation
    of the experts the sample touches and the SwiGLU matmuls.  Not timed:
    drawing the seeded fp32 weights and the oracle's quantisation of them (its
    inputs).  Returns the timed seconds."""
    import concurrent.futures as cf
    from oracle import moe_oracle as O
    s = wl.shape
    r = np.array(x, dtype=np.float64, copy=True)
    timed = 0.0
    pool = cf.ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1)))
    for i, l in enumerate(layer_ids):
        w_r, bias = synth.router(wl, l, dev)
        wr = w_r.float().cpu().numpy().astype(np.float64)
        b = None if bias is None else bias.cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        a = O.rmsnorm_bf16(r) if stack else r[i:i + 1]
        idx = O.topk_select(O.router_logits(a, wr, b), s.top_k)
        timed += time.perf_counter() - t0
        need = sorted({int(e) for e in idx.ravel()})
        draws = []
        for e in need:
            g, u, d = synth.expert_weights(wl, l, dev, experts=slice(e, e + 1))
            draws.append((g[0].cpu().numpy(), u[0].cpu().numpy(), d[0].cpu().numpy()))
        experts = dict(zip(need, pool.map(lambda t: O.QExpert.from_float(*t, s.qbits), draws)))
        sw = synth.shared_weights(wl, l, dev)
        shared = O.QExpert.from_float(*(t.cpu().numpy() for t in sw), s.qbits) if sw is not None else None

        class View:
            def __len__(self):
                return s.n_experts

            def __getitem__(self, e):
                return experts[int(e)]

        t0 = time.perf_counter()
        out = O.layer_forward(a, wr, b, View(), shared, s.top_k)
        if stack:
            r = r + out
        timed += time.perf_counter() - t0
    pool.shutdown()
    return timed


def cpu_baseline(wl, layer_ids, x, dev, log, stack, what):
    """tokens/s of the oracle through the sample: rows of x through the whole
    stack (stack), or one token per layer pass (not stack)."""
    sec = cpu_oracle_sample(wl, layer_ids, x, dev, stack=stack)
    n_tok = x.shape[0]
    passes = n_tok if stack else len(layer_ids)
    log(f"{wl.name}: oracle {what} in {sec:.2f}s")
    return {"value": passes / sec,
            "unit": f"tokens/s (through {len(layer_ids)} layers)" if stack else "tokens/s (one token through one layer)",
            "cores": int(blas_threads()), "kind": "oracle",
            "sample": f"{what} of the {wl.name} workload; float64 numpy; glue, routing, dequantisation of the "
                      f"touched experts and the matmuls timed; drawing and quantising the inputs not timed; "
                      f"{sec:.1f} s of CPU time; BLAS threads {blas_threads()}, host os.cpu_count()={os.cpu_count()}"}


def x_rows(wl, dev, rows, layer=0):
    return synth.tokens(wl, dev, layer=layer)[torch.as_tensor(rows, device=dev)].float().cpu().numpy()


# ----------------------------------------------------------------------------- workloads

def headline_prefill3(args, dev, log):
    wl = synth.WORKLOADS["prefill3"]
    s = wl.shape
    T = wl.tokens
    klayers = list(range(0, args.layers, max(1, args.layers // 8)))[:8]
    layers, st, record, t = stack_bench(wl, dev, log, args.steps, args.warmup, args.layers, klayers)
    del st
    torch.cuda.empty_cache()
    gu, dn, counts = kernel_timing(wl, layers, record, dev, args.kernel_reps, log, "prefill3")
    del layers, record
    release()
    gu_f, dn_f = ffn_flops(s, T)
    per_layer = layer_flops(s, T)
    wbytes = args.layers * (s.n_experts * expert_bytes(s) + shared_bytes(s) + router_bytes(s))
    ms = float(np.median(t["plain"]))
    return {
        "t": t, "ms_per_step": sum(t["plain"]) / len(t["plain"]),
        "gu_ms": gu, "dn_ms": dn, "gu_flops": gu_f, "dn_flops": dn_f,
        "stack_tflops": args.layers * per_layer / ms / 1e9,
        "weight_GBs": wbytes / ms / 1e6,
        "rows_per_expert": {"min": int(counts.min()), "max": int(counts.max()), "mean": float(counts.mean())},
    }


def decode1_bench(args, dev, log):
    """Single-token decode walking 48 resident layers: one graph of 48
    fused layers, replayed; a step = one token through one layer."""
    wl = synth.WORKLOADS["decode1"]
    s = wl.shape
    L = args.layers
    layers = build_layers(wl, L, dev, log)
    xs = [synth.tokens(wl, dev, layer=i, n_tokens=1) for i in range(L)]
    ws = M.alloc_workspace(s, 1, device=dev)
    out = torch.empty(L, 1, s.hidden, device=dev)

    def walk():
        for i in range(L):
            M.layer_forward(xs[i], layers[i], s, out=out[i], ws=ws)

    walk()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        walk()
    rep_ms, _ = event_steps(g.replay, max(20, args.steps), 3)
    if not torch.equal(out, eager):
        raise SystemExit("decode1: graph replay differs from the eager layers")
    layer_ms = [m / L for m in rep_ms]
    nbytes = router_bytes(s) + s.top_k * expert_bytes(s) + shared_bytes(s)
    # the gate/up and down kernels alone with the slot table given (labelled as such)
    states = []
    for i in range(L):
        stt = FfnState(s, 1, dev, "gemv")
        stt.prepare(xs[i], layers[i])
        states.append(stt)
    torch.cuda.synchronize()
    gu = time_phase(states, xs, layers, M.FFN_SKIP_DOWN, reps=20)
    dn = time_phase(states, xs, layers, M.FFN_SKIP_GATEUP, reps=20)
    del states
    probe = probe_gemv(s, layers, dev, log)
    del g, layers
    release()
    med = float(np.median(layer_ms))
    gu_b = (s.top_k * expert_bytes(s) + shared_bytes(s)) * 2 // 3
    dn_b = (s.top_k * expert_bytes(s) + shared_bytes(s)) // 3
    log(f"decode1: {med * 1e3:.2f} us/layer, {nbytes / med / 1e6:.0f} GB/s")
    return {"tokens_per_s": 1.0 / med * 1e3, "layer_us": {k: v * 1e3 for k, v in stats(layer_ms).items() if k != "n"},
            "roofline": {"bound": "hbm", "kernel": "whole single-token layer (router, gate/up with the top-k made "
                                                   "inside it, down + combine: three launches)",
                         "bytes_per_launch": nbytes, "avg_us": med * 1e3, "achieved": nbytes / med / 1e6,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": nbytes / med / 1e6 / HBM_PEAK_GBS,
                         "traffic": None},
            "kernels_alone": {"gateup_gemv_us": float(np.median(gu)) * 1e3,
                              "gateup_GBs": gu_b / float(np.median(gu)) / 1e6,
                              "down_gemv_us": float(np.median(dn)) * 1e3,
                              "down_GBs": dn_b / float(np.median(dn)) / 1e6,
                              "note": "launched alone with the slot table given (not the mode inside the layer)"},
            "probe": probe}


def probe_gemv(s, layers, dev, log):
    """Kernel probe, labelled as such: the decode gate/up and down GEMV
    kernels alone over every expert of a layer (16 tokens, top-32, one pair
    per expert), 8 layers walked."""
    import dataclasses
    ps = dataclasses.replace(s, top_k=32)
    T = s.n_experts // 32
    xs = synth.tokens(synth.WORKLOADS["decode16"], dev, layer=777, n_tokens=T)
    sts = []
    n = min(8, len(layers))
    for l in range(n):
        st = FfnState(s, T, dev, "gemv", shape=ps)
        st.offsets.copy_(torch.arange(s.n_experts + 1, dtype=torch.int32, device=dev))
        st.sp.copy_(torch.arange(s.n_experts, dtype=torch.int32, device=dev))
        st.run(xs, layers[l], 0)
        sts.append(st)
    torch.cuda.synchronize()
    gu = float(np.median(time_phase(sts, [xs] * n, layers[:n], M.FFN_SKIP_DOWN, reps=5)))
    dn = float(np.median(time_phase(sts, [xs] * n, layers[:n], M.FFN_SKIP_GATEUP, reps=5)))
    gu_b = (s.n_experts * expert_bytes(s) + shared_bytes(s)) * 2 // 3
    dn_b = (s.n_experts * expert_bytes(s) + shared_bytes(s)) // 3
    log(f"probe: gate/up {gu * 1e3:.1f} us {gu_b / gu / 1e6:.0f} GB/s; down {dn * 1e3:.1f} us {dn_b / dn / 1e6:.0f} GB/s")
    return {"what": "kernel probe: decode gate/up and down GEMV kernels alone over all 512 experts + shared of a "
                    "layer (16 tokens x top-32, one pair per expert)",
            "gateup": {"avg_us": gu * 1e3, "bytes": gu_b, "GBs": gu_b / gu / 1e6, "frac": gu_b / gu / 1e6 / HBM_PEAK_GBS},
            "down": {"avg_us": dn * 1e3, "bytes": dn_b, "GBs": dn_b / dn / 1e6, "frac": dn_b / dn / 1e6 / HBM_PEAK_GBS}}


def decode_stack_secondary(name, args, dev, log):
    wl = synth.WORKLOADS[name]
    s = wl.shape
    layers, st, record, t = stack_bench(wl, dev, log, max(20, args.steps), 3, args.layers)
    del st, layers
    release()
    nbytes = sum(u * expert_bytes(s) + shared_bytes(s) + router_bytes(s) for u in t["uniq"])
    med = float(np.median(t["graph"]))
    return {"tokens": wl.tokens, "layers": args.layers, "tokens_per_s": wl.tokens / med * 1e3,
            "ms_per_step": {"graph": stats(t["graph"]), "plain": stats(t["plain"])},
            "unique_experts_per_layer": float(np.mean(t["uniq"])),
            "roofline": {"bound": "hbm", "kernel": "whole stack step (per layer: router, gate/up with the selection "
                                                   "inside it, down, combine with the glue), graph replay",
                         "bytes_per_step": nbytes, "achieved": nbytes / med / 1e6, "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": nbytes / med / 1e6 / HBM_PEAK_GBS, "traffic": None}}


def tail_skip_secondary(args, dev, log, first_tail=7):
    """The opt-in route tail skip on the verify-window stack (a token + 3
    drafts through 48 layers): speed with and without it (graph replays), the
    experts it drops, and the output shift it causes -- per layer on the same
    inputs (the exact stack's activations), and at the end of the stack."""
    wl = synth.WORKLOADS["verify4"]
    s = wl.shape
    L = args.layers
    layers = build_layers(wl, L, dev, log)
    exact = Stack(wl, layers, dev)
    skip = Stack(wl, layers, dev, flags=M.ROUTE_TAIL_SKIP)
    acts = {l: None for l in range(L)}
    exact.step(record=acts)
    skip.step()
    torch.cuda.synchronize()
    end_shift = float(torch.linalg.vector_norm(skip.r - exact.r) / torch.linalg.vector_norm(exact.r))
    steps = max(20, args.steps)
    exact.capture()
    skip.capture()
    ms_exact, _ = event_steps(exact.replay, steps, 3)
    ms_skip, _ = event_steps(skip.replay, steps, 3)
    # per layer, the same input through the layer with and without the skip
    ws = M.alloc_workspace(s, wl.tokens, device=dev)
    o0 = torch.empty(wl.tokens, s.hidden, device=dev)
    o1 = torch.empty_like(o0)
    idx = torch.empty(wl.tokens, s.top_k, dtype=torch.int32, device=dev)
    shifts, dropped, used = [], [], []
    for l in range(L):
        M.layer_forward(acts[l], layers[l], s, out=o0, topk_idx=idx, ws=ws)
        M.layer_forward(acts[l], layers[l], s, out=o1, ws=ws, flags=M.ROUTE_TAIL_SKIP)
        shifts.append(float(torch.linalg.vector_norm(o1 - o0) / torch.linalg.vector_norm(o0)))
        ix = idx.cpu().numpy()
        sel = set(np.unique(ix).tolist())
        head = set(np.unique(ix[:, :first_tail]).tolist())
        used.append(len(sel))
        dropped.append(len(sel - head))
    del exact, skip, layers, ws, acts
    release()
    me, ms = float(np.median(ms_exact)), float(np.median(ms_skip))
    log(f"verify4 tail skip: {ms:.3f} vs {me:.3f} ms/step ({me / ms - 1:+.1%}); dropped {np.mean(dropped):.2f} of "
        f"{np.mean(used):.1f} experts per layer; per-layer relL2 shift median {np.median(shifts):.2e}, "
        f"end of stack {end_shift:.2e}")
    return {"what": "route tail skip (opt-in): verify window of 4 tokens through the 48-layer stack; experts no "
                    "token ranks 0..6 are dropped", "ms_per_step": {"exact": stats(ms_exact), "tail_skip": stats(ms_skip)},
            "speedup": me / ms, "experts_per_layer": float(np.mean(used)),
            "dropped_per_layer": float(np.mean(dropped)),
            "expert_bytes_saved_per_layer": float(np.mean(dropped)) * expert_bytes(s),
            "out_shift_relL2_per_layer": {"median": float(np.median(shifts)), "max": float(np.max(shifts))},
            "out_shift_relL2_end_of_stack": end_shift}


def prefill32k_secondary(args, dev, log):
    wl = synth.WORKLOADS["prefill"]
    s = wl.shape
    T = wl.tokens
    layers = build_layers(wl, 1, dev, log)
    layer = layers[0]
    x = synth.tokens(wl, dev)
    ws = M.alloc_workspace(s, T, device=dev)
    out = torch.empty(T, s.hidden, device=dev)
    layer_ms, _ = event_steps(lambda: M.layer_forward(x, layer, s, out=out, ws=ws), 20, 2)
    del ws, out
    torch.cuda.empty_cache()
    gu, dn, counts = kernel_timing(wl, layers, {0: x}, dev, 20, log, "prefill 32k")
    del layers, layer
    release()
    gu_f, dn_f = ffn_flops(s, T)
    tot = layer_flops(s, T)
    med = float(np.median(layer_ms))
    gum = float(np.median(gu))
    return {"tokens": T, "layer_ms": stats(layer_ms), "tokens_per_s": T / med * 1e3,
            "layer_tflops": tot / med / 1e9, "layer_mfma_frac": tot / med / 1e9 / MFMA_PEAK_TFLOPS,
            "roofline": {"bound": "mfma", "kernel": "grouped gate/up GEMM (2-bit, 128-row tiles) + SwiGLU, launched "
                                                    "alone on the layer's plan", "flops_per_launch": gu_f,
                         "avg_us": gum * 1e3, "achieved": gu_f / gum / 1e9, "peak": MFMA_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": gu_f / gum / 1e9 / MFMA_PEAK_TFLOPS, "traffic": None},
            "down": {"avg_ms": stats(dn), "tflops": dn_f / float(np.median(dn)) / 1e9,
                     "frac": dn_f / float(np.median(dn)) / 1e9 / MFMA_PEAK_TFLOPS},
            "experts_used": int((counts > 0).sum()), "largest_expert_tokens": int(counts.max())}


def fourbit_secondary(dev, log, n_layers=8):
    wl = synth.WORKLOADS["prefill4"]
    s = wl.shape
    T = wl.tokens
    layers = build_layers(wl, n_layers, dev, log)
    x = synth.tokens(wl, dev)
    ws = M.alloc_workspace(s, T, device=dev)
    out = torch.empty(T, s.hidden, device=dev)
    layer_ms, _ = event_steps(lambda: M.layer_forward(x, layers[0], s, out=out, ws=ws), 20, 2)
    del ws, out
    xs = [synth.tokens(wl, dev, layer=100 + i, n_tokens=1) for i in range(n_layers)]
    ws1 = M.alloc_workspace(s, 1, device=dev)
    o1 = torch.empty(n_layers, 1, s.hidden, device=dev)

    def walk():
        for i in range(n_layers):
            M.layer_forward(xs[i], layers[i], s, out=o1[i], ws=ws1)

    walk()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        walk()
    rep_ms, _ = event_steps(g.replay, 40, 3)
    del g, layers
    release()
    us = float(np.median(rep_ms)) / n_layers * 1e3
    nbytes = router_bytes(s) + s.top_k * expert_bytes(s) + shared_bytes(s)
    med = float(np.median(layer_ms))
    log(f"4-bit: 4,096-token layer {med:.3f} ms; single-token decode {us:.2f} us/layer")
    return {"prefill4k_layer": {"tokens": T, "layer_ms": stats(layer_ms), "tokens_per_s": T / med * 1e3,
                                "layer_tflops": layer_flops(s, T) / med / 1e9,
                                "layer_mfma_frac": layer_flops(s, T) / med / 1e9 / MFMA_PEAK_TFLOPS},
            "decode1": {"avg_us": us, "tokens_per_s": 1e6 / us, "GBs": nbytes / us / 1e3,
                        "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "layers": n_layers}}


# ----------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed passes of the 48-layer headline stack")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--only", default="",
                    help="comma list: headline,decode1,decode16,verify4,tail_skip,prefill,four_bit")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy 10 times (scales the HBM byte counters)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: --gpus must be 1 (the layer shards as data "
                                   "parallel with no exchange; see the design notes)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    dev = "cuda:0"
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read_per_launch": src.numel() * 4}))
        return
    M.lib()
    only = set(filter(None, args.only.split(",")))
    want = (lambda k: not only or k in only)
    cpu = not args.no_cpu_baseline

    res_sec = {}
    head = None
    if want("headline"):
        head = headline_prefill3(args, dev, log)
    if want("decode1"):
        res_sec["decode1"] = decode1_bench(args, dev, log)
    for name in ("decode16", "verify4"):
        if want(name):
            res_sec[name + "_stack"] = decode_stack_secondary(name, args, dev, log)
    if want("tail_skip"):
        res_sec["verify4_tail_skip"] = tail_skip_secondary(args, dev, log)
    if want("prefill"):
        res_sec["prefill32k_layer"] = prefill32k_secondary(args, dev, log)
    if want("four_bit"):
        res_sec["four_bit"] = fourbit_secondary(dev, log)

    # oracle CPU baselines on bounded samples (after the GPU work)
    if cpu:
        L = args.layers
        if head is not None:
            wl = synth.WORKLOADS["prefill3"]
            rows = [0, 1365, 2730, 4095]
            head["cpu"] = cpu_baseline(wl, list(range(L)), x_rows(wl, dev, rows), dev, log, True,
                                       f"{len(rows)} tokens through all {L} layers")
        if "decode1" in res_sec:
            wl = synth.WORKLOADS["decode1"]
            n = 48
            x = np.concatenate([synth.tokens(wl, dev, layer=i, n_tokens=1).float().cpu().numpy() for i in range(n)])
            res_sec["decode1"]["cpu_baseline"] = cpu_baseline(wl, list(range(n)), x, dev, log, False,
                                                              f"{n} single-token layer passes (token i through layer i)")
        if "decode16_stack" in res_sec:
            wl = synth.WORKLOADS["decode16"]
            res_sec["decode16_stack"]["cpu_baseline"] = cpu_baseline(wl, list(range(L)), x_rows(wl, dev, [0, 15]),
                                                                     dev, log, True,
                                                                     f"2 of the 16 tokens through all {L} layers")
        if "prefill32k_layer" in res_sec:
            wl = synth.WORKLOADS["prefill"]
            rows = list(range(0, wl.tokens, 256))
            res_sec["prefill32k_layer"]["cpu_baseline"] = cpu_baseline(wl, [0], x_rows(wl, dev, rows), dev, log, True,
                                                                       f"{len(rows)} tokens through the layer")

    if head is None:
        print(json.dumps({"secondary": res_sec}), flush=True)
        return
    s3 = synth.WORKLOADS["prefill3"].shape
    T = synth.WORKLOADS["prefill3"].tokens
    steps = args.steps
    ms_per_step = head["ms_per_step"]
    gum = float(np.median(head["gu_ms"]))
    res = {
        "metric": METRIC,
        "value": T / ms_per_step * 1e3,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, 3-bit experts, fp16 MFMA with fp32 accumulation",
        "data": "synthetic: seeded N(0, 0.02) weights quantised to 3-bit blocks, N(0, 1) bf16 tokens",
        "config": {"workload": "prefill3: 4,096 tokens through 48 stacked MoE layers (hidden 2048, 512 experts, "
                               "top-10 renormalised softmax, expert inter 704, shared expert 704, 3-bit blocks of 32 "
                               "with fp16 scales, uniform routing, residual + RMSNorm + bf16 glue); one step = one "
                               "pass of the stack, plain launches",
                   "global_batch": T, "layers": args.layers, "parallelism": "none (1 GPU)"},
        "timing": {"plain_ms": stats(head["t"]["plain"]), "graph_ms": stats(head["t"]["graph"]),
                   "plain_wall_s": head["t"]["plain_wall"], "stack_tflops": head["stack_tflops"],
                   "stack_mfma_frac": head["stack_tflops"] / MFMA_PEAK_TFLOPS, "weight_GBs": head["weight_GBs"],
                   "rows_per_expert": head["rows_per_expert"]},
        "roofline": {"bound": "mfma", "achieved": head["gu_flops"] / gum / 1e9, "peak": MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": head["gu_flops"] / gum / 1e9 / MFMA_PEAK_TFLOPS,
                     "traffic": measured_traffic("grouped_gateup_prefill3"),
                     "kernel": "grouped_gemm2_kernel<3, gate/up, 4 waves, K%128==0, 96-row tiles> (grouped gate/up "
                               "GEMM + SwiGLU of one layer: 40,960 routed pairs + 4,096 shared rows), launched alone "
                               "on the stack's own per-layer inputs (8 layers walked), HIP events on its stream",
                     "flops_per_launch": head["gu_flops"], "avg_us": gum * 1e3,
                     "avg_us_range": [float(np.min(head["gu_ms"])) * 1e3, float(np.max(head["gu_ms"])) * 1e3],
                     "down": {"avg_us": float(np.median(head["dn_ms"])) * 1e3,
                              "tflops": head["dn_flops"] / float(np.median(head["dn_ms"])) / 1e9,
                              "frac": head["dn_flops"] / float(np.median(head["dn_ms"])) / 1e9 / MFMA_PEAK_TFLOPS}},
        "cpu_baseline": head.get("cpu"),
        "secondary": res_sec,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
