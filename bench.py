"""Benchmark of the 2-bit MoE layer on one MI355X.

Default workload (the headline metric's configuration): single-token decode
through one full-shape MoE layer -- hidden 2048, 512 experts, top-10 with
renormalised softmax, expert intermediate 704, one shared expert (704), 2-bit
blocks of 32 with fp16 scales, bf16 router and activations, Zipf(1.1) router
bias.  One step = one token through one layer (route, permute, expert FFN,
shared expert, combine).  48 independent layers are resident in HBM (33 GB of
2-bit experts, like the model's 48 layers) and consecutive steps walk through
them, so the expert bytes come from HBM and not from a warm 256 MB Infinity
Cache.

Also reported (secondary): the 16-token decode stack through the same 48
layers with the residual/RMSNorm/bf16 glue; one 32,768-token prefill layer
(grouped-GEMM path, MFMA roofline of its gate/up and down kernels); the
4,096-token 3-bit prefill through a 48-layer stack with uniform routing.

Output: one JSON line (see the keys below).  --gpus N with N > 1 exits: the
benchmark runs on one GPU.
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


def expert_bytes(s) -> int:
    per = lambda r, k: r * k * s.qbits // 8 + (r * k // 32) * 2  # noqa: E731
    return 2 * per(s.inter, s.hidden) + per(s.hidden, s.inter)


def shared_bytes(s) -> int:
    per = lambda r, k: r * k * s.qbits // 8 + (r * k // 32) * 2  # noqa: E731
    return 2 * per(s.shared_inter, s.hidden) + per(s.hidden, s.shared_inter) if s.shared_inter else 0


def build_layers(wl, n_layers, device, log):
    layers = []
    s = wl.shape
    t0 = time.time()
    for l in range(n_layers):
        w_r, bias = synth.router(wl, l, device)
        gate, up, down = synth.expert_weights(wl, l, device)
        arena = M.QArena(s.n_experts, s.hidden, s.inter, s.qbits, device)
        for m, w in enumerate((gate, up, down)):
            arena.quantize_from(m, w)
        del gate, up, down
        sw = synth.shared_weights(wl, l, device)
        sarena = M.QArena(1, s.hidden, s.shared_inter, s.qbits, device)
        for m, w in enumerate(sw):
            sarena.quantize_from(m, w[None])
        layers.append(M.QLayer(w_r, bias, arena, sarena))
        if (l + 1) % 12 == 0:
            torch.cuda.synchronize()
            log(f"built {l + 1}/{n_layers} layers ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    return layers


class DecodeSteps:
    """G consecutive single-token steps, step i = layer i of the resident
    stack with its own token, through moe_layer_forward (the fused decode
    layer: router GEMV, selection, gate/up GEMV, down GEMV + combine).
    Captured once in a HIP graph so the host launches nothing per step."""

    def __init__(self, s, layers, xs, device):
        self.s, self.layers, self.xs = s, layers, xs
        self.ws = M.alloc_workspace(s, 1, device=device)
        self.out = torch.empty(len(xs), 1, s.hidden, device=device)
        self.graph = None

    def eager(self):
        for i, (layer, x) in enumerate(zip(self.layers, self.xs)):
            M.layer_forward(x, layer, self.s, out=self.out[i], ws=self.ws)

    def capture(self):
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.eager()

    def replay(self):
        self.graph.replay()


class FfnState:
    """Inputs of moe_expert_ffn for one token-batch on one layer: routing,
    permutation and a workspace holding the slot table and activations."""

    def __init__(self, s, T, device, shape=None, algo="gemv"):
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
        self.so = torch.empty(T, s.hidden, device=device)

    def prepare(self, x, layer):
        M.route(x, layer, self.s, self.idx, self.w, ws=self.ws)
        M.permute(self.idx, self.T, self.s, self.counts, self.offsets, self.sp, self.pp, self.ws)
        self.run(x, layer, 0)

    def run(self, x, layer, flags):
        M.expert_ffn(x, layer, self.s, self.offsets, self.sp, self.y, self.so, algo=self.algo, ws=self.ws,
                     flags=flags)


def time_phase(states, xs, layers, skip, reps):
    """Average duration (ms) of one projection kernel launched alone through
    moe_expert_ffn(REUSE_PLAN | skip), walking the layers in turn.  The
    launches are captured back to back in one HIP graph (no host gap between
    them) and timed with HIP events on the capturing stream, so the average
    is the kernel's own duration plus the graph's inter-dispatch gap."""
    flags = M.FFN_REUSE_PLAN | skip
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st, x, layer in zip(states, xs, layers):
            st.run(x, layer, flags)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) / (reps * len(states))


def probe_gemv(s, layers, dev, log):
    """Gate/up and down GEMV kernels over every expert of a layer: 16 tokens,
    32 experts each, routed so that each of the 512 experts gets exactly one
    (token, rank) pair."""
    import dataclasses
    ps = dataclasses.replace(s, top_k=32)
    T = s.n_experts // 32
    xs = synth.tokens(synth.WORKLOADS["decode16"], dev, layer=777, n_tokens=T)
    sts = []
    n = min(8, len(layers))
    for l in range(n):
        st = FfnState(s, T, dev, shape=ps)
        st.offsets.copy_(torch.arange(s.n_experts + 1, dtype=torch.int32, device=dev))
        st.sp.copy_(torch.arange(s.n_experts, dtype=torch.int32, device=dev))
        st.run(xs, layers[l], 0)
        sts.append(st)
    torch.cuda.synchronize()
    gu = time_phase(sts, [xs] * n, layers[:n], M.FFN_SKIP_DOWN, reps=3)
    dn = time_phase(sts, [xs] * n, layers[:n], M.FFN_SKIP_GATEUP, reps=3)
    gu_b = (s.n_experts * expert_bytes(s) + shared_bytes(s)) * 2 // 3
    dn_b = (s.n_experts * expert_bytes(s) + shared_bytes(s)) // 3
    log(f"probe: gate/up {gu * 1e3:.1f} us {gu_b / gu / 1e6:.0f} GB/s; down {dn * 1e3:.1f} us {dn_b / dn / 1e6:.0f} GB/s")
    return {"what": "gate/up and down GEMV kernels alone over all 512 experts + shared of a layer "
                    "(16 tokens x 32 experts, one pair per expert)",
            "gateup": {"avg_us": gu * 1e3, "bytes": gu_b, "GBs": gu_b / gu / 1e6, "frac": gu_b / gu / 1e6 / HBM_PEAK_GBS},
            "down": {"avg_us": dn * 1e3, "bytes": dn_b, "GBs": dn_b / dn / 1e6, "frac": dn_b / dn / 1e6 / HBM_PEAK_GBS}}


MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 / bf16

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_gateup_decode1_traffic.txt")
TRAFFIC_SOURCES = ("ffn_gemv.hip", "common.h", "launch.h")


def source_digest() -> str:
    """SHA-256 of the kernel sources the traffic counters depend on, with
    // comments and blank lines removed (a comment edit does not change the
    code the counters measured)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "bit_quantized_expert_amd", "csrc", f)) as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch of the decode gate/up kernel from the committed
    FETCH_SIZE / WRITE_SIZE counter runs (scaled by the copy-kernel
    calibration), or None when the kernel source changed since they were
    taken."""
    import hashlib
    try:
        kv = {}
        for line in open(TRAFFIC_FILE):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if source_digest() != kv["source_sha256"]:
            return None
        return (float(kv["fetch_kib"]) * float(kv["fetch_scale"]) + float(kv["write_kib"]) * float(kv["write_scale"])) * 1024
    except (OSError, KeyError, ValueError):
        return None


def ffn_flops(s, T) -> tuple[int, int]:
    """Algorithmic flops of the gate/up and down projections for T tokens
    (routed pairs plus the shared expert)."""
    P = T * s.top_k
    gu = 2 * s.hidden * 2 * (P * s.inter + T * s.shared_inter)
    dn = 2 * s.hidden * (P * s.inter + T * s.shared_inter)
    return gu, dn


def decode_stack_bench(wl, s, layers, dev, log, steps):
    """wl.tokens tokens through the resident layers as a stack (residual +
    RMSNorm + bf16 glue between layers), captured as one HIP graph; the
    algorithmic bytes count each layer's distinct experts once."""
    T, L = wl.tokens, len(layers)
    r = torch.empty(T, s.hidden, device=dev)
    a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=dev)
    x0 = synth.tokens(wl, dev).float()
    ws = M.alloc_workspace(s, T, device=dev)
    idx = torch.empty(L, T, s.top_k, dtype=torch.int32, device=dev)

    def stack_pass():
        r.copy_(x0)
        M.rmsnorm_bf16(r, a)
        for l in range(L):
            M.layer_forward(a, layers[l], s, residual=r, next_in=a, topk_idx=idx[l], ws=ws)

    stack_pass()
    torch.cuda.synchronize()
    r_eager = r.clone()
    uniq = [int(torch.unique(idx[l]).numel()) for l in range(L)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack_pass()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(r, r_eager):
        raise SystemExit(f"{wl.name} stack graph replay differs from the eager stack")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g
    router_bytes = s.n_experts * s.hidden * 2
    nbytes = sum(u * expert_bytes(s) + shared_bytes(s) + router_bytes for u in uniq)
    log(f"{wl.name} stack: {ms:.3f} ms/step, {T / ms * 1e3:.0f} tok/s, {nbytes / ms / 1e6:.0f} GB/s, "
        f"unique experts/layer {np.mean(uniq):.1f}")
    return {"tokens": T, "tokens_per_s": T / ms * 1e3, "ms_per_step": ms, "layers": L,
            "achieved_GBs": nbytes / ms / 1e6, "hbm_frac": nbytes / ms / 1e6 / HBM_PEAK_GBS,
            "unique_experts_per_layer": float(np.mean(uniq))}


def prefill_bench(wl, layer, dev, log, reps=5):
    """One prefill layer (T tokens through route, permute, grouped-GEMM FFN,
    combine), and the grouped gate/up and down kernels launched alone."""
    s = wl.shape
    T = wl.tokens
    x = synth.tokens(wl, dev)
    ws = M.alloc_workspace(s, T, device=dev)
    out = torch.empty(T, s.hidden, device=dev)
    M.layer_forward(x, layer, s, out=out, ws=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        M.layer_forward(x, layer, s, out=out, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    layer_ms = e0.elapsed_time(e1) / reps
    del ws
    st = FfnState(s, T, dev, algo="grouped")
    st.prepare(x, layer)
    torch.cuda.synchronize()
    gu = time_phase([st], [x], [layer], M.FFN_SKIP_DOWN, reps=reps)
    dn = time_phase([st], [x], [layer], M.FFN_SKIP_GATEUP, reps=reps)
    used = int((st.counts > 0).sum().item())
    top = int(st.counts.max().item())
    del st
    gu_f, dn_f = ffn_flops(s, T)
    rt_f = 2 * T * s.hidden * s.n_experts
    tot = gu_f + dn_f + rt_f
    log(f"{wl.name}: layer {layer_ms:.3f} ms ({T / layer_ms * 1e3:.0f} tok/s, {tot / layer_ms / 1e9:.0f} TFLOP/s); "
        f"gate/up {gu:.3f} ms {gu_f / gu / 1e9:.0f} TFLOP/s; down {dn:.3f} ms {dn_f / dn / 1e9:.0f} TFLOP/s; "
        f"experts used {used}, largest {top} tokens")
    return {"tokens": T, "layer_ms": layer_ms, "tokens_per_s": T / layer_ms * 1e3,
            "layer_tflops": tot / layer_ms / 1e9, "layer_mfma_frac": tot / layer_ms / 1e9 / MFMA_PEAK_TFLOPS,
            "gateup": {"avg_ms": gu, "flops": gu_f, "tflops": gu_f / gu / 1e9,
                       "frac": gu_f / gu / 1e9 / MFMA_PEAK_TFLOPS},
            "down": {"avg_ms": dn, "flops": dn_f, "tflops": dn_f / dn / 1e9,
                     "frac": dn_f / dn / 1e9 / MFMA_PEAK_TFLOPS},
            "experts_used": used, "largest_expert_tokens": top}


def fourbit_bench(dev, log, n_layers=8, replays=40):
    """The 4-bit block variant (codes -8..7): the 4,096-token layer on the
    grouped GEMM, and single-token decode walking n_layers resident 4-bit
    layers (10 GB, far beyond the 256 MB Infinity Cache) in one graph."""
    wl = synth.WORKLOADS["prefill4"]
    s = wl.shape
    layers = build_layers(wl, n_layers, dev, log)
    pre = prefill_bench(wl, layers[0], dev, log)
    xs = [synth.tokens(wl, dev, layer=100 + i, n_tokens=1) for i in range(n_layers)]
    dec = DecodeSteps(s, layers, xs, dev)
    dec.eager()
    dec.capture()
    for _ in range(3):
        dec.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        dec.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (replays * n_layers) * 1e3
    nbytes = s.n_experts * s.hidden * 2 + s.top_k * expert_bytes(s) + shared_bytes(s)
    log(f"4-bit decode1: {us:.2f} us/layer, {nbytes / us / 1e3:.0f} GB/s")
    del dec, layers
    torch.cuda.empty_cache()
    return {"prefill4k_layer": pre,
            "decode1": {"avg_us": us, "tokens_per_s": 1e6 / us, "bytes": nbytes, "GBs": nbytes / us / 1e3,
                        "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS, "layers": n_layers}}


def prefill3_stack_bench(dev, log, n_layers, steps=2):
    """4,096 tokens through the 48-layer 3-bit stack (uniform routing), with
    the residual / RMSNorm / bf16 glue between layers."""
    wl = synth.WORKLOADS["prefill3"]
    s = wl.shape
    layers = build_layers(wl, n_layers, dev, log)
    T = wl.tokens
    x0 = synth.tokens(wl, dev).float()
    r = torch.empty(T, s.hidden, device=dev)
    a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device=dev)
    ws = M.alloc_workspace(s, T, device=dev)

    def step():
        r.copy_(x0)
        M.rmsnorm_bf16(r, a)
        for l in range(n_layers):
            M.layer_forward(a, layers[l], s, residual=r, next_in=a, ws=ws)

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    gu_f, dn_f = ffn_flops(s, T)
    tot = n_layers * (gu_f + dn_f + 2 * T * s.hidden * s.n_experts)
    wbytes = n_layers * (s.n_experts * expert_bytes(s) + shared_bytes(s) + s.n_experts * s.hidden * 2)
    log(f"prefill3 stack: {ms:.1f} ms/step ({T / ms * 1e3:.0f} tok/s, {tot / ms / 1e9:.0f} TFLOP/s, "
        f"weights {wbytes / ms / 1e6:.0f} GB/s)")
    del layers, ws
    torch.cuda.empty_cache()
    return {"tokens": T, "layers": n_layers, "ms_per_step": ms, "tokens_per_s": T / ms * 1e3,
            "tflops": tot / ms / 1e9, "mfma_frac": tot / ms / 1e9 / MFMA_PEAK_TFLOPS,
            "weight_GBs": wbytes / ms / 1e6}


def cpu_baseline(wl, layers_fp_seed, xs, n_sample, log):
    """The CPU oracle on a bounded sample: n_sample (token, layer) pairs of the
    same workload, timed on this host's cores."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas_threads = 1
    s = wl.shape
    total = 0.0
    for i in range(n_sample):
        l = i % layers_fp_seed
        w_r, bias = synth.router(wl, l, "cuda")
        x = xs[i].float().cpu().numpy().astype(np.float64)
        wr = w_r.float().cpu().numpy().astype(np.float64)
        b = bias.cpu().numpy().astype(np.float64)
        # which experts the token needs (selection by the oracle itself)
        idx = O.topk_select(O.router_logits(x, wr, b), s.top_k)[0]
        experts = {}
        for e in idx:
            g, u, d = synth.expert_weights(wl, l, "cuda", experts=slice(int(e), int(e) + 1))
            experts[int(e)] = O.QExpert.from_float(g[0].cpu().numpy(), u[0].cpu().numpy(), d[0].cpu().numpy(),
                                                   s.qbits)
        sw = synth.shared_weights(wl, l, "cuda")
        shared = O.QExpert.from_float(*(t.cpu().numpy() for t in sw), s.qbits)

        class Lazy:
            def __len__(self):
                return s.n_experts

            def __getitem__(self, e):
                return experts[int(e)]

        t0 = time.perf_counter()
        O.layer_forward(x, wr, b, Lazy(), shared, s.top_k)
        total += time.perf_counter() - t0
    log(f"cpu oracle: {n_sample} token-layers in {total:.2f}s")
    return {"value": n_sample / total, "unit": "tokens/s (one token through one layer)",
            "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{n_sample} single-token layer passes of the decode1 workload over {layers_fp_seed} "
                      f"layers (float64 numpy; dequantisation of the 11 touched experts included; "
                      f"quantisation of the inputs not timed; host os.cpu_count()={os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--stack-steps", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=128)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill3", action="store_true")
    ap.add_argument("--no-4bit", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy 10 times (scales the HBM byte counters)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1"}))
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

    wl = synth.WORKLOADS["decode1"]
    s = wl.shape
    layers = build_layers(wl, args.layers, dev, log)
    L = args.layers
    replays = max(1, args.steps // L)
    steps = replays * L
    xs = [synth.tokens(wl, dev, layer=i, n_tokens=1) for i in range(L)]
    dec = DecodeSteps(s, layers, xs, dev)
    dec.eager()
    torch.cuda.synchronize()
    eager_out = dec.out.clone()
    dec.capture()
    for _ in range(max(1, args.warmup // L)):
        dec.replay()
    torch.cuda.synchronize()
    if not torch.equal(dec.out, eager_out):
        raise SystemExit("graph replay differs from the eager layer")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(replays + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record()
    for r in range(replays):
        dec.replay()
        ev[r + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    ev_ms = [ev[r].elapsed_time(ev[r + 1]) / L for r in range(replays)]
    layer_ms = float(np.mean(ev_ms))
    # algorithmic bytes of one layer step: router weights + 10 routed experts (all distinct at T = 1) + shared
    router_bytes = s.n_experts * s.hidden * 2
    layer_bytes = router_bytes + s.top_k * expert_bytes(s) + shared_bytes(s)
    achieved = layer_bytes / (layer_ms * 1e-3) / 1e9
    log(f"decode1: {ms_per_step * 1e3:.2f} us/step (wall), {layer_ms * 1e3:.2f} us/step (events), "
        f"{achieved:.0f} GB/s")

    # the dominant kernel, alone: the gate/up dequant-GEMV of each layer's token, launched through
    # moe_expert_ffn with the phase flags (slot table and activations prepared beforehand, one
    # workspace per layer, layers walked in turn so the weights come from HBM)
    ffn = []
    for i in range(L):
        st = FfnState(s, 1, dev)
        st.prepare(xs[i], layers[i])
        ffn.append(st)
    torch.cuda.synchronize()
    gu_ms = time_phase(ffn, xs, layers, M.FFN_SKIP_DOWN, reps=max(1, replays // 2))
    dn_ms = time_phase(ffn, xs, layers, M.FFN_SKIP_GATEUP, reps=max(1, replays // 2))
    gu_bytes = (s.top_k * expert_bytes(s) + shared_bytes(s)) * 2 // 3
    dn_bytes = (s.top_k * expert_bytes(s) + shared_bytes(s)) // 3
    gu_gbs = gu_bytes / (gu_ms * 1e-3) / 1e9
    log(f"gate/up GEMV alone: {gu_ms * 1e3:.2f} us, {gu_gbs:.0f} GB/s; down GEMV alone: {dn_ms * 1e3:.2f} us, "
        f"{dn_bytes / dn_ms / 1e6:.0f} GB/s")
    del ffn

    # kernel probe (bandwidth regime): 16 tokens x top-32 = 512 pairs, one per expert, so the gate/up
    # kernel streams all 512 experts (+ the shared one) of a layer
    probe = probe_gemv(s, layers, dev, log)

    # secondary: 16-token decode, and the 4-token verify window (the token plus three drafts),
    # through the 48-layer stack, each as one graph
    stack16 = decode_stack_bench(synth.WORKLOADS["decode16"], s, layers, dev, log, args.stack_steps)
    stack4 = decode_stack_bench(synth.WORKLOADS["verify4"], s, layers, dev, log, args.stack_steps)

    # secondary: prefill workloads on the grouped-GEMM path
    prefill = prefill_bench(synth.WORKLOADS["prefill"], layers[0], dev, log)
    torch.cuda.empty_cache()
    prefill3 = None
    if not args.no_prefill3:
        prefill3 = prefill3_stack_bench(dev, log, args.layers)
        torch.cuda.empty_cache()
    fourbit = None
    if not args.no_4bit:
        fourbit = fourbit_bench(dev, log)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.layers, [synth.tokens(wl, dev, layer=1000 + i, n_tokens=1)
                                             for i in range(args.cpu_sample)], args.cpu_sample, log)

    res = {
        "metric": "MoE-layer tokens/s (single-token decode, one full-shape layer)",
        "value": 1e3 / ms_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 activations, 2-bit experts, fp16 MFMA / fp32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights quantised to 2-bit blocks, N(0,1) bf16 tokens)",
        "config": {"workload": "decode1: 1 token, hidden 2048, 512 experts, top-10, inter 704, shared 704, "
                               "2-bit/32-block fp16 scales, Zipf(1.1) router bias; 48 resident layers walked "
                               "in turn", "global_batch": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": gu_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gu_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     "kernel": "gemv_gateup_1tok_kernel<2, 64, unsigned short> (gate/up dequant-GEMV + SwiGLU, one "
                               "token, 10 routed + shared expert, slot table given), launched alone, HIP "
                               "events on its stream",
                     "bytes_per_launch": gu_bytes, "avg_us": gu_ms * 1e3,
                     "layer": {"avg_us": layer_ms * 1e3, "bytes": layer_bytes, "GBs": achieved},
                     "down_gemv": {"avg_us": dn_ms * 1e3, "bytes": dn_bytes, "GBs": dn_bytes / dn_ms / 1e6},
                     "probe": probe},
        "cpu_baseline": cpu,
        "secondary": {"prefill32k_layer": prefill, "prefill3_4k_stack": prefill3,
                      "decode16_stack": stack16, "verify4_stack": stack4, "four_bit": fourbit},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
