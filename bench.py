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
layers with the residual/RMSNorm/bf16 glue.

Output: one JSON line (see the keys below).  --gpus N with N > 1 exits: this
build runs on one GPU.
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


class Step:
    """One pass of the layer through the C ABI in its four steps (the same
    kernels moe_layer_forward runs), with HIP events around the expert FFN."""

    def __init__(self, s, T, device):
        self.s, self.T = s, T
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
        self.out = torch.empty(T, s.hidden, device=device)

    def __call__(self, x, layer, ev=None, residual=None, next_in=None):
        s, T = self.s, self.T
        M.route(x, layer, s, self.idx, self.w, ws=self.ws)
        M.permute(self.idx, T, s, self.counts, self.offsets, self.sp, self.pp, self.ws)
        if ev is not None:
            ev[0].record()
        M.expert_ffn(x, layer, s, self.offsets, self.sp, self.y, self.so, algo="gemv", ws=self.ws)
        if ev is not None:
            ev[1].record()
        M.combine(self.y, self.pp, self.w, self.so, T, s, out=self.out if residual is None else None,
                  residual=residual, next_in=next_in)


def unique_experts(step: Step) -> int:
    return int((step.counts > 0).sum().item())


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
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU"}))
        sys.exit(1)
    dev = "cuda:0"
    M.lib()

    wl = synth.WORKLOADS["decode1"]
    s = wl.shape
    layers = build_layers(wl, args.layers, dev, log)
    n_tot = args.warmup + args.steps
    xs = [synth.tokens(wl, dev, layer=i, n_tokens=1) for i in range(n_tot)]
    step = Step(s, 1, dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    for i in range(args.warmup):
        step(xs[i], layers[i % args.layers])
    torch.cuda.synchronize()
    uniq = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        j = args.warmup + i
        step(xs[j], layers[j % args.layers], ev=evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    # bytes of one FFN launch: the experts it reads (10 routed, all distinct at T=1) + the shared expert
    ffn_bytes = s.top_k * expert_bytes(s) + shared_bytes(s)
    achieved = ffn_bytes / (ffn_ms * 1e-3) / 1e9
    log(f"decode1: {ms_per_step * 1e3:.1f} us/step, expert FFN {ffn_ms * 1e3:.1f} us, {achieved:.0f} GB/s")

    # secondary: 16-token decode through the 48-layer stack
    T16 = 16
    st16 = Step(s, T16, dev)
    r = torch.empty(T16, s.hidden, device=dev)
    a = torch.empty(T16, s.hidden, dtype=torch.bfloat16, device=dev)
    x16 = synth.tokens(synth.WORKLOADS["decode16"], dev).float()
    uniq_bytes = []

    def stack_pass(count_unique=False):
        r.copy_(x16)
        M.rmsnorm_bf16(r, a)
        for l in range(args.layers):
            st16(a, layers[l], residual=r, next_in=a)
            if count_unique:
                uniq_bytes.append(unique_experts(st16))

    stack_pass(count_unique=True)
    for _ in range(2):
        stack_pass()
    torch.cuda.synchronize()
    ts = time.perf_counter()
    for _ in range(args.stack_steps):
        stack_pass()
    torch.cuda.synchronize()
    stack_ms = (time.perf_counter() - ts) * 1e3 / args.stack_steps
    stack_bytes = sum(u * expert_bytes(s) + shared_bytes(s) + s.n_experts * s.hidden * 2 for u in uniq_bytes)
    log(f"decode16 stack: {stack_ms:.3f} ms/step, {T16 / stack_ms * 1e3:.0f} tok/s, "
        f"{stack_bytes / stack_ms / 1e6:.0f} GB/s, unique experts/layer {np.mean(uniq_bytes):.1f}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.layers, xs, args.cpu_sample, log)

    res = {
        "metric": "MoE-layer tokens/s (single-token decode, one full-shape layer)",
        "value": 1e3 / ms_per_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
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
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "expert FFN step (plan + gate/up + down kernels), HIP events on its stream",
                     "bytes_per_launch": ffn_bytes, "avg_us": ffn_ms * 1e3},
        "cpu_baseline": cpu,
        "secondary": {"decode16_stack": {"tokens_per_s": T16 / stack_ms * 1e3, "ms_per_step": stack_ms,
                                         "layers": args.layers, "achieved_GBs": stack_bytes / stack_ms / 1e6,
                                         "hbm_frac": stack_bytes / stack_ms / 1e6 / HBM_PEAK_GBS,
                                         "unique_experts_per_layer": float(np.mean(uniq_bytes))}},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
