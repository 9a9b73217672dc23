"""GPU parity of the grouped-GEMM (prefill) path against the CPU oracle:
ragged shapes, agreement with the GEMV path, and the full-size prefill
workloads on sampled tokens (every token is independent of the others, so
the oracle computes a sample of rows one by one)."""

import numpy as np
import pytest
import torch

from bit_quantized_expert_amd import synth
from tests.helpers import DeviceLayer, assert_close_output, check_route_protocol, x_to_numpy

pytestmark = pytest.mark.gpu

_CACHE = {}


def _layer(wl, layer=0):
    key = (wl, layer)
    if key not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[key] = DeviceLayer(wl, layer)
    return _CACHE[key]


def _M():
    import bit_quantized_expert_amd as M
    M.lib()
    return M


def _forward(M, dl, x, algo):
    s = dl.s
    T = x.shape[0]
    ws = M.alloc_workspace(s, T, algo=algo)
    out = torch.empty(T, s.hidden, device="cuda")
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    M.layer_forward(x, dl.q, s, out=out, topk_idx=idx, topk_w=w, algo=algo, ws=ws)
    torch.cuda.synchronize()
    del ws
    return out, idx, w


RAGGED = [
    # name, H, I, E, k, Is, qbits, T, dtype
    ("g1", 96, 96, 5, 3, 64, 2, 37, torch.bfloat16),
    ("g2", 96, 96, 5, 3, 64, 3, 37, torch.float32),
    ("g3", 128, 160, 12, 4, 0, 2, 300, torch.bfloat16),
    ("g4", 64, 32, 8, 2, 32, 3, 4, torch.float32),
    ("g5", 256, 192, 33, 8, 96, 3, 517, torch.bfloat16),
    ("g6", 192, 320, 7, 2, 128, 2, 1, torch.bfloat16),
    # segments of at least one 128-row tile per expert on average (the wide-tile kernel),
    # with odd block counts along K (96 = 3 blocks) and partial column tiles
    ("w1", 96, 96, 2, 1, 64, 2, 300, torch.bfloat16),
    ("w2", 160, 96, 3, 2, 32, 3, 400, torch.float32),
    ("w3", 256, 192, 4, 2, 0, 2, 600, torch.bfloat16),
    ("w4", 2048, 704, 4, 2, 704, 3, 520, torch.bfloat16),
    # ~90 rows per expert or fewer on average (96-row tiles), Zipf-skewed so that some segments span
    # several tiles with a ragged last one
    ("b1", 128, 96, 16, 2, 64, 2, 700, torch.bfloat16),
    ("b2", 256, 192, 24, 3, 0, 3, 680, torch.float32),
    # K a multiple of 128 in both projections (no half step), and hidden % 128 == 64 (a half
    # step in gate/up)
    ("k1", 128, 256, 6, 2, 128, 2, 300, torch.bfloat16),
    ("k2", 256, 128, 9, 3, 0, 3, 333, torch.float32),
    ("k3", 320, 128, 5, 2, 256, 3, 250, torch.bfloat16),
    # the 4-bit format: 96-row tiles with fp32 tokens, 128-row tiles with the down half step,
    # K not a multiple of 64
    ("q6", 256, 192, 24, 3, 96, 4, 680, torch.float32),
    ("q7", 2048, 704, 4, 2, 704, 4, 520, torch.bfloat16),
    ("q8", 96, 96, 5, 3, 64, 4, 37, torch.bfloat16),
    # the largest expert count and top-k (4096, 32)
    ("m3", 64, 32, 4096, 32, 32, 2, 40, torch.bfloat16),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_grouped_ragged_layer(case):
    M = _M()
    name, H, I, E, k, Is, qb, T, dt = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=21, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda")
    out, idx, w = _forward(M, dl, x, "grouped")
    ref = dl.oracle_forward(x_to_numpy(x), idx=idx.cpu().numpy())
    assert_close_output(out.cpu().numpy(), ref, f"{name} grouped")


# More than 2048 pairs: the layer's top-k, permutation, plan and fp16 copy of x
# run as one selection pass over 16-token chunks (ragged last chunks, the
# smallest and largest expert counts and top-k, hidden beyond 2048 groups per
# chunk); its selection must equal the stand-alone route's bit for bit
FUSED = [
    # name, H, I, E, k, Is, qbits, T, dtype
    ("v1", 96, 96, 5, 3, 64, 2, 1001, torch.bfloat16),
    ("v2", 128, 160, 12, 4, 0, 3, 777, torch.float32),
    ("v3", 64, 32, 4096, 32, 32, 2, 100, torch.bfloat16),
    ("v4", 160, 96, 3, 1, 32, 4, 2100, torch.bfloat16),
    ("v5", 2304, 96, 64, 2, 96, 2, 1030, torch.bfloat16),
]


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_grouped_fused_selection(case):
    M = _M()
    name, H, I, E, k, Is, qb, T, dt = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=23, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    s = dl.s
    x = synth.tokens(wl, "cuda")
    out, idx, w = _forward(M, dl, x, "grouped")
    logits = torch.empty(T, E, device="cuda")
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    M.route(x, dl.q, s, idx2, w2, logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    ref = dl.oracle_forward(x_to_numpy(x), idx=idx.cpu().numpy(), return_all=True)
    check_route_protocol(logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), ref["logits"], k)
    assert_close_output(out.cpu().numpy(), ref["out"], f"{name} grouped, fused selection")


def test_tiny_grouped():
    M = _M()
    dl = _layer(synth.WORKLOADS["tiny"])
    x = synth.tokens(dl.wl, "cuda")
    out, idx, w = _forward(M, dl, x, "grouped")
    ref = dl.oracle_forward(x_to_numpy(x), idx=idx.cpu().numpy())
    assert_close_output(out.cpu().numpy(), ref, "tiny grouped")


def test_grouped_agrees_with_gemv_decode16():
    """Both expert-FFN algorithms on the same 16-token batch: same routing,
    outputs within the fp32-accumulation tolerance of each other."""
    M = _M()
    dl = _layer(synth.WORKLOADS["decode16"])
    x = synth.tokens(dl.wl, "cuda")
    og, ig, _ = _forward(M, dl, x, "grouped")
    ov, iv, _ = _forward(M, dl, x, "gemv")
    assert torch.equal(ig, iv)
    assert_close_output(og.cpu().numpy(), ov.cpu().numpy().astype(np.float64), "grouped vs gemv")
    ref = dl.oracle_forward(x_to_numpy(x), idx=ig.cpu().numpy())
    assert_close_output(og.cpu().numpy(), ref, "decode16 grouped")


def _sampled_check(M, wl, n_sample, seed):
    dl = _layer(wl)
    s = dl.s
    x = synth.tokens(wl, "cuda")
    T = x.shape[0]
    out, idx, w = _forward(M, dl, x, "auto")
    logits = torch.empty(T, s.n_experts, device="cuda")
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    M.route(x, dl.q, s, idx2, w2, logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    rng = np.random.default_rng(seed)
    rows = np.sort(np.concatenate([[0, T - 1], rng.choice(np.arange(1, T - 1), n_sample - 2, replace=False)]))
    xs = x_to_numpy(x[torch.from_numpy(rows).cuda()])
    ref = dl.oracle_forward(xs, idx=idx.cpu().numpy()[rows], return_all=True)
    check_route_protocol(logits.cpu().numpy()[rows], idx.cpu().numpy()[rows], w.cpu().numpy()[rows],
                         ref["logits"], s.top_k)
    assert_close_output(out.cpu().numpy()[rows], ref["out"], f"{wl.name} sampled")
    # every row is finite, and rows are not all equal (the whole batch was computed)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    assert np.std(o[:, 0]) > 0


def test_prefill_32k_sampled():
    """32,768-token prefill of one full-shape 2-bit layer (Zipf-skewed
    routing: one expert takes almost every token), grouped GEMM path."""
    _sampled_check(_M(), synth.WORKLOADS["prefill"], 24, seed=5)


def test_prefill3_4k_sampled():
    """4,096-token prefill of one full-shape 3-bit layer, uniform routing."""
    _sampled_check(_M(), synth.WORKLOADS["prefill3"], 24, seed=6)


def test_prefill4_4k_sampled():
    """4,096-token prefill of one full-shape 4-bit layer, uniform routing."""
    _sampled_check(_M(), synth.WORKLOADS["prefill4"], 24, seed=7)


@pytest.mark.parametrize("case", [("w3", 256, 192, 4, 2, 0, 2, 600, torch.bfloat16),
                                  ("q6", 256, 192, 24, 3, 96, 4, 680, torch.float32)], ids=["no_shared", "shared"])
def test_grouped_stack_glue(case):
    """The grouped-GEMM layer with the stack glue (residual add, RMSNorm and
    bf16 next input, no `out`), with and without a shared expert: the residual
    update equals the layer output bit for bit, and the next input is the
    oracle's RMSNorm + bf16 rounding of the GPU residual except at rounding
    boundaries."""
    from oracle import moe_oracle as O
    M = _M()
    name, H, I, E, k, Is, qb, T, dt = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=23, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    s = dl.s
    x = synth.tokens(wl, "cuda")
    out, _, _ = _forward(M, dl, x, "grouped")
    r0 = torch.randn(T, s.hidden, device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    r = r0.clone()
    a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device="cuda")
    ws = M.alloc_workspace(s, T, algo="grouped")
    M.layer_forward(x, dl.q, s, residual=r, next_in=a, algo="grouped", ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(r, r0 + out)
    want_a = O.rmsnorm_bf16(r.cpu().numpy().astype(np.float64))
    diff = a.float().cpu().numpy() != want_a
    assert np.mean(diff) < 1e-3


def _stepwise(M, dl, x, algo):
    """route -> permute -> expert_ffn (fp32 y_sorted, shared_out) -> combine,
    each through its own entry point."""
    s = dl.s
    T = x.shape[0]
    ws = M.alloc_workspace(s, T, algo=algo)
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    M.route(x, dl.q, s, idx, w, ws=ws)
    counts = torch.empty(s.n_experts, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * s.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    M.permute(idx, T, s, counts, offsets, sp, pp, ws)
    y = torch.empty(T * s.top_k, s.hidden, device="cuda")
    so = torch.empty(T, s.hidden, device="cuda") if s.shared_inter else None
    M.expert_ffn(x, dl.q, s, offsets, sp, y, so, algo=algo, ws=ws)
    out = torch.empty(T, s.hidden, device="cuda")
    M.combine(y, pp, w, so, T, s, out=out)
    torch.cuda.synchronize()
    return idx, w, offsets, sp, pp, y, so, out


@pytest.mark.parametrize("case", [c for c in RAGGED if c[0] in ("g3", "g5", "w2", "w4", "b1", "k3", "q6", "m3")],
                         ids=lambda c: c[0])
def test_grouped_expert_ffn_standalone(case):
    """moe_expert_ffn with the grouped GEMM writes fp32 y_sorted and
    shared_out (not the fp16 hand-off of the layer): every row against the
    oracle's expert outputs in sorted order and its shared expert, and the
    combine of them against the oracle layer."""
    M = _M()
    name, H, I, E, k, Is, qb, T, dt = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=27, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda")
    idx, w, offsets, sp, pp, y, so, out = _stepwise(M, dl, x, "grouped")
    ref = dl.oracle_forward(x_to_numpy(x), idx=idx.cpu().numpy(), return_all=True)
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(sp.cpu().numpy(), ref["sorted_pair"])
    assert_close_output(y.cpu().numpy(), ref["y"], f"{name} y_sorted")
    if so is not None:
        assert_close_output(so.cpu().numpy(), ref["shared"], f"{name} shared_out")
    assert_close_output(out.cpu().numpy(), ref["out"], f"{name} combine")


def test_grouped_expert_ffn_standalone_4k_sampled():
    """The same at the 3-bit 4,096-token layer: a sample of sorted positions
    (first and last of a few experts, random others) and of shared-expert
    rows, each computed by the oracle on its own."""
    from oracle import moe_oracle as O
    M = _M()
    wl = synth.WORKLOADS["prefill3"]
    dl = _layer(wl)
    s = dl.s
    x = synth.tokens(wl, "cuda")
    idx, w, offsets, sp, pp, y, so, out = _stepwise(M, dl, x, "grouped")
    off = offsets.cpu().numpy()
    spn = sp.cpu().numpy()
    rng = np.random.default_rng(9)
    experts = rng.choice(s.n_experts, 6, replace=False)
    pos = [p for e in experts for p in (off[e], off[e + 1] - 1) if off[e + 1] > off[e]]
    pos = np.unique(np.concatenate([pos, rng.choice(len(spn), 10, replace=False)]))
    xn = x_to_numpy(x)
    got = y[torch.from_numpy(pos).cuda()].cpu().numpy()
    want = np.zeros_like(got, dtype=np.float64)
    for i, p in enumerate(pos):
        e = int(np.searchsorted(off, p, side="right") - 1)
        t = spn[p] // s.top_k
        want[i] = O.swiglu(xn[t:t + 1], *dl.oracle_expert(e).dense())[0]
    assert_close_output(got, want, "4k y_sorted sampled")
    rows = np.array([0, 1, 2047, 4095])
    want_s = O.swiglu(xn[rows], *dl.oracle_shared().dense())
    assert_close_output(so[torch.from_numpy(rows).cuda()].cpu().numpy(), want_s, "4k shared_out sampled")
