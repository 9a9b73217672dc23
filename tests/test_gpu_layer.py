"""GPU parity of the expert FFN and the whole layer against the CPU oracle,
on the tiny and full decode shapes and on ragged shapes."""

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


def _run_layer(M, dl, x, algo="auto"):
    s = dl.s
    T = x.shape[0]
    ws = M.alloc_workspace(s, T, algo=algo)
    out = torch.empty(T, s.hidden, device="cuda")
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    M.layer_forward(x, dl.q, s, out=out, topk_idx=idx, topk_w=w, algo=algo, ws=ws)
    logits = torch.empty(T, s.n_experts, device="cuda")
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    M.route(x, dl.q, s, idx2, w2, logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2)
    return out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), logits.cpu().numpy()


def _check_layer(M, dl, x, algo="auto"):
    out, idx, w, logits = _run_layer(M, dl, x, algo)
    xn = x_to_numpy(x)
    ref = dl.oracle_forward(xn, idx=idx, return_all=True)
    check_route_protocol(logits, idx, w, ref["logits"], dl.s.top_k)
    return assert_close_output(out, ref["out"], f"{dl.wl.name} T={x.shape[0]} {algo}")


def _M():
    import bit_quantized_expert_amd as M
    M.lib()
    return M


RAGGED = [
    # name, H, I, E, k, Is, qbits, T, dtype
    ("r1", 96, 96, 5, 3, 64, 2, 37, torch.bfloat16),
    ("r2", 96, 96, 5, 3, 64, 3, 37, torch.float32),
    ("r3", 128, 160, 12, 4, 0, 2, 21, torch.bfloat16),
    ("r4", 64, 32, 8, 2, 32, 3, 4, torch.float32),
    ("r5", 256, 192, 33, 8, 96, 3, 17, torch.bfloat16),
    # 2..16 tokens touching few experts (reduction split over the waves): 32-weight units, 3-bit
    # with fp32 tokens, hidden above 2048 (several load batches per class)
    ("k1", 96, 96, 40, 2, 64, 2, 5, torch.bfloat16),
    ("k2", 256, 192, 64, 3, 96, 3, 9, torch.float32),
    ("k3", 2304, 96, 64, 2, 96, 2, 12, torch.bfloat16),
    # 2..16 tokens touching most experts (persistent gate/up and down kernels)
    ("p1", 1024, 128, 8, 4, 128, 2, 16, torch.bfloat16),
    ("p2", 2048, 704, 16, 8, 704, 3, 12, torch.float32),
    ("p3", 1024, 256, 4, 2, 0, 2, 3, torch.bfloat16),
    # single-token layers (the fused one-token path), 64- and 32-weight units
    ("s1", 96, 96, 5, 3, 64, 2, 1, torch.bfloat16),
    ("s2", 64, 32, 8, 2, 32, 3, 1, torch.float32),
    ("s3", 128, 160, 12, 4, 0, 2, 1, torch.bfloat16),
    ("s4", 256, 192, 33, 8, 96, 3, 1, torch.bfloat16),
    ("s5", 192, 128, 40, 32, 64, 2, 1, torch.bfloat16),
    # one token whose 33 (or 9) h rows are more than the single-token down + combine kernel can
    # stage in LDS: the layer takes the multi-token decode kernels instead
    ("s6", 64, 2560, 40, 32, 64, 2, 1, torch.bfloat16),
    ("s7", 64, 64, 16, 8, 20480, 3, 1, torch.bfloat16),
    # the 4-bit format on each decode path: per-slot kernels (37 tokens; hidden not a multiple
    # of 1024), the single-token fused path (32-weight down units), the persistent kernels with
    # the in-kernel selection (bf16 and fp32 tokens)
    ("q1", 96, 96, 5, 3, 64, 4, 37, torch.bfloat16),
    ("q2", 256, 192, 33, 8, 96, 4, 1, torch.bfloat16),
    ("q3", 1024, 128, 8, 4, 128, 4, 16, torch.bfloat16),
    ("q4", 2048, 704, 16, 8, 704, 4, 5, torch.float32),
    ("q5", 128, 160, 12, 4, 0, 4, 9, torch.bfloat16),
    # the largest expert count and top-k the library takes (4096, 32): selection over 64 keys per
    # lane, one token through the small-batch path
    ("m1", 64, 32, 4096, 32, 32, 2, 1, torch.bfloat16),
    ("m2", 64, 32, 4096, 32, 32, 3, 16, torch.bfloat16),
]


def test_tiny_layer():
    M = _M()
    dl = _layer(synth.WORKLOADS["tiny"])
    x = synth.tokens(dl.wl, "cuda")
    _check_layer(M, dl, x, "gemv")


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_layer(case):
    M = _M()
    name, H, I, E, k, Is, qb, T, dt = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=11, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda")
    _check_layer(M, dl, x, "gemv")


# fp16 activations (MOE_F16): every path's activation load and the router's
# fp32 path; the oracle is fed the same fp16 values
F16_CASES = [
    # name, H, I, E, k, Is, qbits, T, algo
    ("f1", 96, 96, 5, 3, 64, 2, 1, "auto"),       # single-token fused layer
    ("f2", 256, 192, 33, 8, 96, 3, 1, "gemv"),    # single-token kernels, step by step
    ("f3", 1024, 128, 8, 4, 128, 2, 16, "auto"),  # persistent gate/up with the selection inside
    ("f4", 96, 96, 5, 3, 64, 3, 12, "gemv"),      # multi-token GEMV
    ("f5", 128, 160, 12, 4, 0, 2, 37, "grouped"), # grouped GEMM (the fp16 copy kernel)
    ("f6", 2048, 704, 16, 8, 704, 4, 40, "grouped"),
    ("f7", 160, 96, 3, 1, 32, 4, 2100, "grouped"),  # more than 2048 pairs: the fused selection pass
]


@pytest.mark.parametrize("case", F16_CASES, ids=[c[0] for c in F16_CASES])
def test_fp16_activations(case):
    M = _M()
    name, H, I, E, k, Is, qb, T, algo = case
    wl = synth.custom(name, H, I, E, k, Is, qb, T, seed=13, act_dtype=torch.bfloat16, zipf_bias=True)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda").half()
    _check_layer(M, dl, x, algo)


def test_decode1_full_shape():
    M = _M()
    dl = _layer(synth.WORKLOADS["decode1"])
    for seed_layer in range(3):
        x = synth.tokens(dl.wl, "cuda", layer=seed_layer)
        _check_layer(M, dl, x, "gemv")


@pytest.mark.parametrize("T", [1, 4])
def test_full_shape_4bit(T):
    """One full-shape layer (hidden 2048, 512 experts, top-10, inter 704) in
    the 4-bit format: the single-token path and the verify-window path."""
    M = _M()
    wl = synth.custom("full4", 2048, 704, 512, 10, 704, 4, T, seed=31, act_dtype=torch.bfloat16, zipf_bias=True)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda")
    _check_layer(M, dl, x, "gemv")


@pytest.mark.parametrize("T", [9, 16])
def test_persistent_gateup_many_items(T):
    """Uniform routing of 9 or 16 tokens over 512 experts: about 1,500 (slot,
    64-row block) items of the persistent gate/up kernel with the selection
    inside, several per item group of its 16-wave workgroups, the two groups
    of some workgroups with different counts."""
    M = _M()
    wl = synth.custom(f"u{T}", 1024, 704, 512, 10, 704, 2, T, seed=13, act_dtype=torch.bfloat16, zipf_bias=False)
    dl = _layer(wl)
    x = synth.tokens(wl, "cuda")
    _check_layer(M, dl, x, "gemv")


def test_decode16_layer_and_batch_invariance():
    M = _M()
    wl = synth.WORKLOADS["decode16"]
    dl = _layer(wl, layer=0)
    x = synth.tokens(wl, "cuda")
    _check_layer(M, dl, x, "gemv")
    out_all, idx_all, _, _ = _run_layer(M, dl, x)
    for t in (0, 7, 15):
        out_t, idx_t, _, _ = _run_layer(M, dl, x[t:t + 1].contiguous())
        assert np.array_equal(idx_t[0], idx_all[t])
        assert np.array_equal(out_t[0], out_all[t]), f"token {t} depends on the rest of the batch"
    # every batch size of the multi-token kernels: the first T tokens alone
    for T in range(2, 16):
        out_T, idx_T, _, _ = _run_layer(M, dl, x[:T].contiguous())
        assert np.array_equal(idx_T, idx_all[:T])
        assert np.array_equal(out_T, out_all[:T]), f"batch of {T} differs from the same tokens among 16"


@pytest.mark.parametrize("name", ["tiny", "decode16", "decode1"])
def test_stepwise_api_matches_layer_forward(name):
    """The four single-step entry points (separate kernels) and the fused
    decode layer give the same bits."""
    M = _M()
    dl = _layer(synth.WORKLOADS[name])
    s = dl.s
    x = synth.tokens(dl.wl, "cuda")
    T = x.shape[0]
    ws = M.alloc_workspace(s, T)
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    M.route(x, dl.q, s, idx, w, ws=ws)
    counts = torch.empty(s.n_experts, dtype=torch.int32, device="cuda")
    offsets = torch.empty(s.n_experts + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * s.top_k, dtype=torch.int32, device="cuda")
    pp = torch.empty_like(sp)
    M.permute(idx, T, s, counts, offsets, sp, pp, ws)
    y = torch.empty(T * s.top_k, s.hidden, device="cuda")
    so = torch.empty(T, s.hidden, device="cuda")
    M.expert_ffn(x, dl.q, s, offsets, sp, y, so, ws=ws)
    out = torch.empty(T, s.hidden, device="cuda")
    M.combine(y, pp, w, so, T, s, out=out)
    out2, _, _, _ = _run_layer(M, dl, x)
    assert np.array_equal(out.cpu().numpy(), out2)
    # y_sorted and shared_out individually against the oracle
    ref = dl.oracle_forward(x_to_numpy(x), idx=idx.cpu().numpy(), return_all=True)
    assert_close_output(y.cpu().numpy(), ref["y"], "y_sorted")
    assert_close_output(so.cpu().numpy(), ref["shared"], "shared_out")


def test_single_token_glue_matches_batch():
    """One token through the layer with the residual + RMSNorm + bf16 glue
    (the single-token path) gives the same out, residual and next input bits
    as the same token inside a 16-token batch."""
    M = _M()
    wl = synth.WORKLOADS["decode16"]
    s = wl.shape
    dl = _layer(wl, layer=0)
    x = synth.tokens(wl, "cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    r0 = torch.randn(16, s.hidden, device="cuda", generator=g)

    def run(xx, rr):
        T = xx.shape[0]
        ws = M.alloc_workspace(s, T)
        out = torch.empty(T, s.hidden, device="cuda")
        a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device="cuda")
        idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, s.top_k, device="cuda")
        M.layer_forward(xx, dl.q, s, out=out, residual=rr, next_in=a, topk_idx=idx, topk_w=w, ws=ws)
        torch.cuda.synchronize()
        return out, a, idx, w

    r_all = r0.clone()
    out_all, a_all, idx_all, w_all = run(x, r_all)
    for t in (0, 9, 15):
        r_t = r0[t:t + 1].clone()
        out_t, a_t, idx_t, w_t = run(x[t:t + 1].contiguous(), r_t)
        assert torch.equal(idx_t[0], idx_all[t]) and torch.equal(w_t[0], w_all[t])
        assert torch.equal(out_t[0], out_all[t]), f"token {t}: out"
        assert torch.equal(r_t[0], r_all[t]), f"token {t}: residual"
        assert torch.equal(a_t[0], a_all[t]), f"token {t}: next input"


def test_zero_tokens_is_a_noop():
    M = _M()
    dl = _layer(synth.WORKLOADS["tiny"])
    x = torch.empty(0, dl.s.hidden, device="cuda")
    out = torch.empty(0, dl.s.hidden, device="cuda")
    M.layer_forward(x, dl.q, dl.s, out=out, ws=None)


@pytest.mark.parametrize("name", ["decode16", "verify4"])
def test_decode_stack_teacher_forced(name):
    """Three stacked layers of the 16-token decode workload (and of the
    4-token verify window) through the fused residual + RMSNorm + bf16 glue.  Each layer is checked against the oracle
    fed the GPU's own bf16 activation (teacher forcing); the residual update is
    exact fp32 addition; the next activation matches the oracle's RMSNorm +
    bf16 rounding of the GPU residual except at rounding boundaries."""
    from oracle import moe_oracle as O
    M = _M()
    wl = synth.WORKLOADS[name]
    s = wl.shape
    T = wl.tokens
    x0 = synth.tokens(wl, "cuda").float()
    r = x0.clone()
    a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device="cuda")
    M.rmsnorm_bf16(r, a)
    want_a0 = O.rmsnorm_bf16(x0.cpu().numpy().astype(np.float64))
    assert np.mean(a.float().cpu().numpy() != want_a0) < 1e-3
    ws = M.alloc_workspace(s, T)
    for l in range(3):
        dl = _layer(wl, layer=l)
        a_in = a.clone()
        r_before = r.clone()
        out = torch.empty(T, s.hidden, device="cuda")
        idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
        M.layer_forward(a, dl.q, s, out=out, residual=r, next_in=a, topk_idx=idx, ws=ws)
        torch.cuda.synchronize()
        ref = dl.oracle_forward(x_to_numpy(a_in), idx=idx.cpu().numpy())
        assert_close_output(out.cpu().numpy(), ref, f"stack layer {l}")
        assert torch.equal(r, r_before + out)
        want_a = O.rmsnorm_bf16(r.cpu().numpy().astype(np.float64))
        got_a = a.float().cpu().numpy()
        diff = got_a != want_a
        assert np.mean(diff) < 1e-3, f"layer {l}: {diff.sum()} bf16 activations differ"
        # where they differ it is by one bf16 step
        if diff.any():
            rel = np.abs(got_a[diff] - want_a[diff]) / np.abs(want_a[diff])
            assert np.all(rel <= 2.0 ** -7 * 1.01)


def test_graph_replay_matches_eager():
    """The fused decode layer captured in a HIP graph: every replay, with
    eager work and synchronisations between replays, equals the eager result
    (outputs, indices and the stack glue)."""
    M = _M()
    wl = synth.WORKLOADS["decode16"]
    s = wl.shape
    T = wl.tokens
    dl = _layer(wl, layer=0)
    x0 = synth.tokens(wl, "cuda").float()
    ws = M.alloc_workspace(s, T)
    r = torch.empty(T, s.hidden, device="cuda")
    a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, s.hidden, device="cuda")
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")

    def step():
        r.copy_(x0)
        M.rmsnorm_bf16(r, a)
        M.layer_forward(a, dl.q, s, out=out, residual=r, next_in=a, topk_idx=idx, ws=ws)

    step()
    torch.cuda.synchronize()
    want = (out.clone(), r.clone(), a.clone(), idx.clone())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        out.zero_(); r.zero_(); a.zero_(); idx.zero_()
        M.layer_forward(synth.tokens(wl, "cuda", layer=rep + 1), dl.q, s, out=torch.empty_like(out), ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, w_ in zip((out, r, a, idx), want):
            assert torch.equal(got, w_), f"replay {rep} differs"


TAIL = [
    # name, H, I, E, k, Is, qbits, T, dtype: full shape (single-token kernels, in-kernel selection of the
    # persistent gate/up kernel), and ragged shapes on the one-workgroup selection kernel
    ("full", 2048, 704, 512, 10, 704, 2, None, torch.bfloat16),
    ("r12", 96, 96, 40, 12, 64, 3, None, torch.bfloat16),
    ("e1k", 64, 32, 1024, 16, 32, 2, None, torch.float32),
]


@pytest.mark.parametrize("case", TAIL, ids=[c[0] for c in TAIL])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_route_tail_skip(case, T):
    """The opt-in route tail skip of a verify window against the oracle's
    rule (an expert no token ranks 0..6 adds nothing): the selection and
    weights are those of the exact layer, the output is the oracle's layer
    with the same experts dropped."""
    from oracle import moe_oracle as O
    M = _M()
    name, H, I, E, k, Is, qb, _, dt = case
    wl = synth.custom(f"tail_{name}", H, I, E, k, Is, qb, T, seed=41, act_dtype=dt, zipf_bias=True)
    dl = _layer(wl)
    s = dl.s
    x = synth.tokens(wl, "cuda", n_tokens=T, layer=T)
    res = {}
    for flags in (0, M.ROUTE_TAIL_SKIP):
        out = torch.empty(T, s.hidden, device="cuda")
        idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
        w = torch.empty(T, s.top_k, device="cuda")
        M.layer_forward(x, dl.q, s, out=out, topk_idx=idx, topk_w=w, ws=M.alloc_workspace(s, T), flags=flags)
        torch.cuda.synchronize()
        res[flags] = (out.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy())
    (o0, i0, w0), (o1, i1, w1) = res[0], res[M.ROUTE_TAIL_SKIP]
    assert np.array_equal(i0, i1) and np.array_equal(w0, w1)
    wr, b = dl.oracle_router()
    for e in np.unique(i1):
        dl.oracle_expert(int(e))
    want = O.layer_forward(x_to_numpy(x), wr, b, dl.oracle_experts(), dl.oracle_shared(), k, idx=i1, tail_skip=7)
    assert_close_output(o1, want, f"{name} T={T} tail skip")
    keep = O.tail_skip_keep(i1, 7)
    if not keep.all():  # something was dropped: the output moved off the exact layer
        assert not np.array_equal(o0, o1)
    else:
        assert np.array_equal(o0, o1)


def test_route_tail_skip_no_effect_and_refusals():
    """No tail (top-k <= 7) or more than a window of tokens: the option changes
    no bit.  Forced onto the grouped GEMM at a window's size it is refused."""
    M = _M()
    for (H, I, E, k, Is, T) in [(96, 96, 40, 7, 64, 3), (2048, 704, 512, 10, 704, 5), (2048, 704, 512, 10, 704, 16)]:
        wl = synth.custom(f"tnone{k}_{T}", H, I, E, k, Is, 2, T, seed=43, act_dtype=torch.bfloat16, zipf_bias=True)
        dl = _layer(wl)
        s = dl.s
        x = synth.tokens(wl, "cuda")
        outs = []
        for flags in (0, M.ROUTE_TAIL_SKIP):
            out = torch.empty(T, s.hidden, device="cuda")
            M.layer_forward(x, dl.q, s, out=out, ws=M.alloc_workspace(s, T), flags=flags)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy())
        assert np.array_equal(outs[0], outs[1]), (k, T)
    x4 = x[:4].contiguous()
    with pytest.raises(M.MoeError) as ei:
        M.layer_forward(x4, dl.q, s, out=torch.empty(4, s.hidden, device="cuda"), algo="grouped",
                        ws=M.alloc_workspace(s, 4, algo="grouped"), flags=M.ROUTE_TAIL_SKIP)
    assert ei.value.status == -2
