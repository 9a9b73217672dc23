"""GPU parity of the single-step kernels against the CPU oracle: quantiser
and dequantiser (bit-exact), router (near-tie protocol), permutation
(bit-exact)."""

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from bit_quantized_expert_amd import synth
from tests.helpers import check_route_protocol, tile_quantised

pytestmark = pytest.mark.gpu


def _lib():
    import bit_quantized_expert_amd as M
    M.lib()
    return M


def _weights(rows, k, seed):
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(rows, k, generator=g) * 0.02
    w[0, :32] = 0.0                       # an all-zero block
    w[1, 0:32] = 0.01 * torch.tensor([1.0, -1.0] * 16)   # equal magnitudes: first index wins
    w[min(2, rows - 1), 5] = 0.5          # an outlier
    return w


@pytest.mark.parametrize("qbits", [2, 3, 4])
@pytest.mark.parametrize("rows,k", [(3, 32), (17, 64), (40, 96), (64, 704), (33, 2048)])
def test_quantize_and_dequant_bit_exact(qbits, rows, k):
    M = _lib()
    w = _weights(rows, k, seed=rows * 1000 + k)
    codes = torch.empty(rows * k * qbits // 8, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows * k // 32, dtype=torch.int16, device="cuda")
    M.quantize(w.cuda(), qbits, codes, scales)
    want_codes, want_scales = O.quantize(w.numpy(), qbits)
    # the canonical layout, byte for byte
    assert np.array_equal(codes.cpu().numpy(), want_codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), want_scales.reshape(-1))
    out = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    M.dequant(codes, scales, rows, k, qbits, out)
    want = O.dequant(want_codes, want_scales, rows, k, qbits)
    assert np.array_equal(out.cpu().numpy().astype(np.float64), want)


@pytest.mark.parametrize("qbits", [2, 3, 4])
@pytest.mark.parametrize("rows,k", [(3, 32), (17, 64), (40, 96), (64, 704), (33, 2048)])
def test_repack_matches_kernel_layout(qbits, rows, k):
    """moe_repack of the oracle's canonical bytes gives the kernel layout as
    the tests restate it from its definition."""
    M = _lib()
    w = _weights(rows, k, seed=rows * 7 + k)
    want_codes, want_scales = O.quantize(w.numpy(), qbits)
    codes = torch.from_numpy(want_codes).cuda()
    scales = torch.from_numpy(want_scales.reshape(-1).view(np.int16)).cuda()
    pc = torch.full_like(codes, 0xAB)
    ps = torch.full_like(scales, 0x5A5A)
    M.repack(codes, scales, rows, k, qbits, pc, ps)
    tiled_codes, tiled_scales = tile_quantised(want_codes, want_scales, rows, k, qbits)
    assert np.array_equal(pc.cpu().numpy(), tiled_codes)
    assert np.array_equal(ps.cpu().numpy().view(np.uint16), tiled_scales)


def test_layer_from_caller_canonical_codes():
    """A caller holding canonical row-major codes (here: the oracle's own
    quantiser output) uploads them, repacks them with moe_repack and runs the
    layer: the output matches the oracle layer on those codes."""
    from tests.helpers import assert_close_output
    M = _lib()
    H, I, E, k, Is, qb, T = 256, 192, 12, 3, 96, 3, 9
    rng = np.random.default_rng(17)
    experts = [O.QExpert.from_float(*(rng.normal(0, 0.02, sh).astype(np.float32)
                                      for sh in ((I, H), (I, H), (H, I))), qb) for _ in range(E)]
    shared = O.QExpert.from_float(*(rng.normal(0, 0.02, sh).astype(np.float32)
                                    for sh in ((Is, H), (Is, H), (H, Is))), qb)
    arena = M.QArena(E, H, I, qb, "cuda")
    sarena = M.QArena(1, H, Is, qb, "cuda")
    for m in range(3):
        for e, ex in enumerate(experts):
            c, sc = (ex.gate, ex.up, ex.down)[m]
            arena.load_canonical(m, e, torch.from_numpy(c)[None].cuda(),
                                 torch.from_numpy(sc.reshape(-1).view(np.int16))[None].cuda())
        c, sc = (shared.gate, shared.up, shared.down)[m]
        sarena.load_canonical(m, 0, torch.from_numpy(c)[None].cuda(),
                              torch.from_numpy(sc.reshape(-1).view(np.int16))[None].cuda())
    w_r = (torch.from_numpy(rng.normal(0, 0.02, (E, H)).astype(np.float32))).to(torch.bfloat16).cuda()
    q = M.QLayer(w_r, None, arena, sarena)
    s = synth.MoEShape(H, I, E, k, Is, qb)
    x = torch.from_numpy(rng.normal(size=(T, H)).astype(np.float32)).to(torch.bfloat16).cuda()
    for algo in ("gemv", "grouped"):
        out = torch.empty(T, H, device="cuda")
        idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
        M.layer_forward(x, q, s, out=out, topk_idx=idx, algo=algo, ws=M.alloc_workspace(s, T, algo=algo))
        torch.cuda.synchronize()
        ref = O.layer_forward(x.float().cpu().numpy().astype(np.float64), w_r.float().cpu().numpy().astype(np.float64),
                              None, experts, shared, k, idx=idx.cpu().numpy())
        assert_close_output(out.cpu().numpy(), ref, f"canonical codes, {algo}")


def _route(M, wl, T, layer=0):
    s = wl.shape
    w_r, bias = synth.router(wl, layer, "cuda")
    x = synth.tokens(wl, "cuda", layer=layer, n_tokens=T)
    arena = M.QArena(1, 64, 32, 2, "cuda")  # experts are not read by the router
    q = M.QLayer(w_r, bias, arena, None)
    logits = torch.empty(T, s.n_experts, device="cuda")
    idx = torch.empty(T, s.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, s.top_k, device="cuda")
    M.route(x, q, s, idx, w, logits=logits)
    torch.cuda.synchronize()
    ol = O.router_logits(x.float().cpu().numpy().astype(np.float64), w_r.float().cpu().numpy().astype(np.float64),
                         None if bias is None else bias.cpu().numpy().astype(np.float64))
    return logits.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy(), ol


@pytest.mark.parametrize("name,T", [("tiny", 4), ("decode1", 1), ("decode16", 16), ("decode16", 333),
                                    ("decode16", 2500), ("prefill", 33000)])
def test_route_protocol(name, T):
    M = _lib()
    wl = synth.WORKLOADS[name]
    gl, gi, gw, ol = _route(M, wl, T)
    flagged = check_route_protocol(gl, gi, gw, ol, wl.shape.top_k)
    assert len(flagged) <= max(1, T // 100)


@pytest.mark.parametrize("H,E,T", [(2048, 512, 2100), (96, 40, 2200), (64, 8, 2050), (4096, 130, 2088),
                                   (2048, 512, 8192), (96, 40, 40000), (2048, 512, 65600), (64, 8, 70000)])
def test_router_tiles_match_small_batches(H, E, T):
    """Logits of T >= 2048 tokens at once (128-token tiles 64 experts wide
    below 256 tiles of 128, else 128 wide with either step variant) are the
    same bits as the same tokens routed 16 at a time (16 x 16 tiles): one
    accumulation order for every batch size, ragged token and expert tiles
    included.  Large T: a sample of the 16-token chunks, the first and the
    last among them."""
    M = _lib()
    wl = synth.custom("rt", H, 32, E, min(E, 8), 0, 2, T, seed=H + E, act_dtype=torch.bfloat16, zipf_bias=True)
    s = wl.shape
    w_r, bias = synth.router(wl, 0, "cuda")
    x = synth.tokens(wl, "cuda")
    arena = M.QArena(1, 64, 32, 2, "cuda")
    q = M.QLayer(w_r, bias, arena, None)
    big = torch.empty(T, E, device="cuda")
    M.route(x, q, s, torch.empty(T, s.top_k, dtype=torch.int32, device="cuda"), torch.empty(T, s.top_k, device="cuda"),
            logits=big)
    starts = list(range(0, T, 16))
    if len(starts) > 200:
        rng = np.random.default_rng(T)
        starts = sorted({starts[0], starts[-1], *rng.choice(starts, 60, replace=False).tolist()})
    for t0 in starts:
        t1 = min(T, t0 + 16)
        small = torch.empty(t1 - t0, E, device="cuda")
        M.route(x[t0:t1].contiguous(), q, s, torch.empty(t1 - t0, s.top_k, dtype=torch.int32, device="cuda"),
                torch.empty(t1 - t0, s.top_k, device="cuda"), logits=small)
        assert torch.equal(big[t0:t1], small), f"tokens {t0}..{t1 - 1}"


def test_route_all_equal_logits_tie_rule():
    """Zero router weights and no bias: every logit ties, so the selection is
    experts 0..k-1 with weight 1/k."""
    M = _lib()
    wl = synth.custom("ties", 64, 32, 40, 7, 0, 2, 9, seed=5, act_dtype=torch.bfloat16)
    arena = M.QArena(1, 64, 32, 2, "cuda")
    q = M.QLayer(torch.zeros(40, 64, dtype=torch.bfloat16, device="cuda"), None, arena, None)
    x = synth.tokens(wl, "cuda")
    idx = torch.empty(9, 7, dtype=torch.int32, device="cuda")
    w = torch.empty(9, 7, device="cuda")
    M.route(x, q, wl.shape, idx, w, ws=M.alloc_workspace(wl.shape, 9))
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(7), (9, 1)))
    assert np.allclose(w.cpu().numpy(), 1 / 7, rtol=0, atol=1e-7)


@pytest.mark.parametrize("E,k,T", [(40, 7, 1), (40, 7, 16), (512, 10, 1), (512, 10, 16), (512, 32, 1),
                                   (100, 32, 5), (33, 33 - 1, 16), (8, 8, 3)])
def test_layer_selection_exact_ties(E, k, T):
    """Zero router weights and a bias on a coarse grid: the logits are the
    bias exactly, with many exact ties (at the k-th place too).  The fused
    layer's selection (single-token and small-batch paths) equals the first k
    of the oracle's stable sort, and the standalone router's selection, bit
    for bit (indices and weights)."""
    from oracle import moe_oracle as O
    M = _lib()
    H, I, Is = 64, 32, 32
    g = torch.Generator().manual_seed(E * 1000 + k * 10 + T)
    bias = torch.randint(-3, 4, (E,), generator=g).float() * 0.5
    s = synth.MoEShape(H, I, E, k, Is, 2)
    arena = M.QArena(E, H, I, 2, "cuda")
    for m, (r, c) in enumerate(arena.mat_shapes):
        arena.quantize_from(m, torch.zeros(E, r, c, device="cuda"))
    sarena = M.QArena(1, H, Is, 2, "cuda")
    for m, (r, c) in enumerate(sarena.mat_shapes):
        sarena.quantize_from(m, torch.zeros(1, r, c, device="cuda"))
    q = M.QLayer(torch.zeros(E, H, dtype=torch.bfloat16, device="cuda"), bias.cuda(), arena, sarena)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).cuda()
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, device="cuda")
    out = torch.empty(T, H, device="cuda")
    M.layer_forward(x, q, s, out=out, topk_idx=idx, topk_w=w, algo="gemv", ws=M.alloc_workspace(s, T, algo="gemv"))
    idx2 = torch.empty_like(idx)
    w2 = torch.empty_like(w)
    M.route(x, q, s, idx2, w2, ws=M.alloc_workspace(s, T))
    torch.cuda.synchronize()
    want = O.topk_select(np.tile(bias.numpy().astype(np.float64), (T, 1)), k)
    assert np.array_equal(idx.cpu().numpy(), want)
    assert np.array_equal(idx2.cpu().numpy(), want)
    assert torch.equal(w, w2)


def _permute(M, idx_np, E, k):
    T = idx_np.shape[0]
    s = synth.MoEShape(64, 32, E, k, 0, 2)
    ws = M.alloc_workspace(s, T)
    idx = torch.from_numpy(idx_np.astype(np.int32)).cuda()
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    pp = torch.empty(T * k, dtype=torch.int32, device="cuda")
    M.permute(idx, T, s, counts, offsets, sp, pp, ws)
    return ws, counts.cpu().numpy(), offsets.cpu().numpy(), sp.cpu().numpy(), pp.cpu().numpy()


@pytest.mark.parametrize("T,E,k,skew", [(1, 512, 10, 0), (16, 512, 10, 1), (37, 9, 3, 0), (204, 512, 10, 1),
                                        (205, 512, 10, 1), (3000, 512, 10, 1), (32768, 512, 10, 1),
                                        (4096, 512, 10, 0), (500, 1, 1, 0), (3000, 4096, 32, 1),
                                        (16, 4096, 32, 0)])
def test_permute_bit_exact(T, E, k, skew):
    M = _lib()
    rng = np.random.default_rng(T * 7 + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p = p / p.sum()
        idx = np.stack([rng.choice(E, k, replace=False, p=p) for _ in range(min(T, 2000))])
        idx = np.concatenate([idx] * (T // len(idx) + 1))[:T]
    else:
        idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    _, counts, offsets, sp, pp = _permute(M, idx, E, k)
    wc, wo, wsp, wpp = O.permute(idx, E)
    assert np.array_equal(counts, wc)
    assert np.array_equal(offsets, wo)
    assert np.array_equal(sp, wsp)
    assert np.array_equal(pp, wpp)


@pytest.mark.parametrize("T", [5, 3000])
def test_permute_out_of_range_ids_are_reported(T):
    M = _lib()
    E, k = 16, 2
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    idx[1, 0] = E          # out of range
    idx[2, 1] = -1         # out of range
    ws, counts, offsets, sp, pp = _permute(M, idx, E, k)
    assert counts.sum() == T * k - 2
    assert pp[1 * k + 0] == -1 and pp[2 * k + 1] == -1
    with pytest.raises(M.MoeError) as ei:
        M.read_error(ws)
    assert ei.value.status == -5
    M.read_error(ws)  # cleared


def test_permute_error_survives_expert_ffn():
    """An out-of-range id recorded by moe_permute is still reported after
    moe_expert_ffn ran on the same workspace (the FFN's plan leaves the
    record alone)."""
    M = _lib()
    E, k, T = 16, 2, 5
    wl = synth.custom("err", 64, 32, E, k, 32, 2, T, seed=3, act_dtype=torch.bfloat16)
    s = wl.shape
    arena = M.QArena(E, 64, 32, 2, "cuda")
    for m, (r, c) in enumerate(arena.mat_shapes):
        arena.quantize_from(m, torch.zeros(E, r, c, device="cuda"))
    sarena = M.QArena(1, 64, 32, 2, "cuda")
    for m, (r, c) in enumerate(sarena.mat_shapes):
        sarena.quantize_from(m, torch.zeros(1, r, c, device="cuda"))
    q = M.QLayer(torch.zeros(E, 64, dtype=torch.bfloat16, device="cuda"), None, arena, sarena)
    rng = np.random.default_rng(4)
    idx_np = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    idx_np[3, 1] = E + 7
    for algo in ("gemv", "grouped"):
        ws = M.alloc_workspace(s, T, algo=algo)
        idx = torch.from_numpy(idx_np.astype(np.int32)).cuda()
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        sp = torch.empty(T * k, dtype=torch.int32, device="cuda")
        pp = torch.empty_like(sp)
        M.permute(idx, T, s, counts, offsets, sp, pp, ws)
        x = synth.tokens(wl, "cuda")
        y = torch.empty(T * k, 64, device="cuda")
        so = torch.empty(T, 64, device="cuda")
        M.expert_ffn(x, q, s, offsets, sp, y, so, algo=algo, ws=ws)
        with pytest.raises(M.MoeError) as ei:
            M.read_error(ws)
        assert ei.value.status == -5, algo
        M.read_error(ws)  # cleared
