"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a hand-derived fixture, a closed form, an
invariant, a special case that reduces to a textbook result, or a brute-force
pure-Python computation on tiny inputs.  None of these re-types the oracle's
own formula with the oracle's own library calls.
"""

import math
import os
import struct

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers

def _read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split(":", 1)
            out[key.strip()] = val.strip()
    return out


def _fp16_bits_to_float(bits):
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def _py_code(codes: bytes, rows, k, qbits, r, c):
    """Offset-binary code of weight (r, c), read bit by bit in pure Python."""
    lo_byte = codes[r * (k // 4) + c // 4]
    q = (lo_byte >> (2 * (c % 4))) & 3
    if qbits == 3:
        hi_byte = codes[rows * k // 4 + r * (k // 8) + c // 8]
        q |= ((hi_byte >> (c % 8)) & 1) << 2
    if qbits == 4:
        hi_byte = codes[rows * k // 4 + r * (k // 4) + c // 4]
        q |= ((hi_byte >> (2 * (c % 4))) & 3) << 2
    return q


def _py_dequant(codes, scales, rows, k, qbits):
    codes = bytes(np.asarray(codes, dtype=np.uint8))
    sc = [int(v) for v in np.asarray(scales, dtype=np.uint16).reshape(-1)]
    off = 1 << (qbits - 1)
    out = []
    for r in range(rows):
        row = []
        for c in range(k):
            s = _fp16_bits_to_float(sc[r * (k // 32) + c // 32])
            row.append((_py_code(codes, rows, k, qbits, r, c) - off) * s)
        out.append(row)
    return out


def _py_silu(z):
    return z / (1.0 + math.exp(-z))


def _py_matvec(w, v):
    return [sum(w[r][c] * v[c] for c in range(len(v))) for r in range(len(w))]


def _py_swiglu(x, wg, wu, wd):
    g = _py_matvec(wg, x)
    u = _py_matvec(wu, x)
    h = [_py_silu(a) * b for a, b in zip(g, u)]
    return _py_matvec(wd, h)


def _tiny_layer(seed=0, hidden=64, inter=32, n_experts=8, shared_inter=32, qbits=2, bias=False):
    rng = np.random.default_rng(seed)
    experts = []
    for _ in range(n_experts):
        experts.append(O.QExpert.from_float(
            rng.normal(0, 0.02, (inter, hidden)).astype(np.float32),
            rng.normal(0, 0.02, (inter, hidden)).astype(np.float32),
            rng.normal(0, 0.02, (hidden, inter)).astype(np.float32), qbits))
    shared = None
    if shared_inter:
        shared = O.QExpert.from_float(
            rng.normal(0, 0.02, (shared_inter, hidden)).astype(np.float32),
            rng.normal(0, 0.02, (shared_inter, hidden)).astype(np.float32),
            rng.normal(0, 0.02, (hidden, shared_inter)).astype(np.float32), qbits)
    w_r = rng.normal(0, 0.02, (n_experts, hidden)).astype(np.float32)
    b = rng.normal(0, 0.5, n_experts).astype(np.float32) if bias else None
    return w_r, b, experts, shared


# ---------------------------------------------------------------- format

@pytest.mark.parametrize("qbits", [2, 3, 4])
def test_quant_block_hand_example(qbits):
    g = _read_kv(os.path.join(GOLDEN, "quant_block.txt"))
    w = np.zeros((1, 32), dtype=np.float32)
    for item in g["weights"].split():
        i, v = item.split(":")
        w[0, int(i)] = np.float32(float(v))
    codes, scales = O.quantize(w, qbits)
    want_codes = bytes(int(h, 16) for h in g[f"bits{qbits}_codes"].split())
    assert bytes(codes) == want_codes
    assert int(scales[0, 0]) == int(g[f"bits{qbits}_scale_fp16"], 16)
    want_c = [int(v) for v in g[f"bits{qbits}_c"].split()]
    s = _fp16_bits_to_float(int(g[f"bits{qbits}_scale_fp16"], 16))
    deq = O.dequant(codes, scales, 1, 32, qbits)[0]
    assert list(deq) == [c * s for c in want_c]


@pytest.mark.parametrize("qbits", [2, 3, 4])
def test_pack_unpack_bit_layout_brute_force(qbits):
    rng = np.random.default_rng(1)
    rows, k = 5, 96
    q = rng.integers(0, 1 << qbits, (rows, k)).astype(np.uint8)
    packed = O.pack_codes(q, qbits)
    assert packed.size == rows * k * qbits // 8
    raw = bytes(packed)
    for r in range(rows):
        for c in range(k):
            assert _py_code(raw, rows, k, qbits, r, c) == q[r, c]
    # unpack of arbitrary bytes agrees with bit extraction
    rnd = rng.integers(0, 256, rows * k * qbits // 8).astype(np.uint8)
    un = O.unpack_codes(rnd, rows, k, qbits)
    for r in range(rows):
        for c in range(k):
            assert un[r, c] == _py_code(bytes(rnd), rows, k, qbits, r, c)


@pytest.mark.parametrize("qbits", [2, 3, 4])
def test_dequant_closed_form_brute_force(qbits):
    rng = np.random.default_rng(2)
    rows, k = 3, 64
    codes = rng.integers(0, 256, rows * k * qbits // 8).astype(np.uint8)
    scales = rng.normal(0, 0.01, (rows, k // 32)).astype(np.float16).view(np.uint16)
    got = O.dequant(codes, scales, rows, k, qbits)
    want = np.array(_py_dequant(codes, scales, rows, k, qbits))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("qbits", [2, 3, 4])
def test_quantize_properties(qbits):
    rng = np.random.default_rng(3)
    rows, k = 64, 256
    w = rng.normal(0, 0.02, (rows, k)).astype(np.float32)
    codes, scales = O.quantize(w, qbits)
    q = O.unpack_codes(codes, rows, k, qbits).astype(np.int64)
    cmin, cmax = -(1 << (qbits - 1)), (1 << (qbits - 1)) - 1
    c = q - (1 << (qbits - 1))
    assert c.min() >= cmin and c.max() <= cmax
    d = scales.view(np.float16).astype(np.float64)
    blocks = w.reshape(rows, k // 32, 32).astype(np.float64)
    amax_idx = np.argmax(np.abs(blocks), axis=-1)
    cb = c.reshape(rows, k // 32, 32)
    # the largest-magnitude element always takes the most negative code
    assert np.all(np.take_along_axis(cb, amax_idx[..., None], -1) == cmin)
    # the scale has the opposite sign of that element
    m = np.take_along_axis(blocks, amax_idx[..., None], -1)[..., 0]
    assert np.all(np.sign(d) == -np.sign(m))
    # elements inside the code range are within half a step (plus fp32 slack)
    deq = O.dequant(codes, scales, rows, k, qbits).reshape(rows, k // 32, 32)
    ratio = blocks / d[..., None]
    inside = (ratio >= cmin - 0.5) & (ratio <= cmax + 0.5)
    err = np.abs(deq - blocks)
    assert np.all(err[inside] <= (np.abs(d)[..., None] * (0.5 + 1e-6) + 1e-12).repeat(32, -1)[inside])
    # clamped elements sit at c_max
    assert np.all(cb[~inside] == cmax)
    # quantising the dequantised weights gives the same codes and scales
    codes2, scales2 = O.quantize(deq.reshape(rows, k).astype(np.float32), qbits)
    assert np.array_equal(codes, codes2) and np.array_equal(scales, scales2)


def test_quantize_zero_block():
    codes, scales = O.quantize(np.zeros((2, 64), dtype=np.float32), 2)
    # the scale of an all-zero block is stored as +0 (bit pattern 0)
    assert np.all(scales == 0)
    assert np.all(O.unpack_codes(codes, 2, 64, 2) == 2)
    assert np.all(O.dequant(codes, scales, 2, 64, 2) == 0)


# ---------------------------------------------------------------- router

def test_router_logits_brute_force():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 16))
    w = rng.normal(size=(5, 16))
    b = rng.normal(size=5)
    got = O.router_logits(x, w, b)
    for t in range(3):
        for e in range(5):
            want = sum(float(x[t, h]) * float(w[e, h]) for h in range(16)) + float(b[e])
            assert abs(got[t, e] - want) <= 1e-12 * (1 + abs(want))


def test_topk_equals_full_stable_sort_with_ties():
    rng = np.random.default_rng(5)
    # coarse values force many exact ties
    logits = rng.integers(-3, 4, (50, 12)).astype(np.float64)
    for k in (1, 3, 12):
        idx = O.topk_select(logits, k)
        for t in range(50):
            row = [float(v) for v in logits[t]]
            want = sorted(range(12), key=lambda e: (-row[e], e))[:k]
            assert list(idx[t]) == want


def test_zero_router_selects_first_k_with_equal_weights():
    x = np.random.default_rng(6).normal(size=(4, 8))
    logits, idx, w = O.route(x, np.zeros((6, 8)), None, 3)
    assert np.all(idx == np.arange(3))
    assert np.allclose(w, 1.0 / 3.0, rtol=0, atol=1e-15)


def test_weights_are_softmax_over_selected():
    rng = np.random.default_rng(7)
    logits = rng.normal(0, 2, (20, 30))
    idx = O.topk_select(logits, 5)
    w = O.topk_weights(logits, idx)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)
    for t in range(20):
        sel = [float(logits[t, e]) for e in idx[t]]
        z = [math.exp(v - sel[0]) for v in sel]
        want = [v / sum(z) for v in z]
        assert np.allclose(w[t], want, rtol=1e-13, atol=0)
        # descending order of weight (rank 0 largest)
        assert all(w[t, j] >= w[t, j + 1] for j in range(4))


# ---------------------------------------------------------------- permute

def test_permute_brute_force():
    rng = np.random.default_rng(8)
    t, k, e = 37, 3, 9
    idx = np.stack([rng.choice(e, k, replace=False) for _ in range(t)]).astype(np.int32)
    counts, offsets, sorted_pair, pair_pos = O.permute(idx, e)
    want_sorted = []
    for ex in range(e):
        for tt in range(t):
            for j in range(k):
                if idx[tt, j] == ex:
                    want_sorted.append(tt * k + j)
    assert list(sorted_pair) == want_sorted
    assert list(counts) == [sum(1 for v in idx.reshape(-1) if v == ex) for ex in range(e)]
    assert offsets[0] == 0 and all(offsets[i + 1] - offsets[i] == counts[i] for i in range(e))
    for p in range(t * k):
        assert sorted_pair[pair_pos[p]] == p


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.permute(np.array([[0, 9]]), 9)


# ---------------------------------------------------------------- FFN / combine

def test_single_expert_reduces_to_dense_swiglu():
    """E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN with
    the dequantised weights (checked with torch's float64 silu and matmul)."""
    w_r, b, experts, _ = _tiny_layer(seed=9, n_experts=1, shared_inter=0)
    x = np.random.default_rng(10).normal(size=(5, 64))
    out = O.layer_forward(x, w_r, None, experts, None, 1)
    wg, wu, wd = (torch.from_numpy(m) for m in experts[0].dense())
    xt = torch.from_numpy(x)
    want = (torch.nn.functional.silu(xt @ wg.T) * (xt @ wu.T)) @ wd.T
    assert np.allclose(out, want.numpy(), rtol=1e-12, atol=1e-15)


def test_zero_input_gives_zero_output():
    w_r, _, experts, shared = _tiny_layer(seed=11)
    out = O.layer_forward(np.zeros((3, 64)), w_r, None, experts, shared, 2)
    assert np.all(out == 0)


def test_combine_one_hot_and_linear():
    rng = np.random.default_rng(12)
    t, k, h = 4, 3, 8
    y = rng.normal(size=(t * k, h))
    pair_pos = rng.permutation(t * k).astype(np.int32)
    w = np.zeros((t, k))
    w[:, 1] = 1.0
    out = O.combine(y, pair_pos, w, None)
    for tt in range(t):
        assert np.array_equal(out[tt], y[pair_pos[tt * k + 1]])
    w2 = rng.random((t, k))
    s = rng.normal(size=(t, h))
    a = O.combine(y, pair_pos, w2, s)
    b = O.combine(2 * y, pair_pos, w2, 2 * s)
    assert np.allclose(b, 2 * a, rtol=1e-14, atol=0)


@pytest.mark.parametrize("qbits", [2, 4])
def test_layer_brute_force_tiny(qbits):
    """Whole layer on the tiny workload shape versus pure-Python loops that
    re-derive every step from the definition (bit extraction, loops, sort,
    math.exp) -- relative error <= 1e-12."""
    w_r, b, experts, shared = _tiny_layer(seed=13, bias=True, qbits=qbits)
    rng = np.random.default_rng(14)
    x = rng.normal(size=(4, 64)).astype(np.float32)
    got = O.layer_forward(x, w_r, b, experts, shared, 2)

    def deq(m, rows, k):
        return _py_dequant(m[0], m[1], rows, k, qbits)

    dense = [(deq(e.gate, 32, 64), deq(e.up, 32, 64), deq(e.down, 64, 32)) for e in experts]
    sdense = (deq(shared.gate, 32, 64), deq(shared.up, 32, 64), deq(shared.down, 64, 32))
    for t in range(4):
        xt = [float(v) for v in x[t]]
        logits = [sum(xt[h] * float(w_r[e, h]) for h in range(64)) + float(b[e]) for e in range(8)]
        top = sorted(range(8), key=lambda e: (-logits[e], e))[:2]
        z = [math.exp(logits[e] - logits[top[0]]) for e in top]
        wts = [v / sum(z) for v in z]
        out = _py_swiglu(xt, *sdense)
        for wj, e in zip(wts, top):
            ye = _py_swiglu(xt, *dense[e])
            out = [o + wj * v for o, v in zip(out, ye)]
        out = np.array(out)
        assert np.linalg.norm(got[t] - out) <= 1e-12 * np.linalg.norm(out)


def test_route_tail_skip_brute_force():
    """The route tail skip against pure-Python loops on a 3-token window:
    an expert is dropped iff no token ranks it below the first tail rank, its
    pairs add nothing, the other weights are untouched."""
    w_r, b, experts, shared = _tiny_layer(seed=40, bias=True, n_experts=8)
    rng = np.random.default_rng(41)
    x = rng.normal(size=(3, 64)).astype(np.float32).astype(np.float64)
    k, first_tail = 4, 2
    got = O.layer_forward(x, w_r, b, experts, shared, k, tail_skip=first_tail)
    logits = O.router_logits(x, w_r, b)
    sel = [sorted(range(8), key=lambda e: (-logits[t, e], e))[:k] for t in range(3)]
    head = {sel[t][j] for t in range(3) for j in range(first_tail)}
    want = np.zeros((3, 64))
    for t in range(3):
        z = [math.exp(logits[t, e] - logits[t, sel[t][0]]) for e in sel[t]]
        out = np.array(_py_swiglu(list(x[t]), *shared.dense()))
        for j, e in enumerate(sel[t]):
            if e in head:
                out = out + z[j] / sum(z) * np.array(_py_swiglu(list(x[t]), *experts[e].dense()))
        want[t] = out
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)
    # something was dropped in this window (else the case would not test the rule)
    assert any(e not in head for t in range(3) for e in sel[t])


def test_route_tail_skip_closed_forms():
    w_r, b, experts, shared = _tiny_layer(seed=42, bias=True, n_experts=8)
    x = np.random.default_rng(43).normal(size=(4, 64))
    plain = O.layer_forward(x, w_r, b, experts, shared, 3)
    # a first tail rank at or past k drops nothing
    assert np.array_equal(O.layer_forward(x, w_r, b, experts, shared, 3, tail_skip=3), plain)
    # one token: exactly ranks >= the first tail rank are dropped
    one = O.layer_forward(x[:1], w_r, b, experts, shared, 3, tail_skip=1)
    r = O.layer_forward(x[:1], w_r, b, experts, shared, 3, return_all=True)
    e0 = r["idx"][0, 0]
    want = r["shared"][0] + r["w"][0, 0] * r["y"][r["pair_pos"][0]]
    assert np.allclose(one[0], want, rtol=1e-13, atol=0) and e0 == r["idx"][0, 0]
    # the keep mask: never drops an expert some token ranks in the head
    idx = np.array([[5, 1, 7], [1, 2, 5], [3, 4, 6]])
    keep = O.tail_skip_keep(idx, 2)
    assert keep.tolist() == [[True, True, False], [True, True, True], [True, True, False]]


# ---------------------------------------------------------------- stacks

def test_bf16_round_ties_and_fp32_agreement():
    one = 1.0
    assert O.bf16_round(np.array([one + 2.0 ** -8]))[0] == 1.0                   # tie -> even
    assert O.bf16_round(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2.0 ** -6   # tie -> even
    assert O.bf16_round(np.array([one + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 2.0 ** -7
    assert O.bf16_round(np.array([-(one + 2.0 ** -8)]))[0] == -1.0
    v = np.random.default_rng(15).normal(size=1000).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.bf16_round(v.astype(np.float64)), want)


def test_rmsnorm_closed_form():
    r = np.full((2, 16), 3.0)
    a = O.rmsnorm_bf16(r, eps=0.0)
    assert np.all(a == 1.0)
    r = np.array([[3.0, 4.0]])                     # mean square 12.5
    a = O.rmsnorm_bf16(r, eps=0.0)
    assert np.array_equal(a, O.bf16_round(np.array([[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]])))


def test_stack_two_layers_brute_force():
    layers = [_tiny_layer(seed=20 + l, bias=True) for l in range(2)]
    x0 = np.random.default_rng(22).normal(size=(3, 64))
    r, acts, outs = O.stack_forward(x0, layers, 2)
    rr = x0.copy()
    for l in range(2):
        ms = np.array([sum(v * v for v in row) / 64 for row in rr])
        a = O.bf16_round(rr / np.sqrt(ms + 1e-6)[:, None])
        assert np.array_equal(a, acts[l])
        rr = rr + O.layer_forward(a, *layers[l], 2)
    assert np.allclose(r, rr, rtol=1e-14, atol=0)


def test_stack_teacher_forcing():
    """Teacher forcing replaces a layer's activation and nothing else.
    Closed form: zero activations at every layer give zero layer outputs
    (silu(0) * 0 = 0 for every expert), so the residual stays x0 exactly.
    Brute force: a 2-layer stack whose layer 1 is fed a foreign activation a*
    equals x0 + MoE_0(a_0) + MoE_1(a*) with a_0 the normalised x0 from
    pure-Python loops."""
    layers = [_tiny_layer(seed=30 + l, bias=True) for l in range(3)]
    x0 = np.random.default_rng(33).normal(size=(3, 64))
    r, acts, outs = O.stack_forward(x0, layers, 2, teacher=lambda l: np.zeros((3, 64)))
    assert np.array_equal(r, x0)
    assert all(np.array_equal(o, np.zeros((3, 64))) for o in outs)
    a_star = O.bf16_round(np.random.default_rng(34).normal(size=(3, 64)))
    ms = np.array([sum(v * v for v in row) / 64 for row in x0])
    a0 = O.bf16_round(x0 / np.sqrt(ms + 1e-6)[:, None])
    r, acts, outs = O.stack_forward(x0, layers[:2], 2, teacher=lambda l: a0 if l == 0 else a_star)
    assert np.array_equal(acts[1], a_star)
    want = x0 + O.layer_forward(a0, *layers[0], 2) + O.layer_forward(a_star, *layers[1], 2)
    assert np.allclose(r, want, rtol=1e-14, atol=0)
    # and with the oracle's own activations fed back, teacher forcing changes nothing
    r_plain, acts_plain, _ = O.stack_forward(x0, layers, 2)
    r_tf, _, _ = O.stack_forward(x0, layers, 2, teacher=lambda l: acts_plain[l])
    assert np.array_equal(r_plain, r_tf)


# ---------------------------------------------------------------- sizes

def test_byte_census_matches_pages():
    g = _read_kv(os.path.join(GOLDEN, "pages_census.txt"))
    hidden, inter = 2048, 704
    per_matrix = O.matrix_code_bytes(inter, hidden, 2) + inter * hidden // 32 * 2
    per_expert = 3 * per_matrix
    total = int(g["layers"]) * int(g["experts_per_layer"]) * per_expert
    assert int(g["layers"]) * int(g["experts_per_layer"]) == int(g["routed_experts_total"])
    assert abs(total / 1e9 / float(g["routed_expert_bytes_q2_gb"]) - 1) < 0.025
    per_token = int(g["layers"]) * int(g["active_per_layer"]) * per_expert
    assert abs(per_token / 1e9 / float(g["expert_bytes_read_per_token_gb"]) - 1) < 0.025
    assert abs(1e9 / per_expert / float(g["experts_per_gb"]) - 1) < 0.10
    # a real quantised expert has exactly that many bytes
    q = O.QExpert.from_float(np.zeros((inter, hidden), np.float32), np.zeros((inter, hidden), np.float32),
                             np.zeros((hidden, inter), np.float32), 2)
    n = sum(c.size + s.size * 2 for c, s in (q.gate, q.up, q.down))
    assert n == per_expert == 1_351_680
