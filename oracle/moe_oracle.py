"""Plain, slow CPU oracle of the sparse Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke entry and
the benchmark's CPU-baseline leg may import this module.  The GPU library
never calls it and shares no code with it.

What is computed, and where it comes from:

* The layer: per token, a router scores 512 experts and keeps 10 of them; one
  shared expert always runs; the GPU sums the finished expert vectors.
  Sources: "How Strata runs a 125-billion-parameter model on a single 12 GB to
  24 GB graphics card" (intro: 10 of 512 experts at each of 48 layers;
  Step 2, "Mapped host doorbell and a single captured CUDA graph": the router
  writes the 10 selected IDs; Step 2, "Dynamic PCIe and CPU co-execution": the
  GPU sums the finished vectors), and "Strata Open-Source Runtime: Running a
  125B-Parameter Qwen3 Model on a 12GB GPU" (section "The Model Itself: The
  Compute-Storage Gap in Sparse MoE": 10 active of 512 plus one shared expert
  that always runs).
* The ranks 0..9 of the top-10 are ordered by router weight (page 1, Step 2,
  "Verify-window route tail skip": ranks 7, 8, 9 carry the smallest weights).
* Expert weights are read directly from 2-bit (Q2_0-class) storage (page 1,
  intro and Step 1 byte table).

What the pages leave open, and the reading taken here (the workload's stated
definition fills each gap):

* expert FFN = SwiGLU: y = W_down (silu(W_gate x) * (W_up x)),
  silu(z) = z / (1 + exp(-z));
* router weights = softmax over all E logits, renormalised over the selected k
  (identical to a softmax over the k selected logits);
* selection on logits with key (-logit, expert index): ties go to the lower
  index;
* quantised block format: 32 weights per block along the reduction axis, one
  fp16 scale per block, codes c in [-2^(b-1), 2^(b-1)-1], weight = c * scale;
  codes stored offset-binary q = c + 2^(b-1);
* the shared expert has weight 1 and no gate;
* stacked layers: pre-norm residual, RMSNorm without learned weight, eps 1e-6,
  the normalised activation rounded to bf16 (round to nearest even) before
  each layer.

Precision: everything is float64 except the quantiser's decisions, which are
taken in float32 (the GPU kernel's precision) so that both sides pick the
same integer code.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Block format.  Bit layout (a reading; the pages are silent):
#   2-bit: row-major [rows][K/4] bytes; weight k of a row sits in byte k//4 at
#          bits 2*(k%4) .. 2*(k%4)+1.
#   3-bit: planar.  First a low plane laid out exactly like the 2-bit codes
#          (low two bits of q), then a high plane [rows][K/8] bytes with bit 2
#          of q for weight k in byte k//8 at bit k%8.
#   4-bit: planar.  The low plane as for 3-bit, then a second plane in the
#          same 2-bit layout holding bits 2..3 of q ([rows][K/4] bytes).  The
#          pages' quantisation ladder tops out at a 4-bit file ("Strata serves
#          a 125B MoE at 94 tokens/s ...", section "Quality is a sizing
#          decision"; "How Strata runs a 125-billion-parameter model ...",
#          benchmark table, the R9700 row); they give no bit layout for it.
#   scales: fp16 [rows][K/32], row-major.
# ---------------------------------------------------------------------------

BLOCK = 32


def code_offset(qbits: int) -> int:
    return 1 << (qbits - 1)


def code_range(qbits: int) -> tuple[int, int]:
    off = code_offset(qbits)
    return -off, off - 1


def matrix_code_bytes(rows: int, k: int, qbits: int) -> int:
    return rows * k * qbits // 8


def _check_shape(rows: int, k: int, qbits: int) -> None:
    if qbits not in (2, 3, 4):
        raise ValueError(f"qbits must be 2, 3 or 4, got {qbits}")
    if k % BLOCK != 0:
        raise ValueError(f"K={k} must be a multiple of {BLOCK}")
    if rows < 0:
        raise ValueError("rows must be >= 0")


def pack_codes(q: np.ndarray, qbits: int) -> np.ndarray:
    """Pack offset-binary codes q [rows, K] (values 0..2^b-1) into bytes."""
    q = np.asarray(q, dtype=np.uint8)
    rows, k = q.shape
    _check_shape(rows, k, qbits)
    def plane2(v):  # two bits per weight, four weights per byte, weight k at bits 2 (k % 4)
        v = v.reshape(rows, k // 4, 4).astype(np.uint16)
        return (v[..., 0] | (v[..., 1] << 2) | (v[..., 2] << 4) | (v[..., 3] << 6)).astype(np.uint8)

    lo_bytes = plane2(q & 3)
    if qbits == 2:
        return lo_bytes.reshape(-1)
    if qbits == 4:
        return np.concatenate([lo_bytes.reshape(-1), plane2((q >> 2) & 3).reshape(-1)])
    hi = ((q >> 2) & 1).reshape(rows, k // 8, 8).astype(np.uint16)
    hi_bytes = np.zeros((rows, k // 8), dtype=np.uint16)
    for bit in range(8):
        hi_bytes |= hi[..., bit] << bit
    return np.concatenate([lo_bytes.reshape(-1), hi_bytes.astype(np.uint8).reshape(-1)])


def unpack_codes(codes: np.ndarray, rows: int, k: int, qbits: int) -> np.ndarray:
    """Inverse of pack_codes: bytes -> offset-binary codes q [rows, K] uint8."""
    _check_shape(rows, k, qbits)
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    n_lo = rows * k // 4

    def plane2(b):
        b = b.reshape(rows, k // 4)
        return np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(rows, k)

    lo = plane2(codes[:n_lo])
    if qbits == 2:
        return lo.astype(np.uint8)
    if qbits == 4:
        return (lo | (plane2(codes[n_lo:2 * n_lo]) << 2)).astype(np.uint8)
    hi_bytes = codes[n_lo:n_lo + rows * k // 8].reshape(rows, k // 8)
    hi = np.stack([(hi_bytes >> i) & 1 for i in range(8)], axis=-1).reshape(rows, k)
    return (lo | (hi << 2)).astype(np.uint8)


def quantize(w: np.ndarray, qbits: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 weights [rows, K] to the block format.

    Reading (the pages give no quantiser; the workload names only the format):
    per block of 32 along K, m is the signed element of largest magnitude
    (first index on ties), the scale is d = fp16_RNE(m / c_min) with
    c_min = -2^(b-1), and each code is c = clamp(rint_half_even(w / d),
    c_min, c_max).  A zero scale gives c = 0 for the whole block.  Every step
    is taken in float32 (the kernel's precision) so the integer decisions
    agree with the GPU bit for bit.

    Returns (codes uint8 bytes, scales uint16 fp16 bit patterns [rows, K/32]).
    """
    w = np.asarray(w, dtype=np.float32)
    rows, k = w.shape
    _check_shape(rows, k, qbits)
    cmin, cmax = code_range(qbits)
    blocks = w.reshape(rows, k // BLOCK, BLOCK)
    first_max = np.argmax(np.abs(blocks), axis=-1)          # first index on ties
    m = np.take_along_axis(blocks, first_max[..., None], axis=-1)[..., 0]
    d16 = (m / np.float32(cmin)).astype(np.float32).astype(np.float16)
    d16 = np.where(d16 == 0, np.float16(0.0), d16)          # a zero scale is stored as +0
    d32 = d16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (blocks / d32[..., None]).astype(np.float32)
    c = np.clip(np.rint(ratio), cmin, cmax)
    c = np.where((d32 == 0)[..., None], 0.0, c)
    q = (c.astype(np.int32) + code_offset(qbits)).astype(np.uint8).reshape(rows, k)
    return pack_codes(q, qbits), d16.view(np.uint16)


def dequant(codes: np.ndarray, scales: np.ndarray, rows: int, k: int, qbits: int) -> np.ndarray:
    """W[r, k] = (q - 2^(b-1)) * scale[r, k // 32], float64 (exact).

    The product of a small integer and an fp16 value is exact in float64 (and
    in float32), so this is the closed form with no rounding at all.
    """
    q = unpack_codes(codes, rows, k, qbits).astype(np.int64) - code_offset(qbits)
    s = np.asarray(scales, dtype=np.uint16).reshape(rows, k // BLOCK).view(np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(s, BLOCK, axis=1)


# ---------------------------------------------------------------------------
# Router: logits, top-k selection, renormalised softmax weights.
# ---------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray, bias: np.ndarray | None) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * W_r[e, h] + b[e]  (float64).

    The router scores every expert of the layer for each token before the
    expert IDs are known (page 1, Step 2, "Mapped host doorbell ...").
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_router, dtype=np.float64)
    logits = x @ w.T
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=np.float64)[None, :]
    return logits


def topk_select(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, in descending order.

    Ranks 0..k-1 follow router weight (page 1, Step 2, "Verify-window route
    tail skip": the tail ranks carry the smallest weights).  Ties go to the
    lower expert index: the order key is (-logit, expert).
    """
    logits = np.asarray(logits)
    t, e = logits.shape
    if not 1 <= k <= e:
        raise ValueError(f"k={k} must be in [1, {e}]")
    order = np.lexsort((np.broadcast_to(np.arange(e), (t, e)), -logits), axis=-1)
    return order[:, :k].astype(np.int32)


def topk_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over all E logits, renormalised over the selected experts."""
    logits = np.asarray(logits, dtype=np.float64)
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True)


def route(x, w_router, bias, k: int):
    """Router step: (logits, topk_idx [T,k] int32, topk_w [T,k] float64)."""
    logits = router_logits(x, w_router, bias)
    idx = topk_select(logits, k)
    return logits, idx, topk_weights(logits, idx)


# ---------------------------------------------------------------------------
# Token-to-expert permutation.
# ---------------------------------------------------------------------------

def permute(topk_idx: np.ndarray, n_experts: int):
    """Group the (token, rank) pairs by expert.

    Pair id p = t * k + j.  Within an expert's segment pairs keep ascending
    (t, j) order (a stable sort), which makes the permutation unique.
    Returns counts [E], offsets [E+1], sorted_pair [T*k], pair_pos [T*k]
    (pair_pos[p] = position of pair p in sorted order).
    """
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    if flat.size and (flat.min() < 0 or flat.max() >= n_experts):
        raise ValueError("expert index out of range")
    sorted_pair = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=n_experts).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    pair_pos = np.empty_like(sorted_pair)
    pair_pos[sorted_pair] = np.arange(flat.size, dtype=np.int32)
    return counts, offsets, sorted_pair, pair_pos


# ---------------------------------------------------------------------------
# Expert FFN (SwiGLU) read from quantised weights.
# ---------------------------------------------------------------------------

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu(x_rows: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """y = W_down (silu(W_gate x) * (W_up x)) for each row x (float64)."""
    g = x_rows @ w_gate.T
    u = x_rows @ w_up.T
    return (silu(g) * u) @ w_down.T


class QExpert:
    """One expert's three quantised matrices (gate [I,H], up [I,H], down [H,I])."""

    def __init__(self, gate, up, down, hidden: int, inter: int, qbits: int):
        # each of gate/up/down is a (codes, scales) pair
        self.gate, self.up, self.down = gate, up, down
        self.hidden, self.inter, self.qbits = hidden, inter, qbits

    @classmethod
    def from_float(cls, w_gate, w_up, w_down, qbits: int) -> "QExpert":
        inter, hidden = np.asarray(w_gate).shape
        return cls(quantize(w_gate, qbits), quantize(w_up, qbits), quantize(w_down, qbits),
                   hidden, inter, qbits)

    def dense(self):
        """Dequantised (W_gate, W_up, W_down) in float64."""
        h, i, b = self.hidden, self.inter, self.qbits
        return (dequant(*self.gate, i, h, b), dequant(*self.up, i, h, b),
                dequant(*self.down, h, i, b))


class _OnlyExperts:
    """The experts of a layer, of which only `kept` are evaluated (the others
    are None: their outputs are left at zero)."""

    def __init__(self, experts, kept):
        self.experts, self.kept = experts, kept

    def __len__(self):
        return len(self.experts)

    def __getitem__(self, e):
        return self.experts[e] if int(e) in self.kept else None


def expert_outputs(x: np.ndarray, topk_idx: np.ndarray, experts, sorted_pair: np.ndarray,
                   offsets: np.ndarray) -> np.ndarray:
    """Y[s] = expert(sorted_pair[s] // k)(x[token]) for every pair, sorted order
    (rows of an expert given as None stay zero)."""
    x = np.asarray(x, dtype=np.float64)
    t, k = topk_idx.shape
    y = np.zeros((t * k, x.shape[1]), dtype=np.float64)
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo or experts[e] is None:
            continue
        tokens = sorted_pair[lo:hi] // k
        y[lo:hi] = swiglu(x[tokens], *experts[e].dense())
    return y


def combine(y_sorted: np.ndarray, pair_pos: np.ndarray, topk_w: np.ndarray,
            shared_out: np.ndarray | None) -> np.ndarray:
    """out[t] = s[t] + sum_j w[t, j] * Y[pair_pos[t*k + j]]  (the GPU-side sum
    of the finished expert vectors, page 1, Step 2, "Dynamic PCIe and CPU
    co-execution")."""
    t, k = topk_w.shape
    ys = np.asarray(y_sorted, dtype=np.float64)[np.asarray(pair_pos).reshape(t, k)]
    out = np.einsum("tj,tjh->th", np.asarray(topk_w, dtype=np.float64), ys)
    if shared_out is not None:
        out = out + shared_out
    return out


def tail_skip_keep(idx: np.ndarray, first_tail_rank: int) -> np.ndarray:
    """The route tail skip of a verify window ("How Strata runs a
    125-billion-parameter model ...", Step 2, "Verify-window route tail skip
    (STRATA_ROUTE_TAIL_SKIP=7)"): an expert that every token of the window
    ranks in the tail of its top-k (rank >= first_tail_rank, the smallest
    router weights) contributes almost nothing and is skipped; every expert
    that at least one token ranks below first_tail_rank is kept.  Reading
    taken here: a token that did not select an expert does not rank it, so an
    expert is kept iff some token ranks it 0 .. first_tail_rank - 1, and a
    skipped expert's pairs contribute nothing (the other weights are not
    renormalised).  Returns the keep mask of the pairs [T, k] (rank order)."""
    idx = np.asarray(idx)
    head = np.unique(idx[:, :first_tail_rank])
    return np.isin(idx, head)


def layer_forward(x, w_router, bias, experts, shared, k: int, return_all: bool = False, idx=None,
                  tail_skip: int | None = None):
    """One MoE layer: route, permute, routed SwiGLU experts, shared expert,
    weighted combine.  `experts` is a sequence of QExpert (length E); `shared`
    is a QExpert or None.  If `idx` [T, k] is given it replaces the selection
    (the weights are still the renormalised softmax of this layer's logits at
    those experts) -- used to evaluate the layer at another implementation's
    choice among near-tied experts.  With `tail_skip` (the first tail rank,
    the pages' 7) the T tokens are one verify window and the route tail skip
    drops the experts tail_skip_keep rejects."""
    x = np.asarray(x, dtype=np.float64)
    if idx is None:
        logits, idx, w = route(x, w_router, bias, k)
    else:
        logits = router_logits(x, w_router, bias)
        idx = np.asarray(idx, dtype=np.int32)
        w = topk_weights(logits, idx)
    keep = np.ones(idx.shape, dtype=bool) if tail_skip is None else tail_skip_keep(idx, tail_skip)
    counts, offsets, sorted_pair, pair_pos = permute(idx, len(experts))
    kept_experts = set(np.asarray(idx)[keep].tolist())
    y = expert_outputs(x, idx, _OnlyExperts(experts, kept_experts), sorted_pair, offsets)
    s = swiglu(x, *shared.dense()) if shared is not None else None
    out = combine(y, pair_pos, np.where(keep, w, 0.0), s)
    if return_all:
        return dict(out=out, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                    sorted_pair=sorted_pair, pair_pos=pair_pos, y=y, shared=s)
    return out


# ---------------------------------------------------------------------------
# Stacked layers (the decode and prefill stacks of the workload).
# ---------------------------------------------------------------------------

def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), directly
    from float64 (no intermediate float32 rounding).  Normal range only; the
    activations here never reach bf16 subnormals or overflow."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                       # v = m * 2^e, 0.5 <= |m| < 1
    m = np.rint(m * 256.0) / 256.0           # 8 significant bits, half to even
    return np.ldexp(m, e)


def rmsnorm_bf16(r: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """a = bf16_RNE(r / sqrt(mean(r^2) + eps)) per row."""
    r = np.asarray(r, dtype=np.float64)
    return bf16_round(r / np.sqrt(np.mean(r * r, axis=1, keepdims=True) + eps))


def stack_forward(x0: np.ndarray, layers, k: int, teacher=None):
    """r_0 = x0; for each layer l: a_l = bf16(RMSNorm(r_l)), r_{l+1} = r_l + MoE_l(a_l).

    `layers` is a sequence of (w_router, bias, experts, shared).  If `teacher`
    is given it maps a layer index to the activation a_l to feed instead of
    the oracle's own (teacher forcing).  Returns (r_L, [a_l], [out_l]).
    """
    r = np.asarray(x0, dtype=np.float64)
    acts, outs = [], []
    for l, (w_router, bias, experts, shared) in enumerate(layers):
        a = rmsnorm_bf16(r) if teacher is None else np.asarray(teacher(l), dtype=np.float64)
        out = layer_forward(a, w_router, bias, experts, shared, k)
        acts.append(a)
        outs.append(out)
        r = r + out
    return r, acts, outs
