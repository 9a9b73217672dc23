"""The no-allocation layer entry point against moe_layer_forward: the same
kernels on the same inputs, so the same bits (outputs, selection, weights,
stack glue), on two calls in a row with the second one smaller, on the decode
and grouped-GEMM paths."""

import numpy as np
import pytest
import torch

from bit_quantized_expert_amd import synth
from tests.helpers import DeviceLayer

pytestmark = pytest.mark.gpu


def _M():
    import bit_quantized_expert_amd as M
    M.lib()
    return M


def _both(M, dl, x, algo, glue):
    s = dl.s
    T = x.shape[0]
    res = []
    for noalloc in (False, True):
        out = torch.full((T, s.hidden), float("nan"), device="cuda")
        idx = torch.full((T, s.top_k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, s.top_k), float("nan"), device="cuda")
        r = a = None
        if glue:
            r = torch.randn(T, s.hidden, device="cuda", generator=torch.Generator("cuda").manual_seed(3))
            a = torch.empty(T, s.hidden, dtype=torch.bfloat16, device="cuda")
        if noalloc:
            M.layer_forward_noalloc(x, dl.q, s, out=out, residual=r, next_in=a, topk_idx=idx, topk_w=w, algo=algo)
        else:
            M.layer_forward(x, dl.q, s, out=out, residual=r, next_in=a, topk_idx=idx, topk_w=w, algo=algo,
                            ws=M.alloc_workspace(s, T, algo=algo))
        torch.cuda.synchronize()
        res.append((out, idx, w, r, a))
    (o1, i1, w1, r1, a1), (o2, i2, w2, r2, a2) = res
    assert torch.equal(i1, i2) and torch.equal(w1, w2)
    assert torch.equal(o1, o2)
    assert not torch.isnan(o2).any()
    if glue:
        assert torch.equal(r1, r2) and torch.equal(a1, a2)


@pytest.mark.parametrize("name,algo,T1,T2", [("decode16", "auto", 16, 3), ("decode16", "auto", 9, 1),
                                              ("decode16", "grouped", 149, 40)])
def test_noalloc_matches_layer_forward(name, algo, T1, T2):
    M = _M()
    dl = DeviceLayer(synth.WORKLOADS[name], 0)
    x = synth.tokens(dl.wl, "cuda", n_tokens=T1, layer=5)
    _both(M, dl, x, algo, glue=False)
    _both(M, dl, x[:T2].contiguous(), algo, glue=True)


def test_noalloc_largest_shape_fits():
    """The header's statement of the limit: the full-shape layer fits the
    scratch array up to 149 tokens and not at 150 (argument checks only)."""
    import ctypes
    from bit_quantized_expert_amd import _lib as L
    s = L.Shape(2048, 704, 512, 10, 704, 2)
    limit = 16 << 20
    assert L.lib().moe_workspace_bytes(ctypes.byref(s), 149, None) <= limit
    assert L.lib().moe_workspace_bytes(ctypes.byref(s), 150, None) > limit


def test_noalloc_ragged_and_limit():
    """A ragged shape on both paths, then a request beyond the scratch array:
    refused before any device work, and the array still serves the next call."""
    M = _M()
    wl = synth.custom("na", 256, 192, 33, 8, 96, 3, 64, seed=9, act_dtype=torch.bfloat16, zipf_bias=True)
    dl = DeviceLayer(wl, 0)
    x = synth.tokens(wl, "cuda")
    _both(M, dl, x, "grouped", glue=True)
    _both(M, dl, x[:5].contiguous(), "gemv", glue=False)
    big = synth.tokens(synth.WORKLOADS["decode16"], "cuda", n_tokens=4096)
    dl16 = DeviceLayer(synth.WORKLOADS["decode16"], 0)
    out = torch.empty(4096, 2048, device="cuda")
    with pytest.raises(M.MoeError) as ei:
        M.layer_forward_noalloc(big, dl16.q, dl16.s, out=out)
    assert ei.value.status == -2
    _both(M, dl, x[:7].contiguous(), "auto", glue=False)
