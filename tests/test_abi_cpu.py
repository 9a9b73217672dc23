"""Host-side checks of the C ABI: the library loads, exports every function
the header declares, and rejects bad arguments before any HIP call (these
tests run without a GPU)."""

import ctypes
import os

import pytest

from bit_quantized_expert_amd import _lib as L

if os.environ.get("MOE_ABI_TEST_LIB"):  # the sanitized build (tests/test_abi_sanitized.py)
    L.LIB_PATH = os.environ["MOE_ABI_TEST_LIB"]

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libmoe.so not built")


def _shape(**kw):
    d = dict(hidden=2048, inter=704, n_experts=512, top_k=10, shared_inter=704, qbits=2)
    d.update(kw)
    return L.Shape(**d)


def test_exports_every_header_symbol():
    lib = L.lib()
    names = L.header_symbols()
    assert len(names) == 15
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for code, name in [(0, "MOE_OK"), (-1, "MOE_ERR_INVALID_ARG"), (-2, "MOE_ERR_UNSUPPORTED"),
                       (-3, "MOE_ERR_WORKSPACE"), (-4, "MOE_ERR_DEVICE"), (-5, "MOE_ERR_INDEX")]:
        assert L.status_string(code) == name


def test_workspace_bytes_and_bad_shapes():
    lib = L.lib()
    opts = L.Options(0, 0)
    n1 = lib.moe_workspace_bytes(ctypes.byref(_shape()), 1, ctypes.byref(opts))
    n16 = lib.moe_workspace_bytes(ctypes.byref(_shape()), 16, ctypes.byref(opts))
    assert 0 < n1 < n16
    # the workspace holds at least the sorted expert outputs (P x H fp32)
    assert n16 >= 16 * 10 * 2048 * 4
    for bad in [dict(hidden=100), dict(inter=0), dict(n_experts=0), dict(n_experts=5000), dict(top_k=0),
                dict(top_k=33), dict(qbits=5), dict(qbits=1), dict(shared_inter=48)]:
        assert lib.moe_workspace_bytes(ctypes.byref(_shape(**bad)), 4, ctypes.byref(opts)) == 0, bad
    assert lib.moe_workspace_bytes(ctypes.byref(_shape()), -1, None) == 0


def _layer_struct():
    lay = L.Layer()
    lay.w_router = 0x10000
    lay.router_dtype = 1
    for q in (lay.experts, lay.shared):
        for m in range(3):
            q.codes[m] = 0x20000 + 0x1000 * m
            q.scales[m] = 0x40000 + 0x1000 * m
        q.code_stride = 1_351_680 // 3
        q.scale_stride = 45056
    return lay


def test_validation_before_any_device_call():
    lib = L.lib()
    s = _shape()
    lay = _layer_struct()
    fake = ctypes.c_void_p(0x100000)
    # NULL x
    assert lib.moe_layer_forward(None, 1, 4, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None, None,
                                 None, fake, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    # unsupported qbits
    s4 = _shape(qbits=5)
    assert lib.moe_layer_forward(fake, 1, 4, ctypes.byref(lay), ctypes.byref(s4), fake, None, None, None, None,
                                 None, fake, 1 << 40, None) == L.MOE_ERR_UNSUPPORTED
    # misaligned expert codes
    bad = _layer_struct()
    bad.experts.codes[1] = 0x20008
    assert lib.moe_layer_forward(fake, 1, 4, ctypes.byref(bad), ctypes.byref(s), fake, None, None, None, None,
                                 None, fake, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    assert "16-byte" in L.last_error_detail()
    # workspace too small: reports the bytes needed
    need = lib.moe_workspace_bytes(ctypes.byref(s), 4, None)
    st = lib.moe_layer_forward(fake, 1, 4, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None, None,
                               None, fake, 1024, None)
    assert st == L.MOE_ERR_WORKSPACE
    assert L.last_required_workspace() == need
    assert "MiB short" in L.last_error_detail()
    # activation dtypes: fp32, bf16 and fp16 pass the checks (T == 0 then returns before any device work);
    # another code is refused, and so are fp16 router weights
    for xd in (L.MOE_F32, L.MOE_BF16, L.MOE_F16):
        assert lib.moe_layer_forward(fake, xd, 0, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None,
                                     None, None, None, 0, None) == L.MOE_OK
    assert lib.moe_layer_forward(fake, 3, 4, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None, None,
                                 None, fake, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    assert "x dtype" in L.last_error_detail()
    lay16 = _layer_struct()
    lay16.router_dtype = L.MOE_F16
    assert lib.moe_layer_forward(fake, 1, 4, ctypes.byref(lay16), ctypes.byref(s), fake, None, None, None, None,
                                 None, fake, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    assert "router" in L.last_error_detail()
    # bad options
    o = L.Options(0, 1)
    assert lib.moe_layer_forward(fake, 1, 4, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None, None,
                                 ctypes.byref(o), fake, 1 << 40, None) == L.MOE_ERR_INVALID_ARG
    # next_in without residual
    assert lib.moe_combine(fake, fake, fake, None, 4, ctypes.byref(s), fake, None, fake, None) \
        == L.MOE_ERR_INVALID_ARG
    # T == 0 is a valid no-op
    assert lib.moe_layer_forward(fake, 1, 0, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None, None,
                                 None, None, 0, None) == L.MOE_OK
    assert lib.moe_quantize(None, 0, 64, 2, None, None, None) == L.MOE_OK
    # quantize/dequant argument checks
    assert lib.moe_quantize(fake, 4, 48, 2, fake, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dequant(fake, fake, 4, 64, 5, fake, None) == L.MOE_ERR_UNSUPPORTED
    # permute with a too-small workspace
    assert lib.moe_permute(fake, 4096, ctypes.byref(s), fake, fake, fake, fake, fake, 16, None) \
        == L.MOE_ERR_WORKSPACE
    assert lib.moe_read_error(None, 0, None) == L.MOE_ERR_INVALID_ARG
    # repack argument checks: qbits, cols, NULL, alignment, overlapping buffers (out of place only)
    assert lib.moe_repack(fake, fake, 4, 64, 5, fake, fake, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_repack(fake, fake, 4, 48, 2, fake, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_repack(None, fake, 4, 64, 2, fake, fake, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_repack(ctypes.c_void_p(0x100004), fake, 4, 64, 2, ctypes.c_void_p(0x200000), fake, None) \
        == L.MOE_ERR_INVALID_ARG
    src, dst = 0x100000, 0x100000 + 4 * 64 // 4 - 8   # codes of 4 x 64 2-bit weights: 64 bytes; overlap by 8
    assert lib.moe_repack(ctypes.c_void_p(src), ctypes.c_void_p(0x300000), 4, 64, 2, ctypes.c_void_p(dst),
                          ctypes.c_void_p(0x400000), None) == L.MOE_ERR_INVALID_ARG
    assert "overlap" in L.last_error_detail()
    assert lib.moe_repack(None, None, 0, 64, 2, None, None, None) == L.MOE_OK
    # the no-allocation layer: checks as moe_layer_forward, then the scratch limit, all before any device call
    assert lib.moe_layer_forward_noalloc(None, 1, 4, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None,
                                         None, None, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward_noalloc(fake, 1, 0, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None,
                                         None, None, None) == L.MOE_OK
    assert lib.moe_layer_forward_noalloc(fake, 1, 4096, ctypes.byref(lay), ctypes.byref(s), fake, None, None, None,
                                         None, None, None) == L.MOE_ERR_UNSUPPORTED
    assert "scratch" in L.last_error_detail()
    # the GEMV kernels stage up to 16 token rows of `hidden` in LDS: asked for explicitly where that
    # does not fit (hidden 8192 at 16 tokens), the call is refused before any device work
    big = _shape(hidden=8192)
    lay_big = _layer_struct()
    for q in (lay_big.experts, lay_big.shared):
        q.code_stride = 3 * 704 * 8192 // 4
        q.scale_stride = 3 * 704 * 8192 // 32
    o_gemv = L.Options(1, 0)
    assert lib.moe_layer_forward(fake, 1, 16, ctypes.byref(lay_big), ctypes.byref(big), fake, None, None, None, None,
                                 ctypes.byref(o_gemv), fake, 1 << 40, None) == L.MOE_ERR_UNSUPPORTED
    assert "LDS" in L.last_error_detail()


@pytest.mark.parametrize("rows,K,qbits", [(3, 32, 2), (17, 96, 3), (40, 64, 2), (33, 160, 3), (64, 704, 2),
                                           (5, 96, 4), (48, 704, 4)])
def test_tiled_layout_is_a_permutation(rows, K, qbits):
    """The kernel layout (as the tests restate it) moves every piece of the
    canonical layout to a distinct place, so it keeps the buffer sizes:
    tiling distinct labels gives every label once.  Low planes (and the 4-bit
    second plane) and scales move byte by byte / scale by scale; a 3-bit
    high-plane word moves as a whole, with a bijection of its 32 bits."""
    import numpy as np
    from tests.helpers import _high3_word_bytes, tile_quantised
    n_lo, n_scales = rows * K // 4, rows * K // 32
    lo_planes = 2 if qbits == 4 else 1
    n_codes = rows * K * qbits // 8
    # byte / scale labels of the 2-bit-layout planes
    codes = np.arange(n_codes, dtype=np.int64)
    scales = np.arange(n_scales, dtype=np.int64)
    tc, ts = _tile_positions(codes, scales, rows, K, qbits, tile_quantised)
    assert sorted(tc[:lo_planes * n_lo].tolist()) == list(range(lo_planes * n_lo))
    assert sorted(ts.tolist()) == list(range(n_scales))
    if qbits == 3:
        # word labels of the high plane: a label's bit b fills a whole word (all-ones words are fixed points
        # of the bit rearrangement), so each output word spells the index of its source word
        n_words = rows * K // 32
        got = np.zeros(n_words, np.int64)
        for b in range(max(1, int(n_words - 1).bit_length())):
            hi = np.zeros(n_words * 4, np.uint8)
            for wd in range(n_words):
                if (wd >> b) & 1:
                    hi[4 * wd:4 * wd + 4] = 0xFF
            c = np.concatenate([np.zeros(n_lo, np.uint8), hi])
            out, _ = tile_quantised(c, np.zeros(n_scales, np.uint16), rows, K, 3)
            words = out[n_lo:].reshape(n_words, 4)
            assert np.all((words == 0) | (words == 0xFF))
            got |= (words[:, 0] == 0xFF).astype(np.int64) << b
        assert sorted(got.tolist()) == list(range(n_words))
        # within a word: a bijection of the 32 bit positions
        images = [int.from_bytes(bytes(_high3_word_bytes(np.frombuffer((1 << i).to_bytes(4, "little"), np.uint8))),
                                 "little") for i in range(32)]
        assert all(bin(v).count("1") == 1 for v in images) and len(set(images)) == 32
    # a one-group matrix with K a multiple of 64 keeps each row's 16-byte units in row order
    if rows <= 16 and K % 64 == 0:
        first_unit = tc[:16 * rows].reshape(rows, 16)
        assert np.array_equal(first_unit, np.arange(16)[None, :] + (K // 4) * np.arange(rows)[:, None])


def _tile_positions(codes, scales, rows, K, qbits, tile):
    """tile() on position labels: the helper copies values, so labels that fit
    its dtypes (uint8 bytes / uint16 scales) are tiled in chunks of 256 / 65536.
    (The 3-bit high plane's bits are rearranged within words, so its byte
    labels are not meaningful; the caller checks it separately.)"""
    import numpy as np
    out_c = np.zeros_like(codes)
    out_s = np.zeros_like(scales)
    for shift in range(0, 64, 8):  # byte-plane by byte-plane of the labels
        c8 = ((codes >> shift) & 0xFF).astype(np.uint8)
        s16 = ((scales >> shift) & 0xFF).astype(np.uint16)
        tc, ts = tile(c8, s16, rows, K, qbits)
        out_c |= tc.astype(np.int64) << shift
        out_s |= ts.astype(np.int64) << shift
    return out_c, out_s
