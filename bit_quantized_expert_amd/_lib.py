"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: torch tensors become device pointers, a torch
stream becomes a hipStream_t, structs are filled in.  Every step of the layer
runs in the library's HIP kernels.  There is no fallback: if the library is
missing or the GPU is absent, calls fail loudly.
"""

from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "moe.h")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE, MOE_ERR_INDEX = 0, -1, -2, -3, -4, -5
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
ALGO = {"auto": 0, "gemv": 1, "grouped": 2}
FFN_REUSE_PLAN, FFN_SKIP_GATEUP, FFN_SKIP_DOWN = 1, 2, 4
ROUTE_TAIL_SKIP = 8  # moe_layer_forward option: the verify-window route tail skip


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what} failed: {status_string(status)} ({detail})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("qbits", ctypes.c_int32)]

    @classmethod
    def of(cls, s) -> "Shape":
        return cls(s.hidden, s.inter, s.n_experts, s.top_k, s.shared_inter, s.qbits)


class QWeights(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p * 3), ("scales", ctypes.c_void_p * 3),
                ("code_stride", ctypes.c_int64), ("scale_stride", ctypes.c_int64)]


class Layer(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_dtype", ctypes.c_int), ("router_bias", ctypes.c_void_p),
                ("experts", QWeights), ("shared", QWeights)]


class Options(ctypes.Structure):
    _fields_ = [("ffn_algo", ctypes.c_int), ("flags", ctypes.c_int32)]


_lib = None

_VP, _I64, _I32, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "moe_workspace_bytes": (_SZ, [_VP, _I64, _VP]),
    "moe_route": (ctypes.c_int, [_VP, ctypes.c_int, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_permute": (ctypes.c_int, [_VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_expert_ffn": (ctypes.c_int, [_VP, ctypes.c_int, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "moe_combine": (ctypes.c_int, [_VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP]),
    "moe_layer_forward": (ctypes.c_int, [_VP, ctypes.c_int, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ,
                                         _VP]),
    "moe_layer_forward_noalloc": (ctypes.c_int, [_VP, ctypes.c_int, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                 _VP]),
    "moe_rmsnorm_bf16": (ctypes.c_int, [_VP, _I64, _I32, _VP, _VP]),
    "moe_dequant": (ctypes.c_int, [_VP, _VP, _I64, _I32, _I32, _VP, _VP]),
    "moe_quantize": (ctypes.c_int, [_VP, _I64, _I32, _I32, _VP, _VP, _VP]),
    "moe_repack": (ctypes.c_int, [_VP, _VP, _I64, _I32, _I32, _VP, _VP, _VP]),
    "moe_read_error": (ctypes.c_int, [_VP, _SZ, _VP]),
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error_detail": (ctypes.c_char_p, []),
    "moe_last_required_workspace": (_SZ, []),
}


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built by bit_quantized_expert_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m bit_quantized_expert_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_symbols() -> list[str]:
    """Names of the functions declared in include/moe.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(moe_\w+)\s*\(", text, flags=re.M)))


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def last_error_detail() -> str:
    return lib().moe_last_error_detail().decode()


def last_required_workspace() -> int:
    return int(lib().moe_last_required_workspace())


def _check(status: int, what: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, what, last_error_detail())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensor arguments must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float16:
        return MOE_F16
    raise ValueError(f"unsupported activation dtype {t.dtype}")


def _opts(algo: str, flags: int = 0) -> Options:
    return Options(ALGO[algo], flags)


# ------------------------------------------------------------------ arenas

class QArena:
    """Quantised weights of `n` experts, one contiguous tensor per matrix:
    codes[m] is uint8 [n, bytes_per_expert], scales[m] is int16 (fp16 bits)
    [n, scales_per_expert]; m = 0 gate [inter][H], 1 up [inter][H], 2 down
    [H][inter]."""

    def __init__(self, n: int, hidden: int, inter: int, qbits: int, device):
        self.n, self.hidden, self.inter, self.qbits = n, hidden, inter, qbits
        shapes = [(inter, hidden), (inter, hidden), (hidden, inter)]
        self.codes = [torch.empty(n, r * k * qbits // 8, dtype=torch.uint8, device=device) for r, k in shapes]
        self.scales = [torch.empty(n, r * (k // 32), dtype=torch.int16, device=device) for r, k in shapes]
        self.mat_shapes = shapes

    def c_struct(self) -> QWeights:
        q = QWeights()
        for m in range(3):
            q.codes[m] = self.codes[m].data_ptr()
            q.scales[m] = self.scales[m].data_ptr()
        q.code_stride = self.codes[0].shape[1]
        q.scale_stride = self.scales[0].shape[1]
        assert all(c.shape[1] == q.code_stride for c in self.codes)
        assert all(s.shape[1] == q.scale_stride for s in self.scales)
        return q

    def quantize_from(self, m: int, w: torch.Tensor, experts: slice | None = None, stream=None) -> None:
        """Quantise fp32 weights w [n_sel, rows, K] of matrix m into the arena
        (experts `experts`, default all): moe_quantize into the canonical
        layout, then moe_repack into the kernel layout the arena holds."""
        rows, k = self.mat_shapes[m]
        lo = 0 if experts is None else experts.start
        n = w.shape[0]
        if w.shape[1:] != (rows, k) or w.dtype != torch.float32:
            raise ValueError(f"expected fp32 [n, {rows}, {k}], got {tuple(w.shape)} {w.dtype}")
        w = w.contiguous()
        codes = torch.empty(n, self.codes[m].shape[1], dtype=torch.uint8, device=w.device)
        scales = torch.empty(n, self.scales[m].shape[1], dtype=torch.int16, device=w.device)
        if self.qbits == 2:
            quantize(w.view(n * rows, k), 2, codes, scales, stream=stream)
        else:
            # the 3- and 4-bit planes are per matrix, so each expert is one call
            for i in range(n):
                quantize(w[i], self.qbits, codes[i], scales[i], stream=stream)
        self.load_canonical(m, lo, codes, scales, stream=stream)

    def load_canonical(self, m: int, first: int, codes: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
        """Repack canonical-layout codes uint8 [n, bytes] and scales int16
        [n, count] of matrix m of experts first .. first + n - 1 into the
        arena."""
        rows, k = self.mat_shapes[m]
        n = codes.shape[0]
        if self.qbits == 2 and rows % 16 == 0:
            # one plane, and no row group straddles two experts: the stacked matrices repack as one
            repack(codes.reshape(-1), scales.reshape(-1), n * rows, k, 2, self.codes[m][first:first + n].reshape(-1),
                   self.scales[m][first:first + n].reshape(-1), stream=stream)
            return
        for i in range(n):
            repack(codes[i], scales[i], rows, k, self.qbits, self.codes[m][first + i], self.scales[m][first + i],
                   stream=stream)

    def bytes(self) -> int:
        return sum(c.numel() for c in self.codes) + 2 * sum(s.numel() for s in self.scales)


class QLayer:
    """A layer's device tensors: router weights/bias and the quantised routed
    and shared experts."""

    def __init__(self, w_router: torch.Tensor, bias: torch.Tensor | None, experts: QArena, shared: QArena | None):
        self.w_router, self.bias, self.experts, self.shared = w_router, bias, experts, shared
        self._c = None

    def c_struct(self) -> Layer:
        if self._c is None:
            L = Layer()
            L.w_router = _ptr(self.w_router)
            L.router_dtype = _dtype_code(self.w_router)
            L.router_bias = _ptr(self.bias)
            L.experts = self.experts.c_struct()
            if self.shared is not None:
                L.shared = self.shared.c_struct()
            self._c = L
        return self._c


# ------------------------------------------------------------------ entry points

def workspace_bytes(shape, T: int, algo: str = "auto") -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(Shape.of(shape)), T, ctypes.byref(_opts(algo)))
    if n == 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_workspace_bytes", last_error_detail())
    return int(n)


def alloc_workspace(shape, T: int, device="cuda", algo: str = "auto") -> torch.Tensor:
    return torch.empty(workspace_bytes(shape, T, algo), dtype=torch.uint8, device=device)


def _ws(ws):
    return (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())


def route(x, layer: QLayer, shape, topk_idx, topk_w, logits=None, ws=None, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_route(_ptr(x), _dtype_code(x), x.shape[0], ctypes.byref(layer.c_struct()),
                           ctypes.byref(Shape.of(shape)), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), wp, wn,
                           _stream(stream)), "moe_route")


def permute(topk_idx, T: int, shape, counts, offsets, sorted_pair, pair_pos, ws, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_permute(_ptr(topk_idx), T, ctypes.byref(Shape.of(shape)), _ptr(counts), _ptr(offsets),
                             _ptr(sorted_pair), _ptr(pair_pos), wp, wn, _stream(stream)), "moe_permute")


def expert_ffn(x, layer: QLayer, shape, offsets, sorted_pair, y_sorted, shared_out=None, algo="auto", ws=None,
               stream=None, flags: int = 0) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_expert_ffn(_ptr(x), _dtype_code(x), x.shape[0], ctypes.byref(layer.c_struct()),
                                ctypes.byref(Shape.of(shape)), _ptr(offsets), _ptr(sorted_pair), _ptr(y_sorted),
                                _ptr(shared_out), ctypes.byref(_opts(algo, flags)), wp, wn, _stream(stream)),
           "moe_expert_ffn")


def combine(y_sorted, pair_pos, topk_w, shared_out, T: int, shape, out=None, residual=None, next_in=None,
            stream=None) -> None:
    _check(lib().moe_combine(_ptr(y_sorted), _ptr(pair_pos), _ptr(topk_w), _ptr(shared_out), T,
                             ctypes.byref(Shape.of(shape)), _ptr(out), _ptr(residual), _ptr(next_in),
                             _stream(stream)), "moe_combine")


def layer_forward(x, layer: QLayer, shape, out=None, residual=None, next_in=None, topk_idx=None, topk_w=None,
                  algo="auto", ws=None, stream=None, flags: int = 0) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_layer_forward(_ptr(x), _dtype_code(x), x.shape[0], ctypes.byref(layer.c_struct()),
                                   ctypes.byref(Shape.of(shape)), _ptr(out), _ptr(residual), _ptr(next_in),
                                   _ptr(topk_idx), _ptr(topk_w), ctypes.byref(_opts(algo, flags)), wp, wn,
                                   _stream(stream)), "moe_layer_forward")


def layer_forward_noalloc(x, layer: QLayer, shape, out=None, residual=None, next_in=None, topk_idx=None,
                          topk_w=None, algo="auto", stream=None, flags: int = 0) -> None:
    """moe_layer_forward without a workspace argument (the library's own
    per-GPU scratch array; shapes up to MOE_NOALLOC_SCRATCH_BYTES of
    workspace)."""
    _check(lib().moe_layer_forward_noalloc(_ptr(x), _dtype_code(x), x.shape[0], ctypes.byref(layer.c_struct()),
                                           ctypes.byref(Shape.of(shape)), _ptr(out), _ptr(residual), _ptr(next_in),
                                           _ptr(topk_idx), _ptr(topk_w), ctypes.byref(_opts(algo, flags)),
                                           _stream(stream)),
           "moe_layer_forward_noalloc")


def rmsnorm_bf16(r, a, stream=None) -> None:
    _check(lib().moe_rmsnorm_bf16(_ptr(r), r.shape[0], r.shape[1], _ptr(a), _stream(stream)), "moe_rmsnorm_bf16")


def dequant(codes, scales, rows: int, cols: int, qbits: int, out, stream=None) -> None:
    _check(lib().moe_dequant(_ptr(codes), _ptr(scales), rows, cols, qbits, _ptr(out), _stream(stream)),
           "moe_dequant")


def quantize(w, qbits: int, codes, scales, stream=None) -> None:
    rows, cols = w.shape
    if codes.numel() < rows * cols * qbits // 8 or scales.numel() < rows * cols // 32:
        raise ValueError("codes/scales buffers are too small")
    _check(lib().moe_quantize(_ptr(w), rows, cols, qbits, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize")


def repack(codes, scales, rows: int, cols: int, qbits: int, packed_codes, packed_scales, stream=None) -> None:
    if min(codes.numel(), packed_codes.numel()) < rows * cols * qbits // 8 or \
            min(scales.numel(), packed_scales.numel()) < rows * cols // 32:
        raise ValueError("codes/scales buffers are too small")
    _check(lib().moe_repack(_ptr(codes), _ptr(scales), rows, cols, qbits, _ptr(packed_codes), _ptr(packed_scales),
                            _stream(stream)), "moe_repack")


def read_error(ws, stream=None) -> None:
    wp, wn = _ws(ws)
    _check(lib().moe_read_error(wp, wn, _stream(stream)), "moe_read_error")
