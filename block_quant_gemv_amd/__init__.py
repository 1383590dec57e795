"""Python binding of libqgemv.so, the block-quantized decode GEMV library
for AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/qgemv.h and include/qattn.h. Tensors are torch
tensors on the GPU; streams are torch's current stream. There is no CPU
fallback: importing this package raises if the library is missing, and every
call raises RuntimeError on a non-zero status.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first; the library then binds to it

__all__ = ["FORMATS", "GEMV", "FFN", "MoE", "Attention", "debug_quantize", "debug_quantize_s16",
           "clear_launch_cache", "debug_stream_read", "lib_path", "LAYOUT_VERSION"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMV_LIBRARY: path of another build of the same library (the host-sanitized
# one of the ABI tests); the in-tree build otherwise.
_LIB = os.environ.get("QGEMV_LIBRARY") or os.path.join(_HERE, "libqgemv.so")
LAYOUT_VERSION = 1

FORMATS = {"f32": 0, "q4_0": 1, "q8_0": 2, "q4_k": 3, "q6_k": 4, "iq4_nl": 5, "q5_k": 6, "iq4_xs": 7}
_KIND = {"gemv": 0, "ffn": 1, "moe": 2}


def lib_path() -> str:
    return _LIB


if not os.path.exists(_LIB):
    raise ImportError(
        f"{_LIB} is not built; run `python block_quant_gemv_amd/build.py` "
        "(or __graft_entry__.build()) first")

_lib = ctypes.CDLL(_LIB)


class _Desc(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32), ("layout_version", ctypes.c_int32),
        ("fmt", ctypes.c_int32), ("max_m", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("fmt_gateup", ctypes.c_int32), ("fmt_down", ctypes.c_int32),
        ("hidden", ctypes.c_int64), ("inter", ctypes.c_int64),
        ("n_experts", ctypes.c_int64), ("top_k", ctypes.c_int32),
        ("fmt_expert", ctypes.c_int32),
        ("codebook16", ctypes.POINTER(ctypes.c_int8)),
    ]


_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64
_lib.qgemv_create.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_Desc)]
_lib.qgemv_destroy.argtypes = [_vp]
_lib.qgemv_workspace_size.argtypes = [_vp, _i32, ctypes.POINTER(_sz)]
_lib.qgemv_workspace_offset.argtypes = [_vp, _i32, ctypes.c_char_p, ctypes.POINTER(_sz)]
_lib.qgemv_weight_bytes.argtypes = [_vp, _i32, ctypes.POINTER(_sz)]
_lib.qgemv_run.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.qffn_run.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.qmoe_run.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.qmoe_run_s16.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.qgemv_quantize.argtypes = [_vp, _vp, _i32, _vp, _sz, _vp]
_lib.qgemv_run_quantized.argtypes = [_vp, _vp, _vp, _i32, _vp, _sz, _vp]
_lib.qgemv_status_string.argtypes = [_i32]
_lib.qgemv_status_string.restype = ctypes.c_char_p
_lib.qgemv_last_error.restype = ctypes.c_char_p
_lib.qgemv_debug_quantize.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _vp]
_lib.qgemv_debug_block_dots.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp, ctypes.c_size_t, _vp]
_lib.qgemv_workspace_size_s16.argtypes = [_vp, ctypes.POINTER(_sz)]
_lib.qgemv_run_s16.argtypes = [_vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.qgemv_run_f32act.argtypes = [_vp, _vp, _vp, _vp, ctypes.c_int, _vp]
_lib.qgemv_debug_quantize_s16.argtypes = [_vp, _vp, _vp, _vp, _i32, _i64, _vp]
_lib.qgemv_debug_block_dots_s16.argtypes = [_vp, _vp, _vp, _vp, _vp]
_lib.qgemv_debug_clear_launch_cache.argtypes = []
_lib.qgemv_run_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i32, _vp]
_lib.qgemv_debug_stream_read.argtypes = [_vp, _sz, _vp, _vp]
_lib.qattn_workspace_size.argtypes = [_i32, _i32, _i32, _i64, ctypes.POINTER(_sz)]
_lib.qattn_decode.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _i64, _vp, _sz, _vp]
for _f in ("qgemv_debug_stream_read", "qgemv_run_noalloc", "qgemv_debug_clear_launch_cache", "qmoe_run_s16", "qgemv_workspace_size_s16", "qgemv_run_s16", "qgemv_run_f32act", "qgemv_debug_quantize_s16", "qgemv_debug_block_dots_s16",
           "qattn_workspace_size", "qattn_decode", "qgemv_create", "qgemv_destroy", "qgemv_workspace_size", "qgemv_workspace_offset",
           "qgemv_weight_bytes", "qgemv_run", "qgemv_quantize", "qgemv_run_quantized", "qffn_run", "qmoe_run", "qgemv_debug_quantize",
           "qgemv_debug_block_dots"):
    getattr(_lib, _f).restype = ctypes.c_int


class QgemvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.qgemv_status_string(status).decode()
        detail = _lib.qgemv_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}): {detail}")


def _check(rc: int, where: str):
    if rc != 0:
        raise QgemvError(rc, where)


def _fmt_id(f):
    if isinstance(f, str):
        return FORMATS[f.lower()]
    return int(f)


def _dev(t: torch.Tensor, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class _Plan:
    def __init__(self, desc: _Desc):
        h = _vp()
        _check(_lib.qgemv_create(ctypes.byref(h), ctypes.byref(desc)), "qgemv_create")
        self._h = h
        self.max_m = desc.max_m
        self._ws = {}

    def close(self):
        if getattr(self, "_h", None):
            _lib.qgemv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, m: int) -> int:
        b = _sz()
        _check(_lib.qgemv_workspace_size(self._h, m, ctypes.byref(b)), "qgemv_workspace_size")
        return b.value

    def workspace_offset(self, m: int, name: str) -> int:
        b = _sz()
        _check(_lib.qgemv_workspace_offset(self._h, m, name.encode(), ctypes.byref(b)),
               "qgemv_workspace_offset")
        return b.value

    def weight_bytes(self, which: int = 0) -> int:
        b = _sz()
        _check(_lib.qgemv_weight_bytes(self._h, which, ctypes.byref(b)), "qgemv_weight_bytes")
        return b.value

    def workspace(self, m: int, device=None) -> torch.Tensor:
        """A cached workspace tensor for m tokens (reused across calls)."""
        device = torch.device(device or torch.cuda.current_device())
        key = (device.index, m)
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(self.workspace_size(m), dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws

    def ws_view(self, ws: torch.Tensor, m: int, name: str, dtype, count: int) -> torch.Tensor:
        """View of a named workspace region as a 1-D tensor of `count` items."""
        off = self.workspace_offset(m, name)
        isz = torch.empty((), dtype=dtype).element_size()
        return ws[off:off + count * isz].view(dtype)

    def _check_w(self, w, which, name):
        _dev(w, torch.uint8, name)
        cache = self.__dict__.setdefault("_wb", {})
        need = cache.get(which)
        if need is None:
            need = cache[which] = self.weight_bytes(which)
        if w.numel() < need:
            raise ValueError(f"{name} has {w.numel()} bytes, needs {need}")
        return w.data_ptr()


class GEMV(_Plan):
    """y[m, n] = W[n, k] . x[m, k] with W packed in `fmt` blocks."""

    def __init__(self, fmt, n: int, k: int, max_m: int = 1, codebook=None):
        d = _Desc()
        d.kind, d.layout_version, d.fmt, d.max_m, d.n, d.k = 0, LAYOUT_VERSION, _fmt_id(fmt), max_m, n, k
        self._cb = None
        if codebook is not None:
            cb = [int(v) for v in codebook]
            self._cb = (ctypes.c_int8 * 16)(*cb)
            d.codebook16 = ctypes.cast(self._cb, ctypes.POINTER(ctypes.c_int8))
        super().__init__(d)
        self.fmt, self.n, self.k = _fmt_id(fmt), n, k

    def run(self, w, x, y=None, ws=None, stream=None):
        m = x.shape[0] if x.dim() == 2 else 1
        if x.dim() not in (1, 2) or x.shape[-1] != self.k:
            raise ValueError(f"x must be [m, {self.k}]")
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        if y.numel() != m * self.n:
            raise ValueError("y has the wrong size")
        if ws is None:
            ws = self.workspace(m, x.device)
        wp = self._check_w(w, 0, "w")
        _check(_lib.qgemv_run(self._h, wp, _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"), m,
                              _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "qgemv_run")
        return y

    def run_noalloc(self, w, x, y=None, stream=None):
        """qgemv_run with the library's fixed device scratch as the workspace
        (qgemv_run_noalloc): no device allocation by the library; calls that
        overlap on one GPU race."""
        m = x.shape[0] if x.dim() == 2 else 1
        if x.dim() not in (1, 2) or x.shape[-1] != self.k:
            raise ValueError(f"x must be [m, {self.k}]")
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        if y.numel() != m * self.n:
            raise ValueError("y has the wrong size")
        _check(_lib.qgemv_run_noalloc(self._h, self._check_w(w, 0, "w"), _dev(x, torch.float32, "x"),
                                      _dev(y, torch.float32, "y"), m, _stream(stream)), "qgemv_run_noalloc")
        return y

    def quantize(self, x, ws=None, stream=None):
        """Quantize x[m, k] into the workspace (first half of run)."""
        m = x.shape[0]
        if ws is None:
            ws = self.workspace(m, x.device)
        _check(_lib.qgemv_quantize(self._h, _dev(x, torch.float32, "x"), m, _dev(ws, torch.uint8, "ws"),
                                   ws.numel(), _stream(stream)), "qgemv_quantize")
        return ws

    def run_quantized(self, w, ws, m, y=None, stream=None):
        """GEMV on activations already quantized into ws (second half of run)."""
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=ws.device)
        _check(_lib.qgemv_run_quantized(self._h, self._check_w(w, 0, "w"), _dev(y, torch.float32, "y"), m,
                                        _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
               "qgemv_run_quantized")
        return y

    def workspace_size_s16(self) -> int:
        b = _sz()
        _check(_lib.qgemv_workspace_size_s16(self._h, ctypes.byref(b)), "qgemv_workspace_size_s16")
        return b.value

    def workspace_s16(self, device="cuda") -> torch.Tensor:
        return torch.empty(self.workspace_size_s16(), dtype=torch.uint8, device=device)

    def run_s16(self, w, x, y=None, ws=None, stream=None):
        """One token with 16-bit activation codes (qgemv_run_s16)."""
        if x.numel() != self.k:
            raise ValueError(f"x must hold one token of {self.k} values")
        if y is None:
            y = torch.empty((1, self.n), dtype=torch.float32, device=x.device)
        if y.numel() != self.n:
            raise ValueError("y has the wrong size")
        if ws is None:
            ws = self.workspace_s16(x.device)
        _check(_lib.qgemv_run_s16(self._h, self._check_w(w, 0, "w"), _dev(x, torch.float32, "x"),
                                  _dev(y, torch.float32, "y"), _dev(ws, torch.uint8, "ws"), ws.numel(),
                                  _stream(stream)), "qgemv_run_s16")
        return y

    def run_f32act(self, w, x, y=None, stream=None):
        """y[m, n] with fp32 activations, no activation quantization (qgemv_run_f32act; Q4_0 / Q8_0)."""
        m = x.shape[0] if x.dim() == 2 else 1
        if x.dim() not in (1, 2) or x.shape[-1] != self.k:
            raise ValueError(f"x must be [m, {self.k}]")
        if y is None:
            y = torch.empty((m, self.n), dtype=torch.float32, device=x.device)
        if y.numel() != m * self.n:
            raise ValueError("y has the wrong size")
        _check(_lib.qgemv_run_f32act(self._h, self._check_w(w, 0, "w"), _dev(x, torch.float32, "x"),
                                     _dev(y, torch.float32, "y"), m, _stream(stream)), "qgemv_run_f32act")
        return y

    def block_dots_s16(self, w, xq, stream=None):
        """Exact per-sub-block int32 dots with 16-bit codes xq int16 [k] (checking export)."""
        dots = torch.empty((self.n, self.k // 32), dtype=torch.int32, device=xq.device)
        _check(_lib.qgemv_debug_block_dots_s16(self._h, self._check_w(w, 0, "w"), _dev(xq, torch.int16, "xq"),
                                               _dev(dots, torch.int32, "dots"), _stream(stream)),
               "qgemv_debug_block_dots_s16")
        return dots

    def block_dots(self, w, xq, stream=None):
        """Exact per-block int32 dot products (checking export)."""
        m = xq.shape[0]
        g = 16 if self.fmt == FORMATS["q6_k"] else 32
        dots = torch.empty((m, self.n, self.k // g), dtype=torch.int32, device=xq.device)
        wp = self._check_w(w, 0, "w")
        ws = self.workspace(m, device=xq.device)
        _check(_lib.qgemv_debug_block_dots(self._h, wp, _dev(xq, torch.int8, "xq"),
                                           _dev(dots, torch.int32, "dots"), m, ws.data_ptr(), ws.numel(),
                                           _stream(stream)),
               "qgemv_debug_block_dots")
        return dots


class FFN(_Plan):
    """Fused FFN sublayer: down(silu(gate(x)) * up(x)), one stream, one workspace."""

    def __init__(self, hidden: int, inter: int, fmt_gateup="q4_k", fmt_down="q6_k", max_m: int = 1,
                 codebook=None):
        d = _Desc()
        d.kind, d.layout_version, d.max_m = 1, LAYOUT_VERSION, max_m
        d.fmt_gateup, d.fmt_down, d.hidden, d.inter = _fmt_id(fmt_gateup), _fmt_id(fmt_down), hidden, inter
        self._cb = None
        if codebook is not None:
            self._cb = (ctypes.c_int8 * 16)(*[int(v) for v in codebook])
            d.codebook16 = ctypes.cast(self._cb, ctypes.POINTER(ctypes.c_int8))
        super().__init__(d)
        self.hidden, self.inter = hidden, inter

    def run(self, w_gateup, w_down, x, y=None, ws=None, stream=None):
        m = x.shape[0]
        if x.shape[-1] != self.hidden:
            raise ValueError(f"x must be [m, {self.hidden}]")
        if y is None:
            y = torch.empty((m, self.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = self.workspace(m, x.device)
        _check(_lib.qffn_run(self._h, self._check_w(w_gateup, 0, "w_gateup"), self._check_w(w_down, 1, "w_down"),
                             _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"), m,
                             _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "qffn_run")
        return y


class MoE(_Plan):
    """MoE layer: fp32 router, top-k softmax, routed experts + shared expert."""

    def __init__(self, hidden: int, inter: int, n_experts: int, top_k: int, fmt_expert="q4_0",
                 max_m: int = 1, codebook=None):
        d = _Desc()
        d.kind, d.layout_version, d.max_m = 2, LAYOUT_VERSION, max_m
        d.hidden, d.inter, d.n_experts, d.top_k, d.fmt_expert = hidden, inter, n_experts, top_k, _fmt_id(fmt_expert)
        self._cb = None
        if codebook is not None:
            self._cb = (ctypes.c_int8 * 16)(*[int(v) for v in codebook])
            d.codebook16 = ctypes.cast(self._cb, ctypes.POINTER(ctypes.c_int8))
        super().__init__(d)
        self.hidden, self.inter, self.n_experts, self.top_k = hidden, inter, n_experts, top_k

    def run(self, w_router, w_gateup, w_down, w_shared_gateup, w_shared_down, x, y=None, ws=None,
            stream=None, s16=False):
        """One MoE layer (qmoe_run; with s16=True, qmoe_run_s16: 16-bit activations)."""
        m = x.shape[0]
        if x.shape[-1] != self.hidden:
            raise ValueError(f"x must be [m, {self.hidden}]")
        if tuple(w_router.shape) != (self.n_experts, self.hidden):
            raise ValueError("router must be [n_experts, hidden] fp32")
        if y is None:
            y = torch.empty((m, self.hidden), dtype=torch.float32, device=x.device)
        if ws is None:
            ws = self.workspace(m, x.device)
        fn = _lib.qmoe_run_s16 if s16 else _lib.qmoe_run
        _check(fn(self._h, _dev(w_router, torch.float32, "w_router"),
                  self._check_w(w_gateup, 0, "w_gateup"), self._check_w(w_down, 1, "w_down"),
                  self._check_w(w_shared_gateup, 2, "w_shared_gateup"),
                  self._check_w(w_shared_down, 3, "w_shared_down"),
                  _dev(x, torch.float32, "x"), _dev(y, torch.float32, "y"), m,
                  _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)),
               "qmoe_run_s16" if s16 else "qmoe_run")
        return y


def debug_quantize(x: torch.Tensor, stream=None):
    """Device activation quantizer alone: returns (xq int8, dx fp32, sx int32)."""
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int8, device=x.device)
    dx = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    sx = torch.empty((m, k // 32), dtype=torch.int32, device=x.device)
    _check(_lib.qgemv_debug_quantize(_dev(x, torch.float32, "x"), xq.data_ptr(), dx.data_ptr(), sx.data_ptr(),
                                     m, k, _stream(stream)), "qgemv_debug_quantize")
    return xq, dx, sx


def debug_quantize_s16(x: torch.Tensor, stream=None):
    """Device 16-bit activation quantizer alone: returns (xq int16, dx fp32, sx int32)."""
    m, k = x.shape
    xq = torch.empty((m, k), dtype=torch.int16, device=x.device)
    dx = torch.empty((m, k // 32), dtype=torch.float32, device=x.device)
    sx = torch.empty((m, k // 32), dtype=torch.int32, device=x.device)
    _check(_lib.qgemv_debug_quantize_s16(_dev(x, torch.float32, "x"), xq.data_ptr(), dx.data_ptr(), sx.data_ptr(),
                                         m, k, _stream(stream)), "qgemv_debug_quantize_s16")
    return xq, dx, sx


def clear_launch_cache():
    """Forget the library's cached launch facts (per-device CU counts and
    kernel residencies): the next launch of each kernel queries them again."""
    _check(_lib.qgemv_debug_clear_launch_cache(), "qgemv_debug_clear_launch_cache")


def debug_stream_read(buf: torch.Tensor, out: torch.Tensor, stream=None):
    """Read buf (a contiguous GPU tensor, 16-byte multiple) once with the
    GEMVs' load shape (qgemv_debug_stream_read); out: one int32 on the GPU."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _check(_lib.qgemv_debug_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                        _dev(out, torch.int32, "out"), _stream(stream)),
           "qgemv_debug_stream_read")


class Attention:
    """Decode attention of one token over an fp16 KV cache (qattn_decode):
    q fp32 [n_heads, head_dim], caches fp16 [n_kv_heads, n_ctx, head_dim]."""

    def __init__(self, n_heads: int, n_kv_heads: int, head_dim: int):
        self.n_heads, self.n_kv_heads, self.head_dim = n_heads, n_kv_heads, head_dim

    def workspace_size(self, n_ctx: int) -> int:
        b = _sz()
        _check(_lib.qattn_workspace_size(self.n_heads, self.n_kv_heads, self.head_dim, n_ctx, ctypes.byref(b)),
               "qattn_workspace_size")
        return b.value

    def workspace(self, n_ctx: int, device="cuda") -> torch.Tensor:
        return torch.empty(max(1, self.workspace_size(n_ctx)), dtype=torch.uint8, device=device)

    def run(self, q, k_cache, v_cache, out=None, ws=None, stream=None):
        n_ctx = k_cache.shape[1] if k_cache.dim() == 3 else 0
        if k_cache.shape != (self.n_kv_heads, n_ctx, self.head_dim) or v_cache.shape != k_cache.shape:
            raise ValueError("k_cache and v_cache must be [n_kv_heads, n_ctx, head_dim]")
        if q.shape != (self.n_heads, self.head_dim):
            raise ValueError("q must be [n_heads, head_dim]")
        if out is None:
            out = torch.empty((self.n_heads, self.head_dim), dtype=torch.float32, device=q.device)
        if ws is None:
            ws = self.workspace(n_ctx, q.device)
        _check(_lib.qattn_decode(_dev(q, torch.float32, "q"), _dev(k_cache, torch.float16, "k_cache"),
                                 _dev(v_cache, torch.float16, "v_cache"), _dev(out, torch.float32, "out"),
                                 self.n_heads, self.n_kv_heads, self.head_dim, n_ctx,
                                 _dev(ws, torch.uint8, "ws"), ws.numel(), _stream(stream)), "qattn_decode")
        return out
