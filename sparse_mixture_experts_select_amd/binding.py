"""Thin ctypes binding of libmoe_ffn.so (``include/moe_ffn.h``).

Same entry-point names as the C ABI.  The functions take torch tensors that
live on the GPU, check their shapes and dtypes, and pass raw device pointers
and the current HIP stream to the library; every step of the layer runs in
the library's HIP kernels.  Importing this module loads the library and
raises ``ImportError`` if it has not been built
(``python -m sparse_mixture_experts_select_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_build", "libmoe_ffn.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_HIP = 3
MOE_ERR_OUT_OF_MEMORY = 4
MOE_DTYPE_BF16 = 0
MOE_DTYPE_F32 = 1
MOE_NUM_STAGES = 7

STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_HIP", 4: "MOE_ERR_OUT_OF_MEMORY"}

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe_ffn.so is not built (expected at %s); run "
                      "`python -m sparse_mixture_experts_select_amd.build`" % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class MoeFfnOpts(ctypes.Structure):
    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("router_bias", _P),
        ("topk_ids", _P),
        ("topk_weights", _P),
        ("expert_counts", _P),
        ("expert_offsets", _P),
        ("row_token", _P),
        ("slot_row", _P),
        ("h_out", _P),
        ("y_out", _P),
        ("residual", _P),
        ("workspace", _P),
        ("workspace_bytes", ctypes.c_size_t),
        ("rmsnorm_input", ctypes.c_int32),
        ("rmsnorm_eps", ctypes.c_float),
        ("x_norm_out", _P),
    ]


_FWD_ARGS = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P]
lib.moe_ffn_forward.argtypes = _FWD_ARGS
lib.moe_ffn_forward.restype = ctypes.c_int
lib.moe_ffn_forward_f32.argtypes = _FWD_ARGS
lib.moe_ffn_forward_f32.restype = ctypes.c_int
lib.moe_ffn_forward_ex.argtypes = _FWD_ARGS + [ctypes.POINTER(MoeFfnOpts)]
lib.moe_ffn_forward_ex.restype = ctypes.c_int
lib.moe_ffn_forward_noalloc.argtypes = _FWD_ARGS + [ctypes.POINTER(MoeFfnOpts)]
lib.moe_ffn_forward_noalloc.restype = ctypes.c_int
lib.moe_ffn_noalloc_scratch_bytes.argtypes = []
lib.moe_ffn_noalloc_scratch_bytes.restype = ctypes.c_size_t
lib.moe_ffn_workspace_bytes.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int32]
lib.moe_ffn_workspace_bytes.restype = ctypes.c_size_t
lib.moe_rmsnorm.argtypes = [_P, _P, _I64, _I64, ctypes.c_float, ctypes.c_int32, _P]
lib.moe_rmsnorm.restype = ctypes.c_int
lib.moe_ffn_last_error.argtypes = []
lib.moe_ffn_last_error.restype = ctypes.c_char_p
lib.moe_ffn_release_workspace.argtypes = []
lib.moe_ffn_release_workspace.restype = None
lib.moe_ffn_profile_begin.argtypes = [ctypes.c_int32, ctypes.c_uint32]
lib.moe_ffn_profile_begin.restype = ctypes.c_int
lib.moe_ffn_profile_end.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int32)]
lib.moe_ffn_profile_end.restype = ctypes.c_int
lib.moe_ffn_stage_name.argtypes = [ctypes.c_int32]
lib.moe_ffn_stage_name.restype = ctypes.c_char_p
lib.moe_ffn_version.argtypes = []
lib.moe_ffn_version.restype = ctypes.c_char_p
lib.moe_hbm_read_probe.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32, _P, _P]
lib.moe_hbm_read_probe.restype = ctypes.c_int
lib.moe_mfma_probe.argtypes = [_P, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
lib.moe_mfma_probe.restype = ctypes.c_int


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))
        self.status = status


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, moe_ffn_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return MOE_DTYPE_BF16
    if dt == torch.float32:
        return MOE_DTYPE_F32
    raise TypeError("tensors must be bfloat16 or float32, got %s" % dt)


def _shapes(x, w_router, w1, w3, w2):
    for name, t in (("x", x), ("w_router", w_router), ("w1", w1), ("w3", w3), ("w2", w2)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
    T, d = x.shape
    E, d1, f = w1.shape
    if w_router.shape != (d, E) or w3.shape != (E, d, f) or w2.shape != (E, f, d) or d1 != d:
        raise ValueError("expected x [T,d], w_router [d,E], w1/w3 [E,d,f], w2 [E,f,d]; got %s %s %s %s %s"
                         % (tuple(x.shape), tuple(w_router.shape), tuple(w1.shape), tuple(w3.shape),
                            tuple(w2.shape)))
    dts = {t.dtype for t in (x, w_router, w1, w3, w2)}
    if len(dts) != 1:
        raise TypeError("x and all weights must share one dtype")
    return T, d, f, E


def moe_ffn_forward(x, w_router, w1, w3, w2, k, out=None, stream=None):
    """The layer in bfloat16 (fp32 accumulation); returns ``out`` [T,d]."""
    T, d, f, E = _shapes(x, w_router, w1, w3, w2)
    if x.dtype != torch.bfloat16:
        raise TypeError("moe_ffn_forward takes bfloat16 tensors")
    if out is None:
        out = torch.empty_like(x)
    _check(lib.moe_ffn_forward(_ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3), _ptr(w2),
                               T, d, f, E, k, _ptr(out), _stream(stream)))
    return out


def moe_ffn_forward_f32(x, w_router, w1, w3, w2, k, out=None, stream=None):
    """The layer in binary32; returns ``out`` [T,d]."""
    T, d, f, E = _shapes(x, w_router, w1, w3, w2)
    if x.dtype != torch.float32:
        raise TypeError("moe_ffn_forward_f32 takes float32 tensors")
    if out is None:
        out = torch.empty_like(x)
    _check(lib.moe_ffn_forward_f32(_ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3), _ptr(w2),
                                   T, d, f, E, k, _ptr(out), _stream(stream)))
    return out


def _forward_with_opts(fn, x, w_router, w1, w3, w2, k, out, stream, router_bias, topk_ids,
                       topk_weights, expert_counts, expert_offsets, row_token, slot_row, h_out,
                       y_out, residual, workspace, rmsnorm_eps, x_norm_out):
    T, d, f, E = _shapes(x, w_router, w1, w3, w2)
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.dtype != x.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like x")
    R = T * k
    i32, f32 = torch.int32, torch.float32
    # (tensor, element count, dtype) the library reads or writes for each option
    spec = {
        "router_bias": (router_bias, E, f32), "topk_ids": (topk_ids, R, i32),
        "topk_weights": (topk_weights, R, f32), "expert_counts": (expert_counts, E, i32),
        "expert_offsets": (expert_offsets, E + 1, i32), "row_token": (row_token, R, i32),
        "slot_row": (slot_row, R, i32), "h_out": (h_out, R * f, x.dtype),
        "y_out": (y_out, R * d, f32), "residual": (residual, T * d, x.dtype),
        "x_norm_out": (x_norm_out, T * d, x.dtype),
    }
    if x_norm_out is not None and rmsnorm_eps is None:
        raise ValueError("x_norm_out needs rmsnorm_eps")
    opts = MoeFfnOpts()
    opts.dtype = _dtype_code(x.dtype)
    for name, (t, n, dt) in spec.items():
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % name)
        if t.numel() != n or t.dtype != dt:
            raise ValueError("%s must hold %d elements of %s (got %d of %s)"
                             % (name, n, dt, t.numel(), t.dtype))
        setattr(opts, name, t.data_ptr())
    if workspace is not None:
        opts.workspace = workspace.data_ptr()
        opts.workspace_bytes = workspace.numel() * workspace.element_size()
    if rmsnorm_eps is not None:
        opts.rmsnorm_input = 1
        opts.rmsnorm_eps = float(rmsnorm_eps)
    _check(fn(_ptr(x), _ptr(w_router), _ptr(w1), _ptr(w3), _ptr(w2), T, d, f, E, k, _ptr(out),
              _stream(stream), ctypes.byref(opts)))
    return out


def moe_ffn_forward_ex(x, w_router, w1, w3, w2, k, out=None, stream=None, *, router_bias=None,
                       topk_ids=None, topk_weights=None, expert_counts=None, expert_offsets=None,
                       row_token=None, slot_row=None, h_out=None, y_out=None, residual=None,
                       workspace=None, rmsnorm_eps=None, x_norm_out=None):
    """The layer with options (see ``moe_ffn_opts_t``); every tensor option is
    a GPU tensor or None.  ``rmsnorm_eps`` set: x is the residual stream h and
    the layer runs on RMSNorm(h) (formed by the router; ``x_norm_out``, if
    given, receives it).  Returns ``out``."""
    return _forward_with_opts(lib.moe_ffn_forward_ex, x, w_router, w1, w3, w2, k, out, stream,
                              router_bias, topk_ids, topk_weights, expert_counts, expert_offsets,
                              row_token, slot_row, h_out, y_out, residual, workspace, rmsnorm_eps,
                              x_norm_out)


def moe_ffn_forward_noalloc(x, w_router, w1, w3, w2, k, out=None, stream=None, *, router_bias=None,
                            topk_ids=None, topk_weights=None, expert_counts=None,
                            expert_offsets=None, row_token=None, slot_row=None, h_out=None,
                            y_out=None, residual=None, rmsnorm_eps=None, x_norm_out=None):
    """moe_ffn_forward_ex working in the library's static scratch (no
    allocation; see the header).  ``out`` should be given by callers that
    cannot allocate (None allocates it here, as torch.empty_like(x))."""
    return _forward_with_opts(lib.moe_ffn_forward_noalloc, x, w_router, w1, w3, w2, k, out, stream,
                              router_bias, topk_ids, topk_weights, expert_counts, expert_offsets,
                              row_token, slot_row, h_out, y_out, residual, None, rmsnorm_eps,
                              x_norm_out)


def moe_ffn_noalloc_scratch_bytes() -> int:
    return int(lib.moe_ffn_noalloc_scratch_bytes())


def moe_ffn_workspace_bytes(T, d, f, E, k, dtype=MOE_DTYPE_BF16) -> int:
    return int(lib.moe_ffn_workspace_bytes(T, d, f, E, k, dtype))


def moe_rmsnorm(h, x=None, eps=1e-5, stream=None):
    """Unit-gain RMSNorm of each row of h [T,d]; returns x."""
    if not h.is_cuda or not h.is_contiguous():
        raise ValueError("h must be a contiguous GPU tensor")
    if x is None:
        x = torch.empty_like(h)
    T, d = h.shape
    _check(lib.moe_rmsnorm(_ptr(h), _ptr(x), T, d, float(eps), _dtype_code(h.dtype), _stream(stream)))
    return x


def moe_hbm_read_probe(buf, blocks, sink, stream=None) -> None:
    """Enqueue one streaming read of the whole GPU tensor ``buf`` (see the
    header); ``sink`` is a one-element int32 GPU tensor."""
    if not buf.is_cuda or not buf.is_contiguous() or not sink.is_cuda or sink.dtype != torch.int32:
        raise ValueError("buf must be a contiguous GPU tensor and sink an int32 GPU tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(lib.moe_hbm_read_probe(_ptr(buf), nbytes, int(blocks), _ptr(sink), _stream(stream)))


def moe_mfma_probe(ops, iters, blocks, sink, clocks=None, stream=None) -> None:
    """Enqueue the MFMA probe (see the header) on the contiguous GPU tensor
    ``ops``; ``sink`` is a one-element int32 GPU tensor, ``clocks`` an
    optional int64 GPU tensor of 2 * blocks elements."""
    if not ops.is_cuda or not ops.is_contiguous() or not sink.is_cuda or sink.dtype != torch.int32:
        raise ValueError("ops must be a contiguous GPU tensor and sink an int32 GPU tensor")
    if clocks is not None and (not clocks.is_cuda or clocks.dtype != torch.int64
                               or clocks.numel() < 2 * blocks):
        raise ValueError("clocks must be an int64 GPU tensor of at least 2 * blocks elements")
    nbytes = ops.numel() * ops.element_size()
    _check(lib.moe_mfma_probe(_ptr(ops), nbytes, int(iters), int(blocks), _ptr(sink), _ptr(clocks),
                              _stream(stream)))


def moe_ffn_last_error() -> str:
    return lib.moe_ffn_last_error().decode()


def moe_ffn_release_workspace() -> None:
    lib.moe_ffn_release_workspace()


def moe_ffn_version() -> str:
    return lib.moe_ffn_version().decode()


def moe_ffn_profile_begin(max_calls: int, stages=None) -> None:
    """Time the given stages (names or indices; None = all) of the next
    max_calls forward calls."""
    mask = 0
    for s in stages or ():
        i = s if isinstance(s, int) else [moe_ffn_stage_name(j) for j in range(MOE_NUM_STAGES)].index(s)
        mask |= 1 << i
    _check(lib.moe_ffn_profile_begin(max_calls, mask))


def moe_ffn_profile_end():
    """Returns ({stage name: summed ms} for the timed stages, number of
    recorded calls)."""
    ms = (ctypes.c_float * MOE_NUM_STAGES)()
    calls = ctypes.c_int32(0)
    _check(lib.moe_ffn_profile_end(ms, ctypes.byref(calls)))
    return ({moe_ffn_stage_name(i): float(ms[i]) for i in range(MOE_NUM_STAGES) if ms[i] >= 0},
            int(calls.value))


def moe_ffn_stage_name(i: int) -> str:
    return lib.moe_ffn_stage_name(i).decode()
