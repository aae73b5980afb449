"""Python binding of libhlq.so, the gfx950 HLQ/HOT linear-layer backward.

Argument marshalling only: every step of the backward runs in the HIP kernels
behind the C ABI declared in ``include/hlq.h``.  torch supplies device memory
and the current stream.  Importing fails loudly when the library has not been
built (``python -m hadamard_rank_linear_amd.build``); there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; HLQ_LIBRARY names another build of the same library
# (for side-by-side timing of two builds)
LIB_PATH = os.environ.get("HLQ_LIBRARY") or os.path.join(HERE, "libhlq.so")

HLQ_F32, HLQ_BF16 = 0, 1
HLQ_PER_TOKEN, HLQ_PER_TENSOR = 0, 1
HLQ_SUM, HLQ_MEAN = 0, 1
STEP_NAMES = ("tr_max", "tr_reduce", "tr_quant", "gemm_gx", "gemm_gw")
HLQ_STEPS_ALL = (1 << len(STEP_NAMES)) - 1

EXPORTED = (
    "hlq_compress_act",
    "hlq_linear_forward",
    "hlq_linear_backward_workspace_size",
    "hlq_linear_backward",
    "hlq_linear_backward_steps",
    "hlq_linear_backward_noalloc",
    "hlq_workspace_layout_query",
    "hlq_gemm_pair_acc",
    "hlq_gemm_gx_acc",
    "hlq_gemm_gw_acc",
    "hlq_conv_backward_workspace_size",
    "hlq_conv_backward",
    "hlq_conv_gemm_acc",
    "hlq_ablation_workspace_size",
    "hlq_linear_backward_ablation",
    "hlq_lqs_workspace_size",
    "hlq_lqs_accumulate",
    "hlq_lqs_select",
    "hlq_status_string",
    "hlq_version",
)


class HLQError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: status {status}: {text}")
        self.status = status


class WorkspaceLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("q_gy", "s_gy", "q_w", "s_w", "q_gyl", "s_gyl", "q_xl", "s_xl")] + [
        ("kx_pitch", ctypes.c_int64), ("kw_pitch", ctypes.c_int64),
        ("t_low", ctypes.c_int64), ("total", ctypes.c_size_t),
        ("partial", ctypes.c_size_t), ("partial_bytes", ctypes.c_size_t),
        ("gx_splits", ctypes.c_int32), ("gw_splits", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m hadamard_rank_linear_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.hlq_compress_act.argtypes = [P, I32, I64, I64, P, P, P]
    lib.hlq_compress_act.restype = I32
    lib.hlq_linear_forward.argtypes = [P, P, I64, I64, I64, P, I32, P, P, P]
    lib.hlq_linear_forward.restype = I32
    lib.hlq_linear_backward_workspace_size.argtypes = [I64, I64, I64, I32, I32]
    lib.hlq_linear_backward_workspace_size.restype = SZ
    lib.hlq_linear_backward.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I32, I32,
                                        I32, I32, I32, P, P, P, SZ, P]
    lib.hlq_linear_backward.restype = I32
    lib.hlq_linear_backward_steps.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I32, I32,
                                              I32, I32, I32, P, P, P, SZ, ctypes.c_uint32, P]
    lib.hlq_linear_backward_steps.restype = I32
    lib.hlq_linear_backward_noalloc.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I32, I32,
                                                I32, I32, I32, P, P, P]
    lib.hlq_linear_backward_noalloc.restype = I32
    lib.hlq_workspace_layout_query.argtypes = [I64, I64, I64, I32, I32,
                                               ctypes.POINTER(WorkspaceLayout)]
    lib.hlq_workspace_layout_query.restype = I32
    lib.hlq_gemm_pair_acc.argtypes = [P, SZ, I64, I64, I64, I32, I32, P, P, P]
    lib.hlq_gemm_pair_acc.restype = I32
    lib.hlq_gemm_gx_acc.argtypes = [P, SZ, I64, I64, I64, I32, I32, P, P]
    lib.hlq_gemm_gx_acc.restype = I32
    lib.hlq_gemm_gw_acc.argtypes = [P, SZ, I64, I64, I64, I32, I32, P, P]
    lib.hlq_gemm_gw_acc.restype = I32
    lib.hlq_conv_backward_workspace_size.argtypes = [I64, I64, I64, I64, I64, I32, I32, I32, I32,
                                                     I32, I32]
    lib.hlq_conv_backward_workspace_size.restype = SZ
    lib.hlq_conv_backward.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I64, I64, I32, I32,
                                      I32, I32, I32, I32, I32, I32, I32, P, P, P, SZ, P]
    lib.hlq_conv_backward.restype = I32
    lib.hlq_conv_gemm_acc.argtypes = [P, SZ, I64, I64, I64, I64, I64, I32, I32, I32, I32, I32,
                                      I32, P, P, P]
    lib.hlq_conv_gemm_acc.restype = I32
    lib.hlq_ablation_workspace_size.argtypes = [I64, I64, I64, I32, I32, I32, I32]
    lib.hlq_ablation_workspace_size.restype = SZ
    lib.hlq_linear_backward_ablation.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I32, I32,
                                                 I32, I32, I32, I32, I32, P, P, P, P, P, SZ, P]
    lib.hlq_linear_backward_ablation.restype = I32
    lib.hlq_lqs_workspace_size.argtypes = [I64, I64, I64, I32, I32]
    lib.hlq_lqs_workspace_size.restype = SZ
    lib.hlq_lqs_accumulate.argtypes = [P, I32, P, P, P, I32, I64, I64, I64, I32, I32, P, P,
                                       SZ, P]
    lib.hlq_lqs_accumulate.restype = I32
    lib.hlq_lqs_select.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_double,
                                   ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]
    lib.hlq_lqs_select.restype = I32
    lib.hlq_status_string.argtypes = [I32]
    lib.hlq_status_string.restype = ctypes.c_char_p
    lib.hlq_version.argtypes = []
    lib.hlq_version.restype = I32
    return lib


_lib = _load()


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise HLQError(fn, status, _lib.hlq_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return HLQ_F32
    if t.dtype == torch.bfloat16:
        return HLQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float32 or bfloat16")


def _require_cuda(*ts):
    dev = None
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"tensors on different devices: {dev} and {t.device}")


def _expect(name, t, dtype, shape):
    """Caller-supplied buffer check: dtype and shape the kernels assume."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _nbytes(t):
    return t.numel() * t.element_size()


def version() -> int:
    return _lib.hlq_version()


def status_string(status: int) -> str:
    return _lib.hlq_status_string(status).decode()


def hlq_compress_act(x, x_codes=None, x_scales=None, stream=None):
    """ACBP: x [T, I] (fp32/bf16, GPU) -> (codes uint8 [T, I/2], scales fp32 [T])."""
    import torch
    T, I = x.shape
    if x_codes is None:
        x_codes = torch.empty((T, I // 2), dtype=torch.uint8, device=x.device)
    if x_scales is None:
        x_scales = torch.empty((T,), dtype=torch.float32, device=x.device)
    _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
    _expect("x_scales", x_scales, torch.float32, (T,))
    _require_cuda(x, x_codes, x_scales)
    _check("hlq_compress_act", _lib.hlq_compress_act(
        _ptr(x), _dtype_code(x), T, I, _ptr(x_codes), _ptr(x_scales), _stream(stream)))
    return x_codes, x_scales


def hlq_linear_forward(x, w, y=None, y_dtype=None, compress=True, x_codes=None,
                       x_scales=None, stream=None):
    """y = x . w^T for bf16 x [T, I] and w [O, I] (I % 32 == 0) on the bf16
    matrix cores; with ``compress`` the same launch also returns the ACBP
    codes / scales of x.  Returns y, or (y, x_codes, x_scales)."""
    import torch
    T, I = x.shape
    O, I2 = w.shape
    if I2 != I:
        raise ValueError("w must be [O, I] with I = x.shape[1]")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("hlq_linear_forward takes bf16 x and w")
    if y is None:
        y = torch.empty((T, O), dtype=y_dtype or torch.bfloat16, device=x.device)
    if y.dtype not in (torch.float32, torch.bfloat16) or tuple(y.shape) != (T, O):
        raise ValueError("y must be a float32 or bfloat16 [T, O] tensor")
    if compress:
        if x_codes is None:
            x_codes = torch.empty((T, I // 2), dtype=torch.uint8, device=x.device)
        if x_scales is None:
            x_scales = torch.empty((T,), dtype=torch.float32, device=x.device)
        _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
        _expect("x_scales", x_scales, torch.float32, (T,))
    else:
        x_codes = x_scales = None
    _require_cuda(x, w, y, x_codes, x_scales)
    _check("hlq_linear_forward", _lib.hlq_linear_forward(
        _ptr(x), _ptr(w), T, I, O, _ptr(y), _dtype_code(y), _ptr(x_codes), _ptr(x_scales),
        _stream(stream)))
    return (y, x_codes, x_scales) if compress else y


def hlq_linear_backward_workspace_size(T, I, O, block, rank) -> int:
    return int(_lib.hlq_linear_backward_workspace_size(T, I, O, block, rank))


def hlq_workspace_layout_query(T, I, O, block, rank) -> dict:
    out = WorkspaceLayout()
    _check("hlq_workspace_layout_query",
           _lib.hlq_workspace_layout_query(T, I, O, block, rank, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in WorkspaceLayout._fields_}


def hlq_linear_backward(g_y, x_codes, x_scales, w, block, rank,
                        gx_mode=HLQ_PER_TOKEN, gw_mode=HLQ_PER_TOKEN, reduction=HLQ_SUM,
                        g_x=None, g_w=None, workspace=None, stream=None, steps=None):
    """HLQ/HOT backward: returns (g_x [T, I], g_w [O, I]) fp32.

    g_y [T, O] and w [O, I] are fp32 or bf16; (x_codes, x_scales) come from
    :func:`hlq_compress_act`.  ``workspace`` is a uint8 GPU tensor of at least
    :func:`hlq_linear_backward_workspace_size` bytes; it is allocated here when
    omitted.  ``steps`` (a bit mask over :data:`STEP_NAMES`) restricts the call
    to those launches (``hlq_linear_backward_steps``).
    """
    import torch
    T, O = g_y.shape
    O2, I = w.shape
    if O2 != O:
        raise ValueError("w must be [O, I] with O = g_y.shape[1]")
    dev = g_y.device
    if g_x is None:
        g_x = torch.empty((T, I), dtype=torch.float32, device=dev)
    if g_w is None:
        g_w = torch.empty((O, I), dtype=torch.float32, device=dev)
    need = hlq_linear_backward_workspace_size(T, I, O, block, rank)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
    _expect("x_scales", x_scales, torch.float32, (T,))
    _expect("g_x", g_x, torch.float32, (T, I))
    _expect("g_w", g_w, torch.float32, (O, I))
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _require_cuda(g_y, x_codes, x_scales, w, g_x, g_w, workspace)
    args = (_ptr(g_y), _dtype_code(g_y), _ptr(x_codes), _ptr(x_scales), _ptr(w),
            _dtype_code(w), T, I, O, block, rank, gx_mode, gw_mode, reduction, _ptr(g_x),
            _ptr(g_w), _ptr(workspace), _nbytes(workspace))
    if steps is None:
        _check("hlq_linear_backward", _lib.hlq_linear_backward(*args, _stream(stream)))
    else:
        _check("hlq_linear_backward_steps",
               _lib.hlq_linear_backward_steps(*args, steps, _stream(stream)))
    return g_x, g_w


def _acc_out(workspace, t, shape):
    import torch
    if t is None:
        t = torch.empty(shape, dtype=torch.int32, device=workspace.device)
    _expect("accumulator", t, torch.int32, shape)
    return t


HLQ_NOALLOC_SCRATCH_BYTES = 64 << 20


def hlq_linear_backward_noalloc(g_y, x_codes, x_scales, w, block, rank, gx_mode=HLQ_PER_TOKEN,
                                gw_mode=HLQ_PER_TOKEN, reduction=HLQ_SUM, g_x=None, g_w=None,
                                stream=None):
    """hlq_linear_backward with the library's static scratch array in place of
    a workspace (no device allocation inside the call; calls that overlap on
    one GPU race).  g_x / g_w are allocated here only when omitted."""
    import torch
    T, O = g_y.shape
    O2, I = w.shape
    if O2 != O:
        raise ValueError("w must be [O, I] with O = g_y.shape[1]")
    dev = g_y.device
    if g_x is None:
        g_x = torch.empty((T, I), dtype=torch.float32, device=dev)
    if g_w is None:
        g_w = torch.empty((O, I), dtype=torch.float32, device=dev)
    _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
    _expect("x_scales", x_scales, torch.float32, (T,))
    _expect("g_x", g_x, torch.float32, (T, I))
    _expect("g_w", g_w, torch.float32, (O, I))
    _require_cuda(g_y, x_codes, x_scales, w, g_x, g_w)
    _check("hlq_linear_backward_noalloc", _lib.hlq_linear_backward_noalloc(
        _ptr(g_y), _dtype_code(g_y), _ptr(x_codes), _ptr(x_scales), _ptr(w), _dtype_code(w),
        T, I, O, block, rank, gx_mode, gw_mode, reduction, _ptr(g_x), _ptr(g_w),
        _stream(stream)))
    return g_x, g_w


def hlq_gemm_pair_acc(workspace, T, I, O, block, rank, acc_x=None, acc_w=None, stream=None):
    """INT32 accumulators (acc_x [T, I], acc_w [O, I]) of the one GEMM launch
    hlq_linear_backward runs, from a workspace it has filled."""
    acc_x = _acc_out(workspace, acc_x, (T, I))
    acc_w = _acc_out(workspace, acc_w, (O, I))
    _require_cuda(workspace, acc_x, acc_w)
    _check("hlq_gemm_pair_acc", _lib.hlq_gemm_pair_acc(
        _ptr(workspace), _nbytes(workspace), T, I, O, block, rank, _ptr(acc_x), _ptr(acc_w),
        _stream(stream)))
    return acc_x, acc_w


def hlq_gemm_gx_acc(workspace, T, I, O, block, rank, acc_x=None, stream=None):
    acc_x = _acc_out(workspace, acc_x, (T, I))
    _require_cuda(workspace, acc_x)
    _check("hlq_gemm_gx_acc", _lib.hlq_gemm_gx_acc(
        _ptr(workspace), _nbytes(workspace), T, I, O, block, rank, _ptr(acc_x), _stream(stream)))
    return acc_x


def hlq_gemm_gw_acc(workspace, T, I, O, block, rank, acc_w=None, stream=None):
    acc_w = _acc_out(workspace, acc_w, (O, I))
    _require_cuda(workspace, acc_w)
    _check("hlq_gemm_gw_acc", _lib.hlq_gemm_gw_acc(
        _ptr(workspace), _nbytes(workspace), T, I, O, block, rank, _ptr(acc_w), _stream(stream)))
    return acc_w


def hlq_conv_backward_workspace_size(N, H, W, C, O, R, S, stride, pad, block, rank) -> int:
    return int(_lib.hlq_conv_backward_workspace_size(N, H, W, C, O, R, S, stride, pad, block,
                                                     rank))


def _conv_out(H, R, stride, pad):
    return (H + 2 * pad - R) // stride + 1


def hlq_conv_backward(g_y, x_codes, x_scales, w, N, H, W, C, R, S, stride, pad, block, rank,
                      gx_mode=HLQ_PER_TENSOR, gw_mode=HLQ_PER_TOKEN, reduction=HLQ_SUM,
                      g_x=None, g_w=None, workspace=None, stream=None):
    """HLQ/HOT backward of a 2-D convolution: returns (g_x [N*H*W, C],
    g_w [O, R*S*C]) fp32.  g_y [N*P*Q, O] (rows (n, p, q)); (x_codes,
    x_scales) = hlq_compress_act of x as [N*H*W, C]; w [O, R*S*C] (OHWI)."""
    import torch
    P, Q = _conv_out(H, R, stride, pad), _conv_out(W, S, stride, pad)
    T, O = g_y.shape
    if T != N * P * Q or tuple(w.shape) != (O, R * S * C):
        raise ValueError("g_y must be [N*P*Q, O] and w [O, R*S*C]")
    dev = g_y.device
    if g_x is None:
        g_x = torch.empty((N * H * W, C), dtype=torch.float32, device=dev)
    if g_w is None:
        g_w = torch.empty((O, R * S * C), dtype=torch.float32, device=dev)
    need = hlq_conv_backward_workspace_size(N, H, W, C, O, R, S, stride, pad, block, rank)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _expect("x_codes", x_codes, torch.uint8, (N * H * W, C // 2))
    _expect("x_scales", x_scales, torch.float32, (N * H * W,))
    _expect("g_x", g_x, torch.float32, (N * H * W, C))
    _expect("g_w", g_w, torch.float32, (O, R * S * C))
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _require_cuda(g_y, x_codes, x_scales, w, g_x, g_w, workspace)
    _check("hlq_conv_backward", _lib.hlq_conv_backward(
        _ptr(g_y), _dtype_code(g_y), _ptr(x_codes), _ptr(x_scales), _ptr(w), _dtype_code(w),
        N, H, W, C, O, R, S, stride, pad, block, rank, gx_mode, gw_mode, reduction, _ptr(g_x),
        _ptr(g_w), _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return g_x, g_w


def hlq_conv_gemm_acc(workspace, N, H, W, C, O, R, S, stride, pad, block, rank, stream=None):
    """INT32 accumulators (acc_x [N*H*W, C], acc_w [O, R*S*C]) of the
    convolution backward's GEMMs, from a workspace it has filled."""
    acc_x = _acc_out(workspace, None, (N * H * W, C))
    acc_w = _acc_out(workspace, None, (O, R * S * C))
    _require_cuda(workspace, acc_x, acc_w)
    _check("hlq_conv_gemm_acc", _lib.hlq_conv_gemm_acc(
        _ptr(workspace), _nbytes(workspace), N, H, W, C, O, R, S, stride, pad, block, rank,
        _ptr(acc_x), _ptr(acc_w), _stream(stream)))
    return acc_x, acc_w


HLQ_VAR_HQ4, HLQ_VAR_Q4, HLQ_VAR_HLA8_INT, HLQ_VAR_HLA8_EXT = 0, 1, 2, 3
VARIANT_NAMES = ("hq4", "q4", "hla8_int", "hla8_ext")


def hlq_ablation_workspace_size(T, I, O, block, rank, gx_variant, gw_variant) -> int:
    return int(_lib.hlq_ablation_workspace_size(T, I, O, block, rank, gx_variant, gw_variant))


def hlq_linear_backward_ablation(g_y, x_codes, x_scales, w, block, rank, gx_variant, gw_variant,
                                 gx_mode=HLQ_PER_TOKEN, gw_mode=HLQ_PER_TOKEN,
                                 reduction=HLQ_SUM, want_acc=False, stream=None):
    """The backward under an ablation variant per path (HLQ_VAR_*; names in
    VARIANT_NAMES).  Returns (g_x, g_w) fp32, plus (acc_x, acc_w) INT32 when
    want_acc."""
    import torch
    T, O = g_y.shape
    O2, I = w.shape
    if O2 != O:
        raise ValueError("w must be [O, I] with O = g_y.shape[1]")
    dev = g_y.device
    _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
    _expect("x_scales", x_scales, torch.float32, (T,))
    g_x = torch.empty((T, I), dtype=torch.float32, device=dev)
    g_w = torch.empty((O, I), dtype=torch.float32, device=dev)
    ext = HLQ_VAR_HLA8_EXT
    acc_x = acc_w = None
    if want_acc:
        acc_x = torch.empty((T // block * rank if gx_variant == ext else T, I),
                            dtype=torch.int32, device=dev)
        acc_w = torch.empty((O // block * rank if gw_variant == ext else O, I),
                            dtype=torch.int32, device=dev)
    need = hlq_ablation_workspace_size(T, I, O, block, rank, gx_variant, gw_variant)
    ws = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _require_cuda(g_y, x_codes, x_scales, w, g_x, g_w, ws, acc_x, acc_w)
    _check("hlq_linear_backward_ablation", _lib.hlq_linear_backward_ablation(
        _ptr(g_y), _dtype_code(g_y), _ptr(x_codes), _ptr(x_scales), _ptr(w), _dtype_code(w),
        T, I, O, block, rank, gx_variant, gw_variant, gx_mode, gw_mode, reduction, _ptr(g_x),
        _ptr(g_w), _ptr(acc_x), _ptr(acc_w), _ptr(ws), _nbytes(ws), _stream(stream)))
    return (g_x, g_w, acc_x, acc_w) if want_acc else (g_x, g_w)


HLQ_LQS_STATS = 16
HLQ_LQS_THRESHOLD = 0.5


def hlq_lqs_workspace_size(T, I, O, block, rank) -> int:
    return int(_lib.hlq_lqs_workspace_size(T, I, O, block, rank))


def hlq_lqs_accumulate(g_y, x_codes, x_scales, w, block, rank, stats=None, workspace=None,
                       stream=None):
    """Add one calibration batch to the layer-wise quantizer selection
    statistics: ``stats`` is a float64 GPU tensor of 16 values (zeros when
    omitted), returned.  Same inputs as :func:`hlq_linear_backward`."""
    import torch
    T, O = g_y.shape
    O2, I = w.shape
    if O2 != O:
        raise ValueError("w must be [O, I] with O = g_y.shape[1]")
    dev = g_y.device
    if stats is None:
        stats = torch.zeros((HLQ_LQS_STATS,), dtype=torch.float64, device=dev)
    if stats.dtype != torch.float64 or stats.numel() != HLQ_LQS_STATS:
        raise ValueError("stats must be a float64 tensor of 16 values")
    need = hlq_lqs_workspace_size(T, I, O, block, rank)
    if workspace is None:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    _expect("x_codes", x_codes, torch.uint8, (T, I // 2))
    _expect("x_scales", x_scales, torch.float32, (T,))
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _require_cuda(g_y, x_codes, x_scales, w, stats, workspace)
    _check("hlq_lqs_accumulate", _lib.hlq_lqs_accumulate(
        _ptr(g_y), _dtype_code(g_y), _ptr(x_codes), _ptr(x_scales), _ptr(w), _dtype_code(w),
        T, I, O, block, rank, _ptr(stats), _ptr(workspace),
        _nbytes(workspace), _stream(stream)))
    return stats


def hlq_lqs_select(stats, threshold=HLQ_LQS_THRESHOLD):
    """(gx_mode, gw_mode) from 16 statistics (any host sequence or tensor)."""
    if hasattr(stats, "detach"):
        stats = stats.detach().cpu().tolist()
    vals = [float(v) for v in stats]
    if len(vals) != HLQ_LQS_STATS:
        raise ValueError("expected 16 statistics")
    arr = (ctypes.c_double * HLQ_LQS_STATS)(*vals)
    gx, gw = ctypes.c_int(-1), ctypes.c_int(-1)
    _check("hlq_lqs_select", _lib.hlq_lqs_select(arr, float(threshold), ctypes.byref(gx),
                                                 ctypes.byref(gw)))
    return gx.value, gw.value


def lib_handle():
    """The loaded ctypes library (for tests of the raw C ABI)."""
    return _lib
