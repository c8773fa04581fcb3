"""MI355X (gfx950) chunked gated-delta-rule forward pass: Python binding.

A thin ctypes layer over ``libgdn.so`` (the C ABI of ``include/gdn.h``): it
checks tensor shapes/dtypes/devices (the C side only sees pointers), allocates
outputs and workspace with torch (device memory and streams are torch's
plumbing), and passes pointers. Every step of the computation runs in the HIP
kernels. Importing this module fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK = 0
GDN_ERR_INVALID_ARGUMENT = 1
GDN_ERR_UNSUPPORTED = 2
GDN_ERR_HIP = 3

GDN_L2NORM_QK = 1
GDN_BETA_SIGMOID = 2
GDN_OUTPUT_FINAL_STATE = 4

CHUNK = 64
HEAD_DIM = 128
VEC_ROWS = 8

EXPORTED = (
    "gdn_last_error", "gdn_num_chunks", "gdn_chunk_fwd_workspace_bytes", "kda_chunk_fwd_workspace_bytes",
    "gdn_chunk_fwd", "kda_chunk_fwd", "gdn_stage_prepare", "gdn_stage_fwd_h", "gdn_stage_finalize",
    "gdn_timing_enable", "gdn_timing_read", "gdn_state_summary", "kda_state_summary",
    "gdn_state_summary_workspace_bytes", "gdn_state_summary_apply", "gdn_short_conv",
    "gdn_short_conv_workspace_bytes", "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes",
    "gdn_bwd_timing_read", "gdn_chunk_fwd_gated", "kda_chunk_fwd_gated", "gdn_chunk_bwd_gated",
    "gdn_state_summary_gated", "kda_bwd_state_pass", "kda_bwd_state_pass_workspace_bytes",
    "kda_chunk_bwd", "kda_chunk_bwd_gated", "kda_chunk_bwd_workspace_bytes", "gdn_chunk_fwd_noalloc",
)


class GdnError(RuntimeError):
    """A non-zero status from the library; ``code`` is the GDN_ERR_* value."""

    def __init__(self, code: int, message: str):
        super().__init__("gdn status %d: %s" % (code, message))
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libgdn.so not found at %s; build it with `python -m chunked_gated_delta_03_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, u32, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_num_chunks.restype = ctypes.c_int
    lib.gdn_num_chunks.argtypes = [i32, i32, i32, p, ctypes.POINTER(ctypes.c_int64)]
    for name in ("gdn_chunk_fwd_workspace_bytes", "kda_chunk_fwd_workspace_bytes"):
        fn = getattr(lib, name)
        fn.restype = sz
        fn.argtypes = [i32, i32, i32, i32, i32, i32, p, u32]
    for name in ("gdn_chunk_fwd", "kda_chunk_fwd"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p, p, sz, p]
    lib.gdn_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdn_chunk_fwd_noalloc.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p, p]
    for name in ("gdn_chunk_fwd_gated", "kda_chunk_fwd_gated"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p, p, sz, p]
    lib.gdn_timing_enable.restype = ctypes.c_int
    lib.gdn_timing_enable.argtypes = [i32]
    lib.gdn_timing_read.restype = ctypes.c_int
    lib.gdn_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int64)]
    lib.gdn_state_summary_gated.restype = ctypes.c_int
    lib.gdn_state_summary_gated.argtypes = [i32, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, u32, p, p,
                                            p, sz, p]
    for name in ("gdn_state_summary", "kda_state_summary"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, u32, p, p, p, sz, p]
    lib.gdn_state_summary_workspace_bytes.restype = sz
    lib.gdn_state_summary_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32, p]
    lib.gdn_state_summary_apply.restype = ctypes.c_int
    lib.gdn_state_summary_apply.argtypes = [p, p, p, p, i32, i32, i32, i32, p]
    lib.gdn_short_conv_workspace_bytes.restype = sz
    lib.gdn_short_conv_workspace_bytes.argtypes = [i32, p]
    lib.gdn_short_conv.restype = ctypes.c_int
    lib.gdn_short_conv.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, i32, p, p, sz, p]
    lib.gdn_bwd_timing_read.restype = ctypes.c_int
    lib.gdn_bwd_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.gdn_chunk_bwd_workspace_bytes.restype = sz
    lib.gdn_chunk_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, p, u32]
    lib.gdn_chunk_bwd.restype = ctypes.c_int
    lib.gdn_chunk_bwd.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p,
                                  p, p, p, p, p, p, p, sz, p]
    lib.gdn_chunk_bwd_gated.restype = ctypes.c_int
    lib.gdn_chunk_bwd_gated.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p,
                                        p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_bwd_workspace_bytes.restype = sz
    lib.kda_chunk_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, p, u32]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p,
                                  p, p, p, p, p, p, p, sz, p]
    lib.kda_chunk_bwd_gated.restype = ctypes.c_int
    lib.kda_chunk_bwd_gated.argtypes = [p, p, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p,
                                        p, p, p, p, p, p, p, p, p, sz, p]
    lib.kda_bwd_state_pass_workspace_bytes.restype = sz
    lib.kda_bwd_state_pass_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, p, u32]
    lib.kda_bwd_state_pass.restype = ctypes.c_int
    lib.kda_bwd_state_pass.argtypes = [p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p, p, p, p, p, sz,
                                       p]
    lib.gdn_stage_prepare.restype = ctypes.c_int
    lib.gdn_stage_prepare.argtypes = [i32, p, p, p, p, p, i32, i32, i32, i32, i32, i32, f32, u32, p, p, p, p, p]
    lib.gdn_stage_fwd_h.restype = ctypes.c_int
    lib.gdn_stage_fwd_h.argtypes = [i32, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, u32, p, p, p, p]
    lib.gdn_stage_finalize.restype = ctypes.c_int
    lib.gdn_stage_finalize.argtypes = [i32, p, p, p, p, p, p, p, i32, i32, i32, i32, i32, i32, p, p]
    return lib


lib = _load()


def last_error() -> str:
    return lib.gdn_last_error().decode()


def _check(rc: int) -> None:
    if rc != GDN_OK:
        raise GdnError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(device: torch.device, stream=None):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _cu_array(cu_seqlens) -> Optional[np.ndarray]:
    if cu_seqlens is None:
        return None
    if isinstance(cu_seqlens, torch.Tensor):
        if cu_seqlens.device.type != "cpu":
            raise ValueError("cu_seqlens must be a host (CPU) tensor or sequence")
        cu_seqlens = cu_seqlens.numpy()
    arr = np.asarray(cu_seqlens)
    if arr.ndim != 1 or not np.issubdtype(arr.dtype, np.integer):
        raise ValueError("cu_seqlens must be a one-dimensional integer array")
    if arr.size and (arr.min() < np.iinfo(np.int32).min or arr.max() > np.iinfo(np.int32).max):
        raise ValueError("cu_seqlens values exceed int32")
    return np.ascontiguousarray(arr, dtype=np.int32)


def _cu_ptr(cu: Optional[np.ndarray]):
    return None if cu is None else cu.ctypes.data_as(ctypes.c_void_p)


def _flags(l2norm_qk: bool, beta_sigmoid: bool, output_final_state: bool) -> int:
    return ((GDN_L2NORM_QK if l2norm_qk else 0) | (GDN_BETA_SIGMOID if beta_sigmoid else 0)
            | (GDN_OUTPUT_FINAL_STATE if output_final_state else 0))


def num_chunks(B: int, T: int, cu_seqlens=None) -> int:
    cu = _cu_array(cu_seqlens)
    n = ctypes.c_int64(0)
    _check(lib.gdn_num_chunks(B, T, B if cu is None else len(cu) - 1, _cu_ptr(cu), ctypes.byref(n)))
    return int(n.value)


def _check_inputs(q, k, v, g, beta, kda: bool, initial_state, cu):
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("beta", beta, torch.bfloat16), ("g", g, torch.float32)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if t.dtype != dt:
            raise ValueError("%s must be %s (got %s)" % (name, dt, t.dtype))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.device.type != "cuda":
            raise ValueError("%s must be on the GPU" % name)
        if t.device != q.device:
            raise ValueError("%s is on %s, q on %s" % (name, t.device, q.device))
    if q.dim() != 4:
        raise ValueError("q must have shape [B,T,H,K]")
    B, T, H, K = q.shape
    V = v.shape[-1]
    if tuple(k.shape) != (B, T, H, K) or tuple(v.shape) != (B, T, H, V) or tuple(beta.shape) != (B, T, H):
        raise ValueError("shape mismatch: q %s k %s v %s beta %s" % (tuple(q.shape), tuple(k.shape),
                                                                    tuple(v.shape), tuple(beta.shape)))
    gshape = (B, T, H, K) if kda else (B, T, H)
    if tuple(g.shape) != gshape:
        raise ValueError("g must have shape %s (got %s)" % (gshape, tuple(g.shape)))
    N = B if cu is None else len(cu) - 1
    if initial_state is not None:
        if (initial_state.dtype != torch.float32 or not initial_state.is_contiguous()
                or tuple(initial_state.shape) != (N, H, K, V) or initial_state.device != q.device):
            raise ValueError("initial_state must be a contiguous fp32 [N,H,K,V] = %s tensor on %s"
                             % ((N, H, K, V), q.device))
    return B, T, H, K, V, N


def _check_gate_params(kda, q, A_log, dt_bias, H, K):
    for name, t, shape in (("A_log", A_log, (H,)), ("dt_bias", dt_bias, (H, K) if kda else (H,))):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s must be a torch tensor" % name)
        if t.dtype != torch.float32 or not t.is_contiguous() or t.device != q.device:
            raise ValueError("%s must be a contiguous fp32 tensor on %s" % (name, q.device))
        if tuple(t.shape) != shape:
            raise ValueError("%s must have shape %s (got %s)" % (name, shape, tuple(t.shape)))


def _chunk_fwd(kda, q, k, v, g, beta, scale, initial_state, cu_seqlens, l2norm_qk, beta_sigmoid,
               output_final_state, workspace, stream, A_log=None, dt_bias=None):
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(q, k, v, g, beta, kda, initial_state, cu)
    gated = A_log is not None or dt_bias is not None
    if gated:
        _check_gate_params(kda, q, A_log, dt_bias, H, K)
    scale = K ** -0.5 if scale is None else float(scale)
    flags = _flags(l2norm_qk, beta_sigmoid, output_final_state)
    o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=q.device)
    fs = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device) if output_final_state else None
    wsfn = lib.kda_chunk_fwd_workspace_bytes if kda else lib.gdn_chunk_fwd_workspace_bytes
    need = wsfn(B, T, H, K, V, N, _cu_ptr(cu), flags)
    if need == 0:
        workspace = None  # invalid arguments: the call below reports the precise status
    elif workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(), need))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gated:
        fn = lib.kda_chunk_fwd_gated if kda else lib.gdn_chunk_fwd_gated
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(beta), _ptr(initial_state),
                  _cu_ptr(cu), N, B, T, H, K, V, scale, flags, _ptr(o), _ptr(fs), _ptr(workspace), ws_bytes,
                  _stream_ptr(q.device, stream)))
    else:
        fn = lib.kda_chunk_fwd if kda else lib.gdn_chunk_fwd
        _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _cu_ptr(cu), N,
                  B, T, H, K, V, scale, flags, _ptr(o), _ptr(fs), _ptr(workspace), ws_bytes,
                  _stream_ptr(q.device, stream)))
    return o, fs


def gdn_chunk_fwd(q, k, v, g, beta, scale: Optional[float] = None, initial_state=None, cu_seqlens=None,
                  l2norm_qk: bool = False, beta_sigmoid: bool = False, output_final_state: bool = True,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """GDN forward. q,k,v bf16 [B,T,H,128], g fp32 [B,T,H] (natural log),
    beta bf16 [B,T,H]. Returns (o bf16 [B,T,H,128], final_state fp32 [N,H,128,128] or None)."""
    return _chunk_fwd(False, q, k, v, g, beta, scale, initial_state, cu_seqlens, l2norm_qk, beta_sigmoid,
                      output_final_state, workspace, stream)


NOALLOC_SCRATCH_BYTES = 128 << 20


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, scale: Optional[float] = None, initial_state=None,
                          l2norm_qk: bool = False, beta_sigmoid: bool = False, output_final_state: bool = True,
                          stream=None, out: Optional[Tuple[torch.Tensor, Optional[torch.Tensor]]] = None):
    """GDN forward through the entry that allocates nothing (dense input only;
    intermediates in the library's fixed device scratch of
    NOALLOC_SCRATCH_BYTES). ``out`` = (o, final_state) preallocated by the
    caller (final_state may be None without output_final_state); else this
    binding allocates them with torch. Returns (o, final_state)."""
    B, T, H, K, V, N = _check_inputs(q, k, v, g, beta, False, initial_state, None)
    scale = K ** -0.5 if scale is None else float(scale)
    flags = _flags(l2norm_qk, beta_sigmoid, output_final_state)
    if out is None:
        o = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=q.device)
        fs = torch.empty((N, H, K, V), dtype=torch.float32, device=q.device) if output_final_state else None
    else:
        o, fs = out
        if (o.dtype != torch.bfloat16 or not o.is_contiguous() or tuple(o.shape) != (B, T, H, V)
                or o.device != q.device):
            raise ValueError("o must be a contiguous bf16 [B,T,H,V] tensor on %s" % q.device)
        if output_final_state and (fs is None or fs.dtype != torch.float32 or not fs.is_contiguous()
                                   or tuple(fs.shape) != (N, H, K, V) or fs.device != q.device):
            raise ValueError("final_state must be a contiguous fp32 [N,H,K,V] tensor on %s" % q.device)
    _check(lib.gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), None, N,
                                     B, T, H, K, V, scale, flags, _ptr(o), _ptr(fs) if output_final_state else None,
                                     _stream_ptr(q.device, stream)))
    return o, (fs if output_final_state else None)


def kda_chunk_fwd(q, k, v, g, beta, scale: Optional[float] = None, initial_state=None, cu_seqlens=None,
                  l2norm_qk: bool = False, beta_sigmoid: bool = False, output_final_state: bool = True,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """KDA forward: as :func:`gdn_chunk_fwd` with g fp32 [B,T,H,128] in log2 units."""
    return _chunk_fwd(True, q, k, v, g, beta, scale, initial_state, cu_seqlens, l2norm_qk, beta_sigmoid,
                      output_final_state, workspace, stream)


def gdn_chunk_fwd_gated(q, k, v, g_raw, A_log, dt_bias, beta, scale: Optional[float] = None, initial_state=None,
                        cu_seqlens=None, l2norm_qk: bool = False, beta_sigmoid: bool = False,
                        output_final_state: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """GDN forward with the gate formed in the kernel:
    g = -exp(A_log[h]) * softplus(g_raw + dt_bias[h]). g_raw fp32 [B,T,H],
    A_log, dt_bias fp32 [H]. Otherwise as :func:`gdn_chunk_fwd`."""
    return _chunk_fwd(False, q, k, v, g_raw, beta, scale, initial_state, cu_seqlens, l2norm_qk, beta_sigmoid,
                      output_final_state, workspace, stream, A_log, dt_bias)


def kda_chunk_fwd_gated(q, k, v, g_raw, A_log, dt_bias, beta, scale: Optional[float] = None, initial_state=None,
                        cu_seqlens=None, l2norm_qk: bool = False, beta_sigmoid: bool = False,
                        output_final_state: bool = True, workspace: Optional[torch.Tensor] = None, stream=None):
    """KDA forward with the gate formed in the kernel, in log2 units:
    g = -exp(A_log[h]) * softplus(g_raw + dt_bias[h, :]) / ln 2. g_raw fp32
    [B,T,H,128], A_log fp32 [H], dt_bias fp32 [H,128]. Otherwise as
    :func:`kda_chunk_fwd`."""
    return _chunk_fwd(True, q, k, v, g_raw, beta, scale, initial_state, cu_seqlens, l2norm_qk, beta_sigmoid,
                      output_final_state, workspace, stream, A_log, dt_bias)


def gdn_chunk_bwd(q, k, v, g, beta, do, scale: Optional[float] = None, initial_state=None, d_final_state=None,
                  cu_seqlens=None, l2norm_qk: bool = False, beta_sigmoid: bool = False,
                  workspace: Optional[torch.Tensor] = None, stream=None, A_log=None, dt_bias=None):
    """GDN backward: gradients of <do, o> + <d_final_state, final_state> for the
    forward of :func:`gdn_chunk_fwd` with the same arguments. do bf16
    [B,T,H,128]; d_final_state fp32 [N,H,128,128] or None (zero).
    Returns fp32 (dq, dk, dv [B,T,H,128], dg [B,T,H] w.r.t. the raw gate,
    dbeta [B,T,H] w.r.t. beta as passed, d_initial_state [N,H,128,128]).

    With A_log and dt_bias (fp32 [H]) this is the backward of
    :func:`gdn_chunk_fwd_gated`: g holds the raw gate values, dg is the
    gradient w.r.t. them, and (dA_log [H], ddt_bias [H]) are appended."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(q, k, v, g, beta, False, initial_state, cu)
    gated = A_log is not None or dt_bias is not None
    if gated:
        _check_gate_params(False, q, A_log, dt_bias, H, K)
    if (not isinstance(do, torch.Tensor) or do.dtype != torch.bfloat16 or not do.is_contiguous()
            or tuple(do.shape) != (B, T, H, V) or do.device != q.device):
        raise ValueError("do must be a contiguous bf16 [B,T,H,V] tensor on %s" % q.device)
    if d_final_state is not None and (d_final_state.dtype != torch.float32 or not d_final_state.is_contiguous()
                                      or tuple(d_final_state.shape) != (N, H, K, V)
                                      or d_final_state.device != q.device):
        raise ValueError("d_final_state must be a contiguous fp32 [N,H,K,V] tensor on %s" % q.device)
    scale = K ** -0.5 if scale is None else float(scale)
    flags = _flags(l2norm_qk, beta_sigmoid, False)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv = (torch.empty((B, T, H, K), **f32) for _ in range(3))
    dg, dbeta = torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32)
    ds0 = torch.empty((N, H, K, V), **f32)
    need = lib.gdn_chunk_bwd_workspace_bytes(B, T, H, K, V, N, _cu_ptr(cu), flags)
    if need == 0:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(), need))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gated:
        da, ddt = torch.empty((H,), **f32), torch.empty((H,), **f32)
        _check(lib.gdn_chunk_bwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
                                       _ptr(initial_state), _cu_ptr(cu), N, B, T, H, K, V, scale, flags, _ptr(do),
                                       _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(da),
                                       _ptr(ddt), _ptr(dbeta), _ptr(ds0), _ptr(workspace), ws_bytes,
                                       _stream_ptr(q.device, stream)))
        return dq, dk, dv, dg, dbeta, ds0, da, ddt
    _check(lib.gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _cu_ptr(cu), N,
                             B, T, H, K, V, scale, flags, _ptr(do), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0), _ptr(workspace), ws_bytes,
                             _stream_ptr(q.device, stream)))
    return dq, dk, dv, dg, dbeta, ds0


def kda_chunk_bwd(q, k, v, g, beta, do, scale: Optional[float] = None, initial_state=None, d_final_state=None,
                  cu_seqlens=None, l2norm_qk: bool = False, beta_sigmoid: bool = False,
                  workspace: Optional[torch.Tensor] = None, stream=None, A_log=None, dt_bias=None):
    """KDA backward: as :func:`gdn_chunk_bwd` for the forward of :func:`kda_chunk_fwd`;
    dg is fp32 [B,T,H,128] w.r.t. the raw log2 gate.

    With A_log (fp32 [H]) and dt_bias (fp32 [H,128]) this is the backward of
    :func:`kda_chunk_fwd_gated`: g holds the raw gate values, dg is the
    gradient w.r.t. them, and (dA_log [H], ddt_bias [H,128]) are appended."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(q, k, v, g, beta, True, initial_state, cu)
    gated = A_log is not None or dt_bias is not None
    if gated:
        _check_gate_params(True, q, A_log, dt_bias, H, K)
    if (not isinstance(do, torch.Tensor) or do.dtype != torch.bfloat16 or not do.is_contiguous()
            or tuple(do.shape) != (B, T, H, V) or do.device != q.device):
        raise ValueError("do must be a contiguous bf16 [B,T,H,V] tensor on %s" % q.device)
    if d_final_state is not None and (d_final_state.dtype != torch.float32 or not d_final_state.is_contiguous()
                                      or tuple(d_final_state.shape) != (N, H, K, V)
                                      or d_final_state.device != q.device):
        raise ValueError("d_final_state must be a contiguous fp32 [N,H,K,V] tensor on %s" % q.device)
    scale = K ** -0.5 if scale is None else float(scale)
    flags = _flags(l2norm_qk, beta_sigmoid, False)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq, dk, dv, dg = (torch.empty((B, T, H, K), **f32) for _ in range(4))
    dbeta = torch.empty((B, T, H), **f32)
    ds0 = torch.empty((N, H, K, V), **f32)
    need = lib.kda_chunk_bwd_workspace_bytes(B, T, H, K, V, N, _cu_ptr(cu), flags)
    if need == 0:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(), need))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gated:
        da, ddt = torch.empty((H,), **f32), torch.empty((H, K), **f32)
        _check(lib.kda_chunk_bwd_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
                                       _ptr(initial_state), _cu_ptr(cu), N, B, T, H, K, V, scale, flags, _ptr(do),
                                       _ptr(d_final_state), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(da),
                                       _ptr(ddt), _ptr(dbeta), _ptr(ds0), _ptr(workspace), ws_bytes,
                                       _stream_ptr(q.device, stream)))
        return dq, dk, dv, dg, dbeta, ds0, da, ddt
    _check(lib.kda_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state), _cu_ptr(cu), N,
                             B, T, H, K, V, scale, flags, _ptr(do), _ptr(d_final_state), _ptr(dq), _ptr(dk),
                             _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(ds0), _ptr(workspace), ws_bytes,
                             _stream_ptr(q.device, stream)))
    return dq, dk, dv, dg, dbeta, ds0


def kda_bwd_state_pass(q, k, g, beta, do, scale: Optional[float] = None, d_final_state=None, cu_seqlens=None,
                       l2norm_qk: bool = False, beta_sigmoid: bool = False, workspace: Optional[torch.Tensor] = None,
                       stream=None):
    """KDA backward, reverse state pass: for the forward of :func:`kda_chunk_fwd`
    with these q, k, g, beta and the loss <do, o> + <d_final_state, final_state>,
    returns fp32 (dh_next [H,NT,128,128]: the gradient w.r.t. the state leaving
    each chunk, dv_new [H,NT,64,128]: w.r.t. each chunk's v_new,
    d_initial_state [N,H,128,128])."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(q, k, k, g, beta, True, None, cu)
    if (not isinstance(do, torch.Tensor) or do.dtype != torch.bfloat16 or not do.is_contiguous()
            or tuple(do.shape) != (B, T, H, V) or do.device != q.device):
        raise ValueError("do must be a contiguous bf16 [B,T,H,V] tensor on %s" % q.device)
    if d_final_state is not None and (d_final_state.dtype != torch.float32 or not d_final_state.is_contiguous()
                                      or tuple(d_final_state.shape) != (N, H, K, V)
                                      or d_final_state.device != q.device):
        raise ValueError("d_final_state must be a contiguous fp32 [N,H,K,V] tensor on %s" % q.device)
    scale = K ** -0.5 if scale is None else float(scale)
    flags = _flags(l2norm_qk, beta_sigmoid, False)
    NT = num_chunks(B, T, cu_seqlens)
    f32 = dict(dtype=torch.float32, device=q.device)
    dh = torch.empty((H, NT, K, V), **f32)
    dvn = torch.empty((H, NT, CHUNK, V), **f32)
    ds0 = torch.empty((N, H, K, V), **f32)
    need = lib.kda_bwd_state_pass_workspace_bytes(B, T, H, K, V, N, _cu_ptr(cu), flags)
    if need == 0:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(), need))
    _check(lib.kda_bwd_state_pass(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _cu_ptr(cu), N, B, T, H, K, V, scale, flags,
                                  _ptr(do), _ptr(d_final_state), _ptr(dh), _ptr(dvn), _ptr(ds0), _ptr(workspace),
                                  0 if workspace is None else workspace.numel() * workspace.element_size(),
                                  _stream_ptr(q.device, stream)))
    return dh, dvn, ds0


def state_summary(k, v, g, beta, q=None, cu_seqlens=None, kda: bool = False, l2norm_qk: bool = False,
                  beta_sigmoid: bool = False, workspace: Optional[torch.Tensor] = None,
                  stream=None, A_log=None, dt_bias=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Affine state summary of every (sequence, head): final = M @ initial + S.
    Inputs as :func:`gdn_chunk_fwd` / :func:`kda_chunk_fwd` (q optional, unused);
    with A_log and dt_bias, g holds the raw gate values as for
    :func:`gdn_chunk_fwd_gated` / :func:`kda_chunk_fwd_gated`.
    Returns (M fp32 [N,H,128,128], S fp32 [N,H,128,128])."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(k if q is None else q, k, v, g, beta, kda, None, cu)
    gated = A_log is not None or dt_bias is not None
    if gated:
        _check_gate_params(kda, k, A_log, dt_bias, H, K)
    flags = _flags(l2norm_qk, beta_sigmoid, False)
    M = torch.empty((N, H, K, K), dtype=torch.float32, device=k.device)
    S = torch.empty((N, H, K, V), dtype=torch.float32, device=k.device)
    need = lib.gdn_state_summary_workspace_bytes(int(kda), B, T, H, K, V, N, _cu_ptr(cu))
    if need == 0:
        workspace = None
    elif workspace is None:
        workspace = torch.empty(int(need), dtype=torch.uint8, device=k.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small: %d < %d bytes" % (workspace.numel() * workspace.element_size(), need))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gated:
        _check(lib.gdn_state_summary_gated(int(kda), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(A_log), _ptr(dt_bias),
                                           _ptr(beta), _cu_ptr(cu), N, B, T, H, K, V, flags, _ptr(M), _ptr(S),
                                           _ptr(workspace), ws_bytes, _stream_ptr(k.device, stream)))
        return M, S
    fn = lib.kda_state_summary if kda else lib.gdn_state_summary
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _cu_ptr(cu), N, B, T, H, K, V, flags,
              _ptr(M), _ptr(S), _ptr(workspace), ws_bytes, _stream_ptr(k.device, stream)))
    return M, S


def state_summary_apply(M: torch.Tensor, S: torch.Tensor, state_in: Optional[torch.Tensor] = None,
                        out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """state_out = M @ state_in + S per (sequence, head); fp32 [N,H,128,128] device tensors."""
    for name, t in (("M", M), ("S", S), ("state_in", state_in), ("out", out)):
        if t is None:
            continue
        if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 4 or t.device.type != "cuda":
            raise ValueError("%s must be a contiguous fp32 [N,H,128,128] tensor on the GPU" % name)
        if tuple(t.shape) != tuple(S.shape) or t.device != S.device:
            raise ValueError("%s has shape %s on %s; S has %s on %s" % (name, tuple(t.shape), t.device,
                                                                        tuple(S.shape), S.device))
    N, H, K, V = S.shape
    if out is None:
        out = torch.empty_like(S)
    _check(lib.gdn_state_summary_apply(_ptr(M), _ptr(S), _ptr(state_in), _ptr(out), N, H, K, V,
                                       _stream_ptr(S.device, stream)))
    return out


def short_conv(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
               halo: Optional[torch.Tensor] = None, cu_seqlens=None, dilation: int = 1, silu: bool = True,
               out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Causal depthwise Conv1d (+ SiLU): x bf16 [B,T,D], weight fp32 [D,W] or
    [D,1,W], bias fp32 [D], halo bf16 [B or 1,(W-1)*dilation,D]. Returns y bf16 [B,T,D]."""
    cu = _cu_array(cu_seqlens)
    if x.dtype != torch.bfloat16 or x.dim() != 3 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous bf16 [B,T,D] tensor on the GPU")
    B, T, D = x.shape
    w = weight.reshape(weight.shape[0], -1)
    if w.dtype != torch.float32 or not w.is_contiguous() or w.shape[0] != D or w.device != x.device:
        raise ValueError("weight must be a contiguous fp32 [D,W] (or [D,1,W]) tensor on %s" % x.device)
    W = w.shape[1]
    if bias is not None and (bias.dtype != torch.float32 or tuple(bias.shape) != (D,) or bias.device != x.device):
        raise ValueError("bias must be fp32 [D] on %s" % x.device)
    if halo is not None:
        rows = 1 if cu is not None else B
        if (halo.dtype != torch.bfloat16 or not halo.is_contiguous() or halo.device != x.device
                or tuple(halo.shape) != (rows, (W - 1) * dilation, D)):
            raise ValueError("halo must be a contiguous bf16 %s tensor on %s" % ((rows, (W - 1) * dilation, D),
                                                                                    x.device))
    if out is None:
        out = torch.empty_like(x)
    N = B if cu is None else len(cu) - 1
    need = lib.gdn_short_conv_workspace_bytes(N, _cu_ptr(cu))
    ws = torch.empty(int(need), dtype=torch.uint8, device=x.device) if need else None
    _check(lib.gdn_short_conv(_ptr(x), _ptr(w), _ptr(bias), _ptr(halo), _cu_ptr(cu), N, B, T, D, W, dilation,
                              int(silu), _ptr(out), _ptr(ws), 0 if ws is None else int(need),
                              _stream_ptr(x.device, stream)))
    return out


def workspace_bytes(B, T, H, cu_seqlens=None, kda: bool = False, flags: int = 0) -> int:
    cu = _cu_array(cu_seqlens)
    N = B if cu is None else len(cu) - 1
    fn = lib.kda_chunk_fwd_workspace_bytes if kda else lib.gdn_chunk_fwd_workspace_bytes
    n = fn(B, T, H, HEAD_DIM, HEAD_DIM, N, _cu_ptr(cu), flags)
    if n == 0:
        raise GdnError(GDN_ERR_INVALID_ARGUMENT, last_error())
    return int(n)


# ---- stage entries -------------------------------------------------------------

def gdn_stage_prepare(q, k, g, beta, scale=None, cu_seqlens=None, kda: bool = False, l2norm_qk: bool = False,
                      beta_sigmoid: bool = False, stream=None):
    """Returns (tmat bf16 [H,NT,64,128], aqk bf16 [H,NT,64,64], vec fp32 [H,NT,8,64], gk fp32 [H,NT,64,128] or None).

    tmat rows hold T as bf16 hi (64) then lo (64); tmat and aqk store their
    columns permuted (column 32s+16h+4g+e at position 32s+8g+4h+e)."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K, V, N = _check_inputs(q, k, q, g, beta, kda, None, cu)
    NT = num_chunks(B, T, cu)
    dev = q.device
    tmat = torch.empty((H, NT, CHUNK, 2 * CHUNK), dtype=torch.bfloat16, device=dev)
    aqk = torch.empty((H, NT, CHUNK, CHUNK), dtype=torch.bfloat16, device=dev)
    vec = torch.empty((H, NT, VEC_ROWS, CHUNK), dtype=torch.float32, device=dev)
    gk = torch.empty((H, NT, CHUNK, K), dtype=torch.float32, device=dev) if kda else None
    scale = K ** -0.5 if scale is None else float(scale)
    _check(lib.gdn_stage_prepare(int(kda), _ptr(q), _ptr(k), _ptr(g), _ptr(beta), _cu_ptr(cu), N, B, T, H, K, K,
                                 scale, _flags(l2norm_qk, beta_sigmoid, False), _ptr(tmat), _ptr(aqk), _ptr(vec),
                                 _ptr(gk), _stream_ptr(dev, stream)))
    return tmat, aqk, vec, gk


def gdn_stage_fwd_h(k, v, tmat, vec, gk=None, initial_state=None, cu_seqlens=None, kda: bool = False,
                    output_final_state: bool = True, stream=None):
    """Returns (h fp32 [H,NT,128,128], v_new fp32 [H,NT,64,128], final_state fp32 [N,H,128,128] or None)."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K = k.shape
    V = v.shape[-1]
    N = B if cu is None else len(cu) - 1
    NT = num_chunks(B, T, cu)
    dev = k.device
    for name, t, shape, dt in (("tmat", tmat, (H, NT, CHUNK, 2 * CHUNK), torch.bfloat16),
                               ("vec", vec, (H, NT, VEC_ROWS, CHUNK), torch.float32)):
        if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError("%s must be contiguous %s %s" % (name, dt, shape))
    if tuple(v.shape) != (B, T, H, V) or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("k, v must be bf16 [B,T,H,128]")
    if initial_state is not None and tuple(initial_state.shape) != (N, H, K, V):
        raise ValueError("initial_state must be [N,H,K,V]")
    h = torch.empty((H, NT, K, V), dtype=torch.float32, device=dev)
    v_new = torch.empty((H, NT, CHUNK, V), dtype=torch.float32, device=dev)
    fs = torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if output_final_state else None
    _check(lib.gdn_stage_fwd_h(int(kda), _ptr(k), _ptr(v), _ptr(tmat), _ptr(vec), _ptr(gk), _ptr(initial_state),
                               _cu_ptr(cu), N, B, T, H, K, V, _flags(False, False, output_final_state), _ptr(h),
                               _ptr(v_new), _ptr(fs), _stream_ptr(dev, stream)))
    return h, v_new, fs


def gdn_stage_finalize(q, aqk, vec, h, v_new, gk=None, cu_seqlens=None, kda: bool = False, stream=None):
    """Returns o bf16 [B,T,H,128]."""
    cu = _cu_array(cu_seqlens)
    B, T, H, K = q.shape
    N = B if cu is None else len(cu) - 1
    NT = num_chunks(B, T, cu)
    for name, t, shape in (("h", h, (H, NT, K, K)), ("v_new", v_new, (H, NT, CHUNK, K)),
                           ("vec", vec, (H, NT, VEC_ROWS, CHUNK)), ("aqk", aqk, (H, NT, CHUNK, CHUNK))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("%s must be contiguous %s" % (name, shape))
    o = torch.empty((B, T, H, K), dtype=torch.bfloat16, device=q.device)
    _check(lib.gdn_stage_finalize(int(kda), _ptr(q), _ptr(aqk), _ptr(vec), _ptr(gk), _ptr(h), _ptr(v_new),
                                  _cu_ptr(cu), N, B, T, H, K, K, _ptr(o), _stream_ptr(q.device, stream)))
    return o


def timing_enable(enable: bool = True) -> None:
    """Record per-kernel HIP events in every whole-pass call of this thread."""
    _check(lib.gdn_timing_enable(1 if enable else 0))


def bwd_timing_read() -> Tuple[Tuple[float, ...], int]:
    """Summed ms of the backward's five kernels (prepare, forward state pass,
    reverse state pass, state products, per-chunk gradients) over the calls
    made while timing was enabled, and the number of calls."""
    ms = (ctypes.c_double * 5)()
    n = ctypes.c_int64(0)
    _check(lib.gdn_bwd_timing_read(ms, ctypes.byref(n)))
    return tuple(float(x) for x in ms), int(n.value)


def timing_read() -> Tuple[float, float, int]:
    """(prepare ms summed, state/output ms summed, calls) since the last read."""
    a, b, n = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_int64(0)
    _check(lib.gdn_timing_read(ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)))
    return a.value, b.value, int(n.value)
