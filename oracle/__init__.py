"""Oracle for the chunked gated-delta-rule forward pass (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP path and
never imports it.

Two independent fp64 definitions of the same result:

* :func:`recur` -- the token-by-token recurrence, in plain C (``recur.c``),
  OpenMP over (sequence, head) units. This is the reference result.
* :func:`chunk` (module ``oracle.chunk``) -- the chunk form of the same
  recurrence in numpy fp64, derived in that module's header from the token
  recurrence (the method of the hyper-parallel "Diff Coverage" page of
  2026-09-10, ``torch_chunk_gated_delta_rule``), exporting its per-chunk
  intermediates (T, U, W, the output matrix, h, v_new) for stage parity.

Besides these, :func:`state_summary` / :func:`apply_state_summary` (the
affine summary of a sequence) and :func:`short_conv` (module ``oracle.conv``,
the causal depthwise Conv1d + SiLU that forms q, k, v) and module
``oracle.grad`` (gradients of the recurrence by fp64 reverse-mode
differentiation, pinned by ``tests/test_grad_pins.py``) and module
``oracle.gate`` (the in-kernel gate's formula, pinned by
``tests/test_gate_pins.py``).

Every function is pinned by ``tests/test_oracle_pins.py`` (and
``tests/test_conv_pins.py``) against facts fixed by the mathematics (closed forms, invariants, hand-derived fixtures); see the
header of each function for what pins it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

L2NORM = 1
BETA_SIGMOID = 2


def build(force: bool = True) -> str:
    """Compile ``recur.c`` with gcc (-O2, OpenMP) into ``liboracle.so``."""
    src = os.path.join(_HERE, "recur.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i = ctypes.c_int
        lib.oracle_recur.argtypes = [i, p, p, p, p, p, p, p, i, i, i, i, i, i,
                                     ctypes.c_double, ctypes.c_uint, p, i, p, p]
        lib.oracle_recur.restype = i
        lib.oracle_num_threads.restype = i
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recur(inp, units: Optional[Sequence[tuple]] = None, flags: Optional[int] = None):
    """fp64 token recurrence on a :class:`gdn_inputs.GdnInputs` problem.

    ``units`` restricts the work to a list of (sequence, head) pairs (the
    other rows of ``o`` stay zero). Returns ``(o, final_state)``: o fp64
    [B,T,H,V], final_state fp64 [N,H,K,V].
    """
    lib = _load()
    flags = inp.flags if flags is None else flags
    N = inp.num_seqs
    q = np.ascontiguousarray(inp.q, dtype=np.uint16)
    k = np.ascontiguousarray(inp.k, dtype=np.uint16)
    v = np.ascontiguousarray(inp.v, dtype=np.uint16)
    g = np.ascontiguousarray(inp.g, dtype=np.float32)
    beta = np.ascontiguousarray(inp.beta, dtype=np.uint16)
    s0 = None if inp.initial_state is None else np.ascontiguousarray(inp.initial_state, dtype=np.float32)
    cu = None if inp.cu_seqlens is None else np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
    o = np.zeros((inp.B, inp.T, inp.H, inp.V), dtype=np.float64)
    fs = np.zeros((N, inp.H, inp.K, inp.V), dtype=np.float64)
    u_arr = None
    n_units = 0
    if units is not None:
        u_arr = np.ascontiguousarray(np.asarray(units, dtype=np.int32).reshape(-1, 2))
        n_units = u_arr.shape[0]
    rc = lib.oracle_recur(int(inp.kda), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(cu),
                          N, inp.B, inp.T, inp.H, inp.K, inp.V, float(inp.scale), int(flags),
                          _ptr(u_arr), n_units, _ptr(o), _ptr(fs))
    if rc != 0:
        raise ValueError("oracle_recur rejected its arguments")
    return o, fs


from .chunk import apply_state_summary, chunk, decode_bf16, l2norm, state_summary  # noqa: E402  (pure numpy, no C)
from .conv import short_conv  # noqa: E402  (pure numpy, no C)

__all__ = ["build", "recur", "chunk", "decode_bf16", "l2norm", "num_threads", "L2NORM", "BETA_SIGMOID"]
