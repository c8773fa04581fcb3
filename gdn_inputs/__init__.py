"""Seeded synthetic inputs for the chunked gated-delta-rule forward pass.

This module is the only code shared by the oracle side and the HIP side. It
draws random numbers and packs them into the storage formats of the kernel
contract (bf16 bit patterns, fp32, int32 offsets). It holds none of the
method's arithmetic: no normalisation, cumulative sums, decays or products of
the recurrence. The one transform applied to q/k for the tiny workload --
scaling each row to unit length before rounding to bf16 -- is part of that
workload's input distribution, not of the method (the method's own
normalisation, with its epsilon, lives in the oracle and in the kernels).

Workloads (natural-log gate for GDN, log2 gate for KDA):

* ``tiny``    B=1 T=256 H=2, unit-length q/k, beta=sigmoid(N(0,1)) stored as
  bf16, g=-softplus(N(0,1))*0.1, flags: final state only.
* ``gdn``     B=4 T=4096 H=16, q/k/v/beta-logits ~ N(0,1) bf16,
  g[b,t,h] = -exp(A_log[h]) * softplus(a[b,t,h] + dt_bias[h]),
  A_log ~ U(0, ln 16), a ~ N(0,1), dt_bias ~ N(0, 0.1^2);
  flags: in-kernel L2-norm, in-kernel sigmoid(beta), final state.
* ``varlen``  B=1 T=32768 H=16 packed by cu_seqlens, document lengths
  ~ U{17..8192} drawn until they cover T (the last one trimmed), per-document
  initial state ~ N(0, 0.02^2); other inputs as ``gdn``.
* ``long``    B=1 T=131072 H=32, as ``gdn``.
* ``kda``     B=2 T=8192 H=32 with a per-channel log2 gate
  g[b,t,h,d] = -softplus(x + dt_bias[h,d]) * exp(A_log[h]) / ln 2,
  x ~ N(0,1), A_log ~ U(0, ln 16), dt_bias ~ N(0, 0.1^2) of shape [H,128].

Every workload can be drawn at reduced B/T/H with the same recipe, which is
how the parity tests obtain sizes the oracle finishes in seconds.

``make_conv_inputs`` draws the input of the causal depthwise Conv1d + SiLU
that forms q, k, v: projections x ~ N(0,1) in bf16 of D = 3 * H * 128
channels for the GDN layer shape (q, k, v of H heads), weights and bias with
a depthwise Conv1d's default initialisation U(-1/sqrt(W), 1/sqrt(W)), W = 4.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

FLAG_L2NORM_QK = 1
FLAG_BETA_SIGMOID = 2
FLAG_OUTPUT_FINAL_STATE = 4

WORKLOADS = {
    # name: (B, T, H, kda, flags, seed)
    "tiny": (1, 256, 2, False, FLAG_OUTPUT_FINAL_STATE, 1001),
    "gdn": (4, 4096, 16, False, FLAG_L2NORM_QK | FLAG_BETA_SIGMOID | FLAG_OUTPUT_FINAL_STATE, 1002),
    "varlen": (1, 32768, 16, False, FLAG_L2NORM_QK | FLAG_BETA_SIGMOID | FLAG_OUTPUT_FINAL_STATE, 1003),
    "long": (1, 131072, 32, False, FLAG_L2NORM_QK | FLAG_BETA_SIGMOID | FLAG_OUTPUT_FINAL_STATE, 1004),
    "kda": (2, 8192, 32, True, FLAG_L2NORM_QK | FLAG_BETA_SIGMOID | FLAG_OUTPUT_FINAL_STATE, 1005),
}

HEAD_DIM = 128


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + rounding) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


@dataclasses.dataclass
class GdnInputs:
    """One synthetic problem in the kernel contract's storage formats.

    q, k, v: uint16 bf16 bits, [B,T,H,K] / [B,T,H,V], token-major.
    g: fp32, [B,T,H] (GDN, natural log) or [B,T,H,K] (KDA, log2).
    beta: uint16 bf16 bits, [B,T,H] (logits when the sigmoid flag is set).
    initial_state: fp32 [N,H,K,V] or None.
    cu_seqlens: int32 [N+1] or None (dense).
    """

    name: str
    B: int
    T: int
    H: int
    K: int
    V: int
    kda: bool
    flags: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    initial_state: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    # the draws g was made from (gdn, varlen, long, kda recipes): the raw gate
    # (a [B,T,H] or x [B,T,H,K]), A_log [H] and dt_bias [H] or [H,K], fp32
    gate_raw: Optional[np.ndarray] = None
    A_log: Optional[np.ndarray] = None
    dt_bias: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return self.B if self.cu_seqlens is None else int(len(self.cu_seqlens) - 1)

    @property
    def tokens(self) -> int:
        return self.B * self.T


def draw_doc_lengths(rng: np.random.Generator, total: int, lo: int = 17, hi: int = 8192) -> np.ndarray:
    """Document lengths ~ U{lo..hi} drawn until they cover ``total``; the last is trimmed."""
    lengths = []
    covered = 0
    while covered < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - covered)
        if n > 0:
            lengths.append(n)
        covered += n
    return np.asarray(lengths, dtype=np.int64)


def make_inputs(
    name: str,
    B: Optional[int] = None,
    T: Optional[int] = None,
    H: Optional[int] = None,
    seed: Optional[int] = None,
    doc_lengths: Optional[list] = None,
    doc_hi: int = 8192,
    K: int = HEAD_DIM,
    V: int = HEAD_DIM,
) -> GdnInputs:
    """Draw the named workload, optionally at reduced size.

    For ``varlen`` the documents are drawn from U{17..doc_hi} unless
    ``doc_lengths`` is given (then T is their sum).
    """
    B0, T0, H0, kda, flags, seed0 = WORKLOADS[name]
    B = B0 if B is None else B
    T = T0 if T is None else T
    H = H0 if H is None else H
    seed = seed0 if seed is None else seed
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(K)

    cu = None
    if name == "varlen":
        if doc_lengths is None:
            lengths = draw_doc_lengths(rng, T, 17, doc_hi)
        else:
            lengths = np.asarray(doc_lengths, dtype=np.int64)
            T = int(lengths.sum())
        B = 1
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)

    shape_tok = (B, T, H)
    q = rng.standard_normal((*shape_tok, K), dtype=np.float32)
    k = rng.standard_normal((*shape_tok, K), dtype=np.float32)
    v = rng.standard_normal((*shape_tok, V), dtype=np.float32)
    beta_logit = rng.standard_normal(shape_tok, dtype=np.float32)

    gate_raw = A_log = dt_bias = None
    if name == "tiny":
        q /= np.sqrt((q.astype(np.float64) ** 2).sum(-1, keepdims=True)).astype(np.float32)
        k /= np.sqrt((k.astype(np.float64) ** 2).sum(-1, keepdims=True)).astype(np.float32)
        beta = (1.0 / (1.0 + np.exp(-beta_logit.astype(np.float64)))).astype(np.float32)
        g = (-_softplus(rng.standard_normal(shape_tok, dtype=np.float32)) * np.float32(0.1)).astype(np.float32)
    elif kda:
        beta = beta_logit
        A_log = rng.uniform(0.0, math.log(16.0), size=(H,)).astype(np.float32)
        dt_bias = (rng.standard_normal((H, K), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
        x = rng.standard_normal((*shape_tok, K), dtype=np.float32)
        g = (-_softplus(x + dt_bias[None, None]) * np.exp(A_log)[None, None, :, None] / np.float32(math.log(2.0))).astype(np.float32)
        gate_raw = x
    else:
        beta = beta_logit
        A_log = rng.uniform(0.0, math.log(16.0), size=(H,)).astype(np.float32)
        dt_bias = (rng.standard_normal((H,), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
        a = rng.standard_normal(shape_tok, dtype=np.float32)
        g = (-np.exp(A_log)[None, None, :] * _softplus(a + dt_bias[None, None, :])).astype(np.float32)
        gate_raw = a

    s0 = None
    if name == "varlen":
        s0 = (rng.standard_normal((len(cu) - 1, H, K, V), dtype=np.float32) * np.float32(0.02)).astype(np.float32)

    return GdnInputs(
        name=name, B=B, T=T, H=H, K=K, V=V, kda=kda, flags=flags, scale=scale,
        q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
        g=np.ascontiguousarray(g, dtype=np.float32), beta=f32_to_bf16_bits(beta),
        initial_state=s0, cu_seqlens=cu, gate_raw=gate_raw, A_log=A_log, dt_bias=dt_bias,
    )


def random_problem(
    rng: np.random.Generator,
    B: int,
    T: int,
    H: int,
    K: int,
    V: int,
    kda: bool = False,
    gate_scale: float = 1.0,
    with_initial_state: bool = False,
    cu_seqlens: Optional[np.ndarray] = None,
    flags: int = FLAG_L2NORM_QK | FLAG_BETA_SIGMOID | FLAG_OUTPUT_FINAL_STATE,
    scale: Optional[float] = None,
) -> GdnInputs:
    """A generic small problem for unit tests (any K, V; gate ~ -gate_scale*softplus(N(0,1)))."""
    shape_tok = (B, T, H)
    q = rng.standard_normal((*shape_tok, K), dtype=np.float32)
    k = rng.standard_normal((*shape_tok, K), dtype=np.float32)
    v = rng.standard_normal((*shape_tok, V), dtype=np.float32)
    beta = rng.standard_normal(shape_tok, dtype=np.float32)
    gshape = (*shape_tok, K) if kda else shape_tok
    g = (-_softplus(rng.standard_normal(gshape, dtype=np.float32)) * np.float32(gate_scale)).astype(np.float32)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    s0 = None
    if with_initial_state:
        s0 = (rng.standard_normal((N, H, K, V), dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    return GdnInputs(
        name="random", B=B, T=T, H=H, K=K, V=V, kda=kda, flags=flags,
        scale=(1.0 / math.sqrt(K)) if scale is None else scale,
        q=f32_to_bf16_bits(q), k=f32_to_bf16_bits(k), v=f32_to_bf16_bits(v),
        g=g, beta=f32_to_bf16_bits(beta), initial_state=s0,
        cu_seqlens=None if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int32),
    )


# ---------------------------------------------------------------------------
# Causal depthwise Conv1d (+ SiLU) that forms q, k, v from the projections
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class ConvInputs:
    """x bf16 bits [B,T,D] (token-major), weight fp32 [D,W] (a depthwise
    Conv1d's [D,1,W] weight), bias fp32 [D] or None, halo bf16 bits
    [B,(W-1)*dilation,D] or None (rows preceding each sequence; packed input:
    preceding the first document), cu_seqlens int32 or None (then B = 1)."""
    B: int
    T: int
    D: int
    W: int
    dilation: int
    silu: bool
    x: np.ndarray
    weight: np.ndarray
    bias: Optional[np.ndarray]
    halo: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]


def make_conv_inputs(B: int, T: int, D: int, W: int = 4, dilation: int = 1, seed: int = 2001, silu: bool = True,
                     bias: bool = False, halo: bool = False, doc_lengths: Optional[list] = None) -> ConvInputs:
    """x ~ N(0,1) in bf16; weight and bias ~ U(-1/sqrt(W), 1/sqrt(W)) (the
    default initialisation of a depthwise Conv1d, fan-in W); halo ~ N(0,1).
    With doc_lengths, B must be 1 and T is their sum."""
    rng = np.random.default_rng(seed)
    cu = None
    if doc_lengths is not None:
        assert B == 1
        cu = np.concatenate([[0], np.cumsum(np.asarray(doc_lengths, dtype=np.int64))]).astype(np.int32)
        T = int(cu[-1])
    bound = np.float32(1.0 / math.sqrt(W))
    x = f32_to_bf16_bits(rng.standard_normal((B, T, D), dtype=np.float32))
    w = rng.uniform(-bound, bound, size=(D, W)).astype(np.float32)
    b = rng.uniform(-bound, bound, size=(D,)).astype(np.float32) if bias else None
    hw = (W - 1) * dilation
    h = f32_to_bf16_bits(rng.standard_normal((B, hw, D), dtype=np.float32)) if (halo and hw > 0) else None
    return ConvInputs(B=B, T=T, D=D, W=W, dilation=dilation, silu=silu, x=x, weight=w, bias=b, halo=h, cu_seqlens=cu)
