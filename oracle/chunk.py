"""Chunked form of the gated delta rule in fp64 numpy (TEST INFRASTRUCTURE ONLY).

Follows, step by step and in its order, the eager chunk algorithm that the
hyper-parallel "Diff Coverage" page of the 2026-09-10 gate build writes out
(functions ``torch_chunk_gated_delta_rule``, ``_prepare_gdn_chunks_for_summary``
and ``_run_prepared_gdn_chunks``):

1. optional L2 normalisation of q and k, ``x * rsqrt(sum(x*x) + 1e-6)``
   (``_l2norm``);
2. head-major layout, zero padding of T to a multiple of the chunk size;
3. q scaled by ``scale``; ``k_beta = k*beta``, ``v_beta = v*beta``;
4. per chunk: ``G = cumsum(g)``; decay mask ``Gamma[i,j] = exp(G_i - G_j)`` for
   i >= j, with the causal mask applied before the exponential so no positive
   exponent is ever evaluated;
5. ``A = -(k_beta k^T * Gamma)`` with the diagonal and upper triangle zeroed;
6. forward substitution row by row, ``A[i,:i] += sum_m A[i,m] A[m,:i]``, then
   ``T = A + I`` (this is ``(I + strictLower(diag(beta) K K^T * Gamma))^-1``);
7. ``U = T v_beta`` and ``W = T (k_beta * exp(G))``;
8. sequentially over chunks, with S the state entering the chunk:
   ``v_new = U - W S``;
   ``o = (q * exp(G)) S + (q k^T * Gamma) v_new`` (diagonal included);
   ``S <- exp(G_last) S + (k * exp(G_last - G))^T v_new``;
9. trim the padding.

The Kimi-Delta-Attention variant (``kda=True``) takes a per-key-channel gate
in log2 units (the ``gk`` slot of the KDA prepare stage on the
``kimi_delta_attention_ascendc.py`` coverage page is a chunk-local cumulative
log2 decay). Reading of the pages: every ``exp(x)`` above becomes ``2**x`` of
a per-channel difference, so ``Gamma`` gains a channel index d and the
products over d carry it inside the sum, and ``exp(G_last) S`` becomes
``diag(2**G_last) S``. Here too the mask comes before the power.

Chunks never span documents: for packed input (cu_seqlens) each document is
its own sequence with its own initial and final state, and chunk numbering
restarts at every document (the chunk table of the same KDA page).

Pinned by tests/test_oracle_pins.py: equality with the C token recurrence
(``oracle.recur``) on many shapes, chunk sizes and both gate kinds; the
state-summary identity of ``_compute_gdn_state_summary_from_prepared``
(2026-09-10 page), which re-derives the state from W and the decayed keys.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def l2norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """``x * rsqrt(sum(x*x, -1) + eps)`` in fp64 (the pages' ``_l2norm``)."""
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def _forward_substitution(A: np.ndarray) -> np.ndarray:
    """Row recursion of step 6 on a batch of strictly-lower C x C matrices; returns T = A' + I."""
    A = A.copy()
    C = A.shape[-1]
    for i in range(1, C):
        row = A[..., i, :i].copy()
        sub = A[..., :i, :i].copy()
        A[..., i, :i] = row + (row[..., :, None] * sub).sum(-2)
    return A + np.eye(C)


def _chunk_one(q, k, v, beta, g, scale, s0, C, kda, keep):
    """One batch of equal-length sequences. q,k: [B,H,T,K]; v: [B,H,T,V];
    beta: [B,H,T]; g: [B,H,T] (GDN, natural log) or [B,H,T,K] (KDA, log2);
    s0: [B,H,K,V] fp64."""
    B, H, T, K = q.shape
    V = v.shape[-1]
    pad = (C - T % C) % C
    if pad:
        zp = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (pad,) + x.shape[3:])], axis=2)
        q, k, v, beta, g = zp(q), zp(k), zp(v), zp(beta), zp(g)
    Tp = T + pad
    NC = Tp // C
    q = q * scale
    v_beta = v * beta[..., None]
    k_beta = k * beta[..., None]
    rs = lambda x: x.reshape(B, H, NC, C, *x.shape[3:])
    q, k, v_beta, k_beta, g = rs(q), rs(k), rs(v_beta), rs(k_beta), rs(g)

    G = np.cumsum(g, axis=3)
    lower = np.tril(np.ones((C, C), dtype=bool))
    strict = np.tril(np.ones((C, C), dtype=bool), -1)

    if not kda:
        diff = G[..., :, None] - G[..., None, :]
        Gamma = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
        A = -((k_beta @ np.swapaxes(k, -1, -2)) * Gamma)
        A = np.where(strict, A, 0.0)
        Aqk = (q @ np.swapaxes(k, -1, -2)) * Gamma
        eG = np.exp(G)[..., None]
        Tm = _forward_substitution(A)
        U = Tm @ v_beta
        W = Tm @ (k_beta * eG)
    else:
        A = np.zeros((B, H, NC, C, C))
        Aqk = np.zeros((B, H, NC, C, C))
        for c in range(NC):
            Gc = G[:, :, c]                                   # [B,H,C,K]
            diff = Gc[:, :, :, None, :] - Gc[:, :, None, :, :]  # [B,H,C,C,K]
            Gam = np.where(lower[..., None], np.exp2(np.where(lower[..., None], diff, 0.0)), 0.0)
            kk = np.einsum("bhid,bhjd,bhijd->bhij", k_beta[:, :, c], k[:, :, c], Gam)
            A[:, :, c] = -np.where(strict, kk, 0.0)
            Aqk[:, :, c] = np.einsum("bhid,bhjd,bhijd->bhij", q[:, :, c], k[:, :, c], Gam)
        Tm = _forward_substitution(A)
        U = Tm @ v_beta
        W = Tm @ (k_beta * np.exp2(G))

    S = s0.copy()
    o = np.zeros((B, H, NC, C, V))
    h = np.zeros((B, H, NC, K, V)) if keep else None
    v_new_all = np.zeros((B, H, NC, C, V)) if keep else None
    for c in range(NC):
        if keep:
            h[:, :, c] = S
        v_new = U[:, :, c] - W[:, :, c] @ S
        if not kda:
            Gc = G[:, :, c]
            qd = q[:, :, c] * np.exp(Gc)[..., None]
            kd = k[:, :, c] * np.exp(Gc[..., -1:] - Gc)[..., None]
            o[:, :, c] = qd @ S + Aqk[:, :, c] @ v_new
            S = S * np.exp(Gc[..., -1])[..., None, None] + np.swapaxes(kd, -1, -2) @ v_new
        else:
            Gc = G[:, :, c]                                   # [B,H,C,K]
            qd = q[:, :, c] * np.exp2(Gc)
            kd = k[:, :, c] * np.exp2(Gc[:, :, -1:, :] - Gc)
            o[:, :, c] = qd @ S + Aqk[:, :, c] @ v_new
            S = S * np.exp2(Gc[:, :, -1, :])[..., :, None] + np.swapaxes(kd, -1, -2) @ v_new
        if keep:
            v_new_all[:, :, c] = v_new
    o = o.reshape(B, H, Tp, V)[:, :, :T]
    inter = None
    if keep:
        inter = dict(G=G, T=Tm, W=W, U=U, Aqk=Aqk, h=h, v_new=v_new_all, k=k, k_beta=k_beta)
    return o, S, inter


def _row_vectors(beta, rq, rk, C):
    """Per-row beta (after the optional sigmoid) and the normalisation factors
    1/sqrt(sum x^2 + 1e-6) (1 without normalisation), chunked [B,H,NC,C] with
    zero padding."""
    B, H, T = beta.shape
    pad = (C - T % C) % C
    out = {}
    for name, x in (("beta", beta), ("rq", rq), ("rk", rk)):
        x = np.concatenate([x, np.zeros((B, H, pad))], axis=2) if pad else x
        out[name] = x.reshape(B, H, -1, C)
    return out


def chunk(inp, chunk_size: int = 64, flags: Optional[int] = None, keep: bool = False):
    """Chunked fp64 forward on a :class:`gdn_inputs.GdnInputs` problem.

    Returns ``(o, final_state, inter)``: o fp64 [B,T,H,V], final_state fp64
    [N,H,K,V]; ``inter`` (when ``keep``) is a list with one dict of chunk
    intermediates per dense batch (``[B,H,NC,...]``) or per document
    (``[1,H,NC,...]``), in sequence order.
    """
    flags = inp.flags if flags is None else flags
    q = decode_bf16(inp.q)
    k = decode_bf16(inp.k)
    v = decode_bf16(inp.v)
    beta = decode_bf16(inp.beta)
    g = np.asarray(inp.g, dtype=np.float64)
    rq = np.ones(q.shape[:3])
    rk = np.ones(k.shape[:3])
    if flags & 1:
        rq = 1.0 / np.sqrt((q * q).sum(-1) + 1e-6)
        rk = 1.0 / np.sqrt((k * k).sum(-1) + 1e-6)
        q = l2norm(q)
        k = l2norm(k)
    if flags & 2:
        beta = 1.0 / (1.0 + np.exp(-beta))
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = inp.num_seqs
    s0 = np.zeros((N, H, K, V)) if inp.initial_state is None else np.asarray(inp.initial_state, dtype=np.float64)

    hm = lambda x: np.ascontiguousarray(np.moveaxis(x, 2, 1))  # [B,T,H,...] -> [B,H,T,...]
    o_all = np.zeros((B, T, H, V))
    fs = np.zeros((N, H, K, V))
    inters = []
    if inp.cu_seqlens is None:
        o, S, inter = _chunk_one(hm(q), hm(k), hm(v), hm(beta), hm(g), inp.scale, s0, chunk_size, inp.kda, keep)
        o_all[:] = np.moveaxis(o, 1, 2)
        fs[:] = S
        if keep:
            inter.update(_row_vectors(hm(beta), hm(rq), hm(rk), chunk_size))
        inters.append(inter)
    else:
        cu = [int(x) for x in inp.cu_seqlens]
        for n in range(N):
            a, b = cu[n], cu[n + 1]
            sl = lambda x: hm(x[:, a:b])
            o, S, inter = _chunk_one(sl(q), sl(k), sl(v), sl(beta), sl(g), inp.scale, s0[n:n + 1],
                                     chunk_size, inp.kda, keep)
            o_all[:, a:b] = np.moveaxis(o, 1, 2)
            fs[n] = S[0]
            if keep:
                inter.update(_row_vectors(sl(beta), sl(rq), sl(rk), chunk_size))
            inters.append(inter)
    return o_all, fs, (inters if keep else None)


def state_summary(inp, chunk_size: int = 64, flags: Optional[int] = None):
    """Affine state summary ``state_out = M state_in + S`` of every sequence.

    Follows ``_compute_gdn_state_summary_from_prepared`` (2026-09-10 page):
    starting from ``S = 0`` and ``M = I``, for each chunk in order,
    ``transition = decay I - (k * e^{G_last - G})^T W`` and
    ``S <- transition S + (k * e^{G_last - G})^T U``, ``M <- transition M``,
    with W, U the chunk form's WY terms. For KDA the decay is
    ``diag(2^{G_last})`` and the key decay per channel (the reading of the
    chunk form above). The initial state of ``inp`` is ignored.

    Returns ``(M, S)``: fp64 [N,H,K,K] and [N,H,K,V].
    """
    zero = type(inp)(**{**inp.__dict__, "initial_state": None})
    _, _, inters = chunk(zero, chunk_size=chunk_size, flags=flags, keep=True)
    Ms, Ss = [], []
    for it in inters:
        G, W, U, kk = it["G"], it["W"], it["U"], it["k"]
        Bn, H, NC = G.shape[:3]
        K = kk.shape[-1]
        V = U.shape[-1]
        M = np.broadcast_to(np.eye(K), (Bn, H, K, K)).copy()
        S = np.zeros((Bn, H, K, V))
        for c in range(NC):
            Gc = G[:, :, c]
            if inp.kda:
                kd = kk[:, :, c] * np.exp2(Gc[:, :, -1:, :] - Gc)
                decay = np.eye(K) * np.exp2(Gc[:, :, -1, :])[..., None, :]
            else:
                kd = kk[:, :, c] * np.exp(Gc[..., -1:] - Gc)[..., None]
                decay = np.exp(Gc[..., -1])[..., None, None] * np.eye(K)
            kdt = np.swapaxes(kd, -1, -2)
            trans = decay - kdt @ W[:, :, c]
            S = trans @ S + kdt @ U[:, :, c]
            M = trans @ M
        Ms.append(M)
        Ss.append(S)
    return np.concatenate(Ms, axis=0), np.concatenate(Ss, axis=0)


def apply_state_summary(M: np.ndarray, S: np.ndarray, state_in: Optional[np.ndarray]) -> np.ndarray:
    """``state_out = M state_in + S`` (``_apply_gdn_state_summary``, 2026-09-10
    page); ``state_in`` None means zero."""
    if state_in is None:
        return np.asarray(S, dtype=np.float64).copy()
    return np.asarray(M, dtype=np.float64) @ np.asarray(state_in, dtype=np.float64) + S
