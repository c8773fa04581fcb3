"""Chunk form of the gated delta rule, derived from the token recurrence, in
fp64 numpy (TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and
the CPU baseline of bench.py; the library never uses it).

The recurrence, per sequence and head, with the state S a K x V matrix
(hyper-parallel "Diff Coverage" page, gate build 2026-09-10:
torch_chunk_gated_delta_rule and _l2norm; the per-channel gate: the coverage
page of kimi_delta_attention_ascendc.py, the gk slot of the KDA prepare
stage):

    S_t = D_t(S_{t-1}) + k_t w_t^T,   w_t = beta_t (v_t - D_t(S_{t-1})^T k_t),
    o_t = scale S_t^T q_t,

with D_t(S) = e^{g_t} S for GDN (one natural-log gate per token) and
D_t(S) = diag(2^{g_t}) S for KDA (one log2 gate per token and key channel);
q and k optionally L2-normalised first (x / sqrt(sum x^2 + 1e-6)) and beta
optionally given as a logit (sigmoid applied).

Derivation of the chunk form computed here. Take a chunk of C tokens entered
with state S and let G_i be the gate summed over its tokens 0..i (per channel
for KDA). Write E_i for the decay from the chunk start to token i (e^{G_i}, or
diag 2^{G_i}) and F_ij for the decay from token j to token i (e^{G_i - G_j},
or diag 2^{G_i - G_j}), j <= i. Unrolling the recurrence,

    S_i = E_i S + sum_{j <= i} F_ij k_j w_j^T,

so the decayed state that token i sees is E_i S + sum_{j < i} F_ij k_j w_j^T,
and the rows w_i satisfy a unit-lower-triangular system

    w_i + beta_i sum_{j < i} <k_i, F_ij k_j> w_j = beta_i v_i - beta_i (E_i k_i)^T S,

i.e. (I + L) w = diag(beta) V - diag(beta) (K E) S with L strictly lower,
L_ij = beta_i <k_i, F_ij k_j>. With T = (I + L)^-1 (LAPACK's triangular
solve here):

    w = U - W S,   U = T diag(beta) V,   W = T diag(beta) (K E),
    o_i = scale <E_i q_i, S> + scale sum_{j <= i} <q_i, F_ij k_j> w_j,
    S_out = E_last S + sum_j (F_last,j k_j) w_j^T.

In the pages' names: A = -L (the strictly lower beta K K^T * Gamma), T the
inverse of I - A, U and W the WY terms, w the chunk's v_new, and
Aqk_ij = scale <q_i, F_ij k_j> (j <= i) the intra-chunk output matrix. Padding
a sequence with tokens of beta = 0, k = q = v = 0 and g = 0 changes nothing,
so sequences are zero-padded to whole chunks. Documents of packed input are
separate sequences with their own states, and chunking restarts at each
(the chunk table of the KDA coverage page).

Pinned by tests/test_oracle_pins.py: equality with the C token recurrence
(oracle.recur) over shapes, chunk sizes and both gate kinds; the affine
state summary against the recurrence; closed forms (beta = 0, retrieval) and
the hand-derived fixtures.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
from scipy.linalg import solve_triangular


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp64 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def l2norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """``x / sqrt(sum(x*x, -1) + eps)`` in fp64 (the pages' ``_l2norm``)."""
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def _decayed_products(x, y, G, kda):
    """P_ij = <x_i, F_ij y_j> for j <= i and 0 above the diagonal, over the
    last two axes of one chunk (x, y: [..., C, K]; G: [..., C] or [..., C, K]).
    The exponent is masked to 0 above the diagonal before exponentiating, so
    no growing factor is ever formed."""
    C = x.shape[-2]
    lower = np.tril(np.ones((C, C), dtype=bool))
    if not kda:
        diff = np.where(lower, G[..., :, None] - G[..., None, :], 0.0)
        F = np.where(lower, np.exp(diff), 0.0)
        return (x @ np.swapaxes(y, -1, -2)) * F
    m = lower[:, :, None]
    diff = np.where(m, G[..., :, None, :] - G[..., None, :, :], 0.0)
    F = np.where(m, np.exp2(diff), 0.0)
    return np.einsum("...id,...jd,...ijd->...ij", x, y, F)


def _unit_lower_inverse(L):
    """(I + L)^-1 for strictly lower L [..., C, C]: LAPACK's triangular solve
    of (I + L) X = I (unit diagonal) for every matrix of the batch."""
    C = L.shape[-1]
    flat = L.reshape(-1, C, C)
    eye = np.eye(C)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        out[i] = solve_triangular(eye + flat[i], eye, lower=True, unit_diagonal=True)
    return out.reshape(L.shape)


def _chunked_pass(q, k, v, beta, g, scale, s0, C, kda, keep):
    """Sequences of one length. q, k: [B,H,T,K]; v: [B,H,T,V]; beta: [B,H,T];
    g: [B,H,T] (GDN) or [B,H,T,K] (KDA); s0: [B,H,K,V]. Returns o [B,H,T,V],
    the final state and (keep) the per-chunk intermediates [B,H,NC,...]."""
    B, H, T, K = q.shape
    V = v.shape[-1]
    pad = -T % C
    if pad:
        zpad = lambda x: np.concatenate([x, np.zeros(x.shape[:2] + (pad,) + x.shape[3:])], axis=2)
        q, k, v, beta, g = zpad(q), zpad(k), zpad(v), zpad(beta), zpad(g)
    NC = (T + pad) // C
    chunks = lambda x: x.reshape(B, H, NC, C, *x.shape[3:])
    q, k, v, beta, g = chunks(q), chunks(k), chunks(v), chunks(beta), chunks(g)
    G = np.cumsum(g, axis=3)
    strict = np.tril(np.ones((C, C), dtype=bool), -1)
    power = np.exp2 if kda else np.exp
    row = (lambda x: x) if kda else (lambda x: x[..., None])  # decay of a row: per channel or one factor

    S = np.array(s0, dtype=np.float64)
    o = np.zeros((B, H, NC, C, V))
    if keep:
        names = ("T", "W", "U", "Aqk", "h", "v_new")
        shapes = ((C, C), (C, K), (C, V), (C, C), (K, V), (C, V))
        inter = {n: np.zeros((B, H, NC) + s) for n, s in zip(names, shapes)}
    for c in range(NC):
        qc, kc, vc, bc, Gc = q[:, :, c], k[:, :, c], v[:, :, c], beta[:, :, c], G[:, :, c]
        L = np.where(strict, bc[..., :, None] * _decayed_products(kc, kc, Gc, kda), 0.0)
        Tm = _unit_lower_inverse(L)
        E = power(Gc)                                   # decay from the chunk start
        U = Tm @ (bc[..., None] * vc)
        W = Tm @ (bc[..., None] * kc * row(E))
        Aqk = scale * _decayed_products(qc, kc, Gc, kda)
        if keep:
            inter["h"][:, :, c] = S
        w = U - W @ S                                   # the chunk's new values
        o[:, :, c] = (scale * qc * row(E)) @ S + Aqk @ w
        Glast = Gc[:, :, -1:]
        k_out = kc * row(power(Glast - Gc))             # keys decayed to the chunk end
        if kda:
            S = power(Glast)[:, :, 0, :, None] * S + np.swapaxes(k_out, -1, -2) @ w
        else:
            S = power(Glast)[..., None] * S + np.swapaxes(k_out, -1, -2) @ w
        if keep:
            for n, x in zip(names, (Tm, W, U, Aqk, None, w)):
                if x is not None:
                    inter[n][:, :, c] = x
    o = o.reshape(B, H, NC * C, V)[:, :, :T]
    if not keep:
        return o, S, None
    inter.update(G=G, k=k, k_beta=beta[..., None] * k)
    return o, S, inter


def _row_vectors(beta, rq, rk, C):
    """Per-row beta (after the optional sigmoid) and the normalisation factors
    1/sqrt(sum x^2 + 1e-6) (1 without normalisation), chunked [B,H,NC,C] with
    zero padding."""
    B, H, T = beta.shape
    pad = -T % C
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
    (``[1,H,NC,...]``), in sequence order: G, T, W, U, Aqk, h (state entering
    each chunk), v_new, k (normalised), k_beta, beta, rq, rk.
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
        spans = [(slice(None), slice(None), slice(None))]
    else:
        cu = [int(x) for x in inp.cu_seqlens]
        spans = [(slice(None), slice(cu[n], cu[n + 1]), slice(n, n + 1)) for n in range(N)]
    for bsl, tsl, ssl in spans:
        sl = lambda x: hm(x[bsl, tsl])
        o, S, inter = _chunked_pass(sl(q), sl(k), sl(v), sl(beta), sl(g), inp.scale, s0[ssl], chunk_size,
                                    inp.kda, keep)
        o_all[bsl, tsl] = np.moveaxis(o, 1, 2)
        fs[ssl] = S
        if keep:
            inter.update(_row_vectors(sl(beta), sl(rq), sl(rk), chunk_size))
        inters.append(inter)
    return o_all, fs, (inters if keep else None)


def state_summary(inp, chunk_size: int = 64, flags: Optional[int] = None):
    """Affine state summary ``state_out = M state_in + S`` of every sequence
    (the summary of _compute_gdn_state_summary_from_prepared, 2026-09-10 page).

    By the chunk form above, a chunk maps its entering state affinely:
    S_out = (E_last - K_out^T W) S + K_out^T U, with K_out the keys decayed
    to the chunk end. Composing these maps over the chunks of a sequence,
    from the identity map, gives (M, S). The initial state of ``inp`` is
    ignored.

    Returns ``(M, S)``: fp64 [N,H,K,K] and [N,H,K,V].
    """
    zero = type(inp)(**{**inp.__dict__, "initial_state": None})
    _, _, inters = chunk(zero, chunk_size=chunk_size, flags=flags, keep=True)
    Ms, Ss = [], []
    for it in inters:
        G, W, U, kk = it["G"], it["W"], it["U"], it["k"]
        Bn, H, NC = G.shape[:3]
        K = kk.shape[-1]
        M = np.broadcast_to(np.eye(K), (Bn, H, K, K)).copy()
        S = np.zeros((Bn, H, K, U.shape[-1]))
        for c in range(NC):
            Gc = G[:, :, c]
            Glast = Gc[:, :, -1:]
            if inp.kda:
                k_out = kk[:, :, c] * np.exp2(Glast - Gc)
                e_last = np.eye(K) * np.exp2(Glast)             # diag(2^{G_last})
            else:
                k_out = kk[:, :, c] * np.exp(Glast - Gc)[..., None]
                e_last = np.exp(Glast)[..., None] * np.eye(K)
            kt = np.swapaxes(k_out, -1, -2)
            step = e_last - kt @ W[:, :, c]
            M = step @ M
            S = step @ S + kt @ U[:, :, c]
        Ms.append(M)
        Ss.append(S)
    return np.concatenate(Ms, axis=0), np.concatenate(Ss, axis=0)


def apply_state_summary(M: np.ndarray, S: np.ndarray, state_in: Optional[np.ndarray]) -> np.ndarray:
    """``state_out = M state_in + S`` (``_apply_gdn_state_summary``, 2026-09-10
    page); ``state_in`` None means zero."""
    if state_in is None:
        return np.asarray(S, dtype=np.float64).copy()
    return np.asarray(M, dtype=np.float64) @ np.asarray(state_in, dtype=np.float64) + S
