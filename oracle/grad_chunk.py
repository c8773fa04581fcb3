"""Chunk-form gradients of the gated delta rule, GDN and KDA, fp64 (TEST
INFRASTRUCTURE ONLY).

The reverse pass of the chunked forward (the prepared-chunk algorithm of
torch_chunk_gated_delta_rule on the hyper-parallel "Diff Coverage" page,
gate build 2026-09-10), written step by step so that a backward kernel can be
checked stage by stage: per chunk, from the last, the gradient of the state
entering it and of every intermediate (v_new, T, the intra-chunk matrices,
the cumulative gate). The pages print no backward formula; each step below is
the derivative of the forward step it follows, and the whole is pinned to
``oracle.grad`` (reverse-mode differentiation of the token recurrence, an
independent computation) by tests/test_grad_pins.py.

Both gate kinds run in one form: per-channel natural-log decays G (GDN: the
token's gate on every channel; KDA: the log2 gate times ln 2). Every decay
between two rows is formed as exp(G_i - G_j) with the causal mask applied
before the exponential, so no positive exponent is evaluated.

Forward of one chunk (rows i, state S entering, K x V):
  KD = k^ exp(G), QD = q^ exp(G), KG = k^ exp(G_last - G)
  A[i,j] = -b_i sum_d k^_id k^_jd exp(G_id - G_jd)   (i > j)
  T = (I - A)^-1,  W = T diag(b) KD,  U = T diag(b) V,  V' = U - W S
  P[i,j] = sum_d q^_id k^_jd exp(G_id - G_jd)        (i >= j)
  O = scale (QD S + P V'),  S_next = diag(exp(G_last)) S + KG^T V'
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .chunk import decode_bf16


def _chunk_fwd(qn, kn, v, b, G, S, scale):
    """Forward of one chunk, keeping what the reverse pass needs."""
    L = qn.shape[0]
    ii, jj = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    lower, incl = ii > jj, ii >= jj
    diff = G[:, None, :] - G[None, :, :]                       # [i, j, d]
    Ekk = np.exp(np.where(lower[..., None], diff, -np.inf))
    Eqk = np.exp(np.where(incl[..., None], diff, -np.inf))
    GL = G[-1]
    eG, eLG = np.exp(G), np.exp(GL - G)
    KD, QD, KG = kn * eG, qn * eG, kn * eLG
    A = -b[:, None] * np.einsum("id,jd,ijd->ij", kn, kn, Ekk)
    T = np.linalg.inv(np.eye(L) - A)
    W = T @ (b[:, None] * KD)
    U = T @ (b[:, None] * v)
    vn = U - W @ S
    P = np.einsum("id,jd,ijd->ij", qn, kn, Eqk)
    O = scale * (QD @ S + P @ vn)
    S_next = np.exp(GL)[:, None] * S + KG.T @ vn
    return dict(Ekk=Ekk, Eqk=Eqk, eG=eG, eLG=eLG, KD=KD, QD=QD, KG=KG, A=A, T=T, W=W, U=U, vn=vn, P=P, O=O,
                S=S, S_next=S_next, GL=GL, lower=lower, incl=incl)


def _chunk_bwd(f, qn, kn, v, b, dO, dS_next, scale):
    """Reverse of one chunk. Returns the gradients of the state entering it
    and of the chunk's q^, k^, v, b and cumulative gate G (natural log, per
    channel), and the intermediates dV', dA, dP."""
    S, T, W, vn, P = f["S"], f["T"], f["W"], f["vn"], f["P"]
    KD, QD, KG, GL = f["KD"], f["QD"], f["KG"], f["GL"]
    # O = scale (QD S + P V')
    dP = scale * (dO @ vn.T) * f["incl"]
    dvn = scale * P.T @ dO + KG @ dS_next
    dQD = scale * dO @ S.T
    dS = scale * QD.T @ dO + np.exp(GL)[:, None] * dS_next
    # S_next = diag(exp(G_last)) S + KG^T V'
    dKG = vn @ dS_next.T
    dGL = np.exp(GL) * (S * dS_next).sum(1)
    # V' = U - W S
    dU, dW = dvn, -dvn @ S.T
    dS = dS - W.T @ dvn
    # U = T diag(b) V, W = T diag(b) KD
    dT = dU @ (b[:, None] * v).T + dW @ (b[:, None] * KD).T
    tU, tW = T.T @ dU, T.T @ dW
    dv = b[:, None] * tU
    db = (tU * v).sum(1) + (tW * KD).sum(1)
    dKD = b[:, None] * tW
    # T = (I - A)^-1: dA = T^T dT T^T on the strictly lower part
    dA = (T.T @ dT @ T.T) * f["lower"]
    # A[i,j] = -b_i sum_d k^_id k^_jd exp(G_id - G_jd)
    Ckk = np.einsum("id,jd,ijd->ijd", kn, kn, f["Ekk"])
    db = db - np.einsum("ij,ijd->i", dA, Ckk)
    wA = -b[:, None] * dA
    dkn = np.einsum("ij,jd,ijd->id", wA, kn, f["Ekk"]) + np.einsum("ij,id,ijd->jd", wA, kn, f["Ekk"])
    dG = np.einsum("ij,ijd->id", wA, Ckk) - np.einsum("ij,ijd->jd", wA, Ckk)
    # P[i,j] = sum_d q^_id k^_jd exp(G_id - G_jd)
    Cqk = np.einsum("id,jd,ijd->ijd", qn, kn, f["Eqk"])
    dqn = np.einsum("ij,jd,ijd->id", dP, kn, f["Eqk"])
    dkn = dkn + np.einsum("ij,id,ijd->jd", dP, qn, f["Eqk"])
    dG = dG + np.einsum("ij,ijd->id", dP, Cqk) - np.einsum("ij,ijd->jd", dP, Cqk)
    # KD = k^ exp(G), QD = q^ exp(G), KG = k^ exp(G_last - G)
    dkn = dkn + dKD * f["eG"] + dKG * f["eLG"]
    dqn = dqn + dQD * f["eG"]
    dG = dG + dKD * KD + dQD * QD - dKG * KG
    dGL = dGL + (dKG * KG).sum(0)
    dG[-1] += dGL
    return dict(dS=dS, dqn=dqn, dkn=dkn, dv=dv, db=db, dG=dG, dvn=dvn, dA=dA, dP=dP)


def grads_chunk(inp, do: np.ndarray, ds_final: Optional[np.ndarray], chunk_size: int = 64,
                flags: Optional[int] = None) -> dict:
    """Gradients of L = <dO, o> + <dS_T, S_T> for a :class:`gdn_inputs.GdnInputs`
    problem by the chunk-form reverse pass; same outputs as ``oracle.grad.grads``
    (dq, dk, dv, dbeta, dg, ds0, dh, o, s_final), fp64, and per sequence the
    gradient w.r.t. each chunk's v_new, dvn [NC,H,C,V] (rows past a partial
    chunk's end zero)."""
    flags = inp.flags if flags is None else flags
    C = chunk_size
    q_all, k_all, v_all = decode_bf16(inp.q), decode_bf16(inp.k), decode_bf16(inp.v)
    beta_all, g_all = decode_bf16(inp.beta), inp.g.astype(np.float64)
    N, H, K, V = inp.num_seqs, inp.H, inp.K, inp.V
    out = {n: np.zeros(x.shape) for n, x in (("dq", q_all), ("dk", k_all), ("dv", v_all), ("dbeta", beta_all),
                                             ("dg", g_all))}
    o_all = np.zeros((inp.B, inp.T, H, V))
    ds0 = np.zeros((N, H, K, V))
    s_fin = np.zeros((N, H, K, V))
    dh, dvn_all = [], []
    if inp.cu_seqlens is None:
        spans = [(n, n, 0, inp.T) for n in range(inp.B)]
    else:
        cu = [int(x) for x in inp.cu_seqlens]
        spans = [(n, 0, cu[n], cu[n + 1]) for n in range(N)]
    for n, row, a, e in spans:
        dh_n = np.zeros(((e - a + C - 1) // C, H, K, V))
        dvn_n = np.zeros(((e - a + C - 1) // C, H, C, V))
        for h in range(H):
            q, k, v = q_all[row, a:e, h], k_all[row, a:e, h], v_all[row, a:e, h]
            if flags & 1:
                rq = 1.0 / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
                rk = 1.0 / np.sqrt((k * k).sum(-1, keepdims=True) + 1e-6)
            else:
                rq, rk = np.ones((e - a, 1)), np.ones((e - a, 1))
            qn, kn = q * rq, k * rk
            bl = beta_all[row, a:e, h]
            b = 1.0 / (1.0 + np.exp(-bl)) if flags & 2 else bl
            g = g_all[row, a:e, h]
            gn = g * np.log(2.0) if inp.kda else np.repeat(g[:, None], K, axis=1)
            S = np.zeros((K, V)) if inp.initial_state is None else inp.initial_state[n, h].astype(np.float64)
            fwd = []
            for c0 in range(0, e - a, C):
                sl = slice(c0, min(c0 + C, e - a))
                G = np.cumsum(gn[sl], axis=0)
                f = _chunk_fwd(qn[sl], kn[sl], v[sl], b[sl], G, S, inp.scale)
                fwd.append((sl, f))
                o_all[row, a + sl.start:a + sl.stop, h] = f["O"]
                S = f["S_next"]
            s_fin[n, h] = S
            dS = np.zeros((K, V)) if ds_final is None else ds_final[n, h].astype(np.float64)
            dqn, dkn = np.zeros_like(qn), np.zeros_like(kn)
            dv, db, dgn = np.zeros_like(v), np.zeros_like(b), np.zeros_like(gn)
            for ci in range(len(fwd) - 1, -1, -1):
                sl, f = fwd[ci]
                r = _chunk_bwd(f, qn[sl], kn[sl], v[sl], b[sl], do[row, a + sl.start:a + sl.stop, h], dS,
                               inp.scale)
                dS = r["dS"]
                dh_n[ci, h] = dS
                dvn_n[ci, h, :sl.stop - sl.start] = r["dvn"]
                dqn[sl], dkn[sl], dv[sl], db[sl] = r["dqn"], r["dkn"], r["dv"], r["db"]
                # G is the cumulative sum of the chunk's gates: reverse cumulative sum
                dgn[sl] = np.cumsum(r["dG"][::-1], axis=0)[::-1]
            ds0[n, h] = dS
            # l2 norm x^ = x r: dx = r (dx^ - x^ (x^ . dx^)); sigmoid: b (1 - b)
            dq = rq * (dqn - qn * (qn * dqn).sum(-1, keepdims=True)) if flags & 1 else dqn
            dk = rk * (dkn - kn * (kn * dkn).sum(-1, keepdims=True)) if flags & 1 else dkn
            out["dq"][row, a:e, h] = dq
            out["dk"][row, a:e, h] = dk
            out["dv"][row, a:e, h] = dv
            out["dbeta"][row, a:e, h] = db * b * (1.0 - b) if flags & 2 else db
            out["dg"][row, a:e, h] = dgn * np.log(2.0) if inp.kda else dgn.sum(1)
        dh.append(dh_n)
        dvn_all.append(dvn_n)
    return dict(**out, ds0=ds0, dh=dh, dvn=dvn_all, o=o_all, s_final=s_fin)
