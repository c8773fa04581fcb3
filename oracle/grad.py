"""Gradients of the gated delta rule forward in fp64 (TEST INFRASTRUCTURE ONLY).

Reverse-mode differentiation (PyTorch autograd on the CPU, fp64) of the
token-by-token recurrence that ``oracle.recur`` computes in C:

    q^ = l2norm(q) (optional), k^ = l2norm(k) (optional), b = sigmoid(beta) (optional),
    S_t = D_t S_{t-1};  S_t += b_t k^_t (v_t - S_t^T k^_t)^T;  o_t = scale S_t^T q^_t,

with D_t = exp(g_t) (GDN, natural log) or diag(2^{g_t,d}) (KDA, log2), the
l2norm ``x / sqrt(sum x^2 + 1e-6)`` (the ``_l2norm`` helper of the 2026-09-10
"Diff Coverage" page) and K x V states, as the forward oracle. For an output
cotangent dO and a final-state cotangent dS_T, the loss
L = <dO, o> + <dS_T, S_T> is differentiated with respect to the raw inputs
(q, k, v, beta, g, S_0) and to the state entering every chunk of C tokens
(the quantity a reverse state pass computes).

Pinned by tests/test_grad_pins.py: its forward equals ``oracle.recur``, and
directional finite differences of L match every gradient.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from .chunk import decode_bf16


def _forward(q, k, v, beta, g, s0, scale, kda, flags, chunk_size, keep_states):
    """q, k [T,H,K], v [T,H,V], beta [T,H], g [T,H] or [T,H,K], s0 [H,K,V] (one
    sequence, fp64 tensors). Returns o [T,H,V], S_T [H,K,V] and the list of
    states entering each chunk (each retaining its gradient)."""
    if flags & 1:
        q = q / torch.sqrt((q * q).sum(-1, keepdim=True) + 1e-6)
        k = k / torch.sqrt((k * k).sum(-1, keepdim=True) + 1e-6)
    b = torch.sigmoid(beta) if flags & 2 else beta
    S = s0
    outs = []
    entry = []
    for t in range(q.shape[0]):
        if keep_states and t % chunk_size == 0:
            S = S.clone()
            S.retain_grad()
            entry.append(S)
        if kda:
            S = S * torch.exp2(g[t])[..., :, None]
        else:
            S = S * torch.exp(g[t])[..., None, None]
        pred = torch.einsum("hkv,hk->hv", S, k[t])
        S = S + b[t][:, None, None] * k[t][:, :, None] * (v[t] - pred)[:, None, :]
        outs.append(scale * torch.einsum("hkv,hk->hv", S, q[t]))
    return torch.stack(outs, 0), S, entry


def grads(inp, do: np.ndarray, ds_final: Optional[np.ndarray], chunk_size: int = 64,
          flags: Optional[int] = None) -> dict:
    """Gradients of L = <dO, o> + <dS_T, S_T> for a :class:`gdn_inputs.GdnInputs`
    problem. do: [B,T,H,V]; ds_final: [N,H,K,V] or None (zero).

    Returns fp64 numpy arrays: dq, dk, dv [B,T,H,*], dbeta [B,T,H], dg (shape
    of g), ds0 [N,H,K,V], dh (list per sequence of [NC,H,K,V]: gradient with
    respect to the state entering each chunk), and o, s_final (the forward)."""
    flags = inp.flags if flags is None else flags
    f64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    q_all, k_all, v_all = f64(decode_bf16(inp.q)), f64(decode_bf16(inp.k)), f64(decode_bf16(inp.v))
    b_all, g_all = f64(decode_bf16(inp.beta)), f64(inp.g)
    for t in (q_all, k_all, v_all, b_all, g_all):
        t.requires_grad_(True)
    N = inp.num_seqs
    s0_all = torch.zeros((N, inp.H, inp.K, inp.V), dtype=torch.float64) if inp.initial_state is None \
        else f64(inp.initial_state)
    s0_all.requires_grad_(True)
    do_t = f64(do)
    dsf = None if ds_final is None else f64(ds_final)
    if inp.cu_seqlens is None:
        spans = [(n, n, 0, inp.T) for n in range(inp.B)]           # (seq, batch row, start, end)
    else:
        cu = [int(x) for x in inp.cu_seqlens]
        spans = [(n, 0, cu[n], cu[n + 1]) for n in range(N)]
    loss = torch.zeros((), dtype=torch.float64)
    entries, outs, finals = [], [], []
    for n, b, a, e in spans:
        o, S, entry = _forward(q_all[b, a:e], k_all[b, a:e], v_all[b, a:e], b_all[b, a:e], g_all[b, a:e],
                               s0_all[n], inp.scale, inp.kda, flags, chunk_size, True)
        loss = loss + (do_t[b, a:e] * o).sum()
        if dsf is not None:
            loss = loss + (dsf[n] * S).sum()
        entries.append(entry)
        outs.append((b, a, e, o))
        finals.append(S)
    loss.backward()
    o_np = np.zeros(tuple(do.shape))
    for b, a, e, o in outs:
        o_np[b, a:e] = o.detach().numpy()
    return dict(
        dq=q_all.grad.numpy(), dk=k_all.grad.numpy(), dv=v_all.grad.numpy(), dbeta=b_all.grad.numpy(),
        dg=g_all.grad.numpy(), ds0=s0_all.grad.numpy(),
        dh=[np.stack([s.grad.numpy() for s in entry], 0) for entry in entries],
        o=o_np, s_final=np.stack([s.detach().numpy() for s in finals], 0),
    )


def loss_value(inp, do: np.ndarray, ds_final: Optional[np.ndarray], flags: Optional[int] = None,
               overrides: Optional[dict] = None) -> float:
    """L = <dO, o> + <dS_T, S_T> in fp64, with float inputs in ``overrides``
    (q, k, v, beta as decoded values, g, initial_state) replacing those of
    ``inp`` (used by the finite-difference pins)."""
    flags = inp.flags if flags is None else flags
    ov = overrides or {}
    f64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    q = f64(ov.get("q", decode_bf16(inp.q)))
    k = f64(ov.get("k", decode_bf16(inp.k)))
    v = f64(ov.get("v", decode_bf16(inp.v)))
    beta = f64(ov.get("beta", decode_bf16(inp.beta)))
    g = f64(ov.get("g", inp.g))
    N = inp.num_seqs
    s0 = ov.get("initial_state", inp.initial_state)
    s0 = torch.zeros((N, inp.H, inp.K, inp.V), dtype=torch.float64) if s0 is None else f64(s0)
    if inp.cu_seqlens is None:
        spans = [(n, n, 0, inp.T) for n in range(inp.B)]
    else:
        cu = [int(x) for x in inp.cu_seqlens]
        spans = [(n, 0, cu[n], cu[n + 1]) for n in range(N)]
    total = 0.0
    with torch.no_grad():
        for n, b, a, e in spans:
            o, S, _ = _forward(q[b, a:e], k[b, a:e], v[b, a:e], beta[b, a:e], g[b, a:e], s0[n], inp.scale,
                               inp.kda, flags, 64, False)
            total += float((f64(do)[b, a:e] * o).sum())
            if ds_final is not None:
                total += float((f64(ds_final)[n] * S).sum())
    return total


def gate_grads(kda: bool, x: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray, dg: np.ndarray) -> dict:
    """Chain rule through the in-kernel gate of ``oracle.gate`` (fp64 autograd):
    for the gradient dg of the loss with respect to g = -exp(A_log) softplus(x
    + dt_bias) (divided by ln 2 for KDA), returns the gradients with respect to
    x (shape of x), A_log [H] and dt_bias ([H] GDN, [H,K] KDA)."""
    f64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    xt, at, bt = f64(x), f64(a_log), f64(dt_bias)
    for t in (xt, at, bt):
        t.requires_grad_(True)
    zero = torch.zeros((), dtype=torch.float64)
    if kda:
        g = -torch.exp(at)[:, None] * torch.logaddexp(zero, xt + bt) / float(np.log(2.0))
    else:
        g = -torch.exp(at) * torch.logaddexp(zero, xt + bt)
    (g * f64(dg)).sum().backward()
    return dict(dx=xt.grad.numpy(), da_log=at.grad.numpy(), ddt_bias=bt.grad.numpy())
