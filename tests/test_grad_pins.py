"""Pins of the gradient oracle (``oracle.grad``) against facts that do not
come from it: the C token recurrence, finite differences of the loss, the
exact affinity of the loss in the state entering a chunk, and closed forms.

The loss is L = <dO, o> + <dS_T, S_T> for seeded cotangents dO and dS_T.
"""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from oracle import grad as og
from oracle.chunk import decode_bf16


def _cot(inp, seed):
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((inp.B, inp.T, inp.H, inp.V))
    ds = rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1
    return do, ds


def _problems():
    rng = np.random.default_rng(77)
    return {
        "gdn_dense": gi.random_problem(rng, 2, 70, 2, 128, 128, gate_scale=0.3, with_initial_state=True),
        "gdn_packed": gi.random_problem(rng, 1, 90, 2, 128, 128, gate_scale=0.3, with_initial_state=True,
                                        cu_seqlens=np.array([0, 1, 66, 90])),
        "gdn_noflags": gi.random_problem(rng, 1, 40, 1, 128, 128, gate_scale=0.3, flags=gi.FLAG_OUTPUT_FINAL_STATE),
        "kda_dense": gi.random_problem(rng, 1, 70, 2, 128, 128, kda=True, gate_scale=0.3, with_initial_state=True),
    }


PROBLEMS = _problems()


@pytest.mark.parametrize("name", list(PROBLEMS))
def test_grad_forward_matches_c_recurrence(name):
    """The autograd forward is a second, independent transcription of the
    recurrence: o and S_T equal the C oracle's to rounding."""
    inp = PROBLEMS[name]
    do, ds = _cot(inp, 1)
    r = og.grads(inp, do, ds)
    o_ref, s_ref = oracle.recur(inp)
    assert np.abs(r["o"] - o_ref).max() <= 1e-10 * max(1.0, np.abs(o_ref).max())
    assert np.abs(r["s_final"] - s_ref).max() <= 1e-10 * max(1.0, np.abs(s_ref).max())


@pytest.mark.parametrize("name", list(PROBLEMS))
def test_grad_matches_finite_differences(name):
    """For a random direction D of each input X: (L(X + eps D) - L(X - eps D)) /
    (2 eps) = <dL/dX, D>, central differences in fp64 (error O(eps^2))."""
    inp = PROBLEMS[name]
    do, ds = _cot(inp, 2)
    r = og.grads(inp, do, ds)
    base = {"q": decode_bf16(inp.q), "k": decode_bf16(inp.k), "v": decode_bf16(inp.v),
            "beta": decode_bf16(inp.beta), "g": inp.g.astype(np.float64),
            "initial_state": inp.initial_state.astype(np.float64) if inp.initial_state is not None else None}
    grads = {"q": r["dq"], "k": r["dk"], "v": r["dv"], "beta": r["dbeta"], "g": r["dg"], "initial_state": r["ds0"]}
    rng = np.random.default_rng(3)
    eps = 1e-6
    for key, x in base.items():
        if x is None:
            continue
        d = rng.standard_normal(x.shape)
        lp = og.loss_value(inp, do, ds, overrides={key: x + eps * d})
        lm = og.loss_value(inp, do, ds, overrides={key: x - eps * d})
        fd = (lp - lm) / (2 * eps)
        an = float((grads[key] * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


@pytest.mark.parametrize("name", ["gdn_dense", "kda_dense", "gdn_packed"])
def test_state_entry_gradient_is_exact_affine_difference(name):
    """L restricted to the tokens from chunk c on is affine in the state S_c
    entering chunk c, so L_tail(S_c + D) - L_tail(S_c) = <dh_c, D> for any D
    (S_c from the C recurrence over the tokens before chunk c)."""
    inp = PROBLEMS[name]
    do, ds = _cot(inp, 4)
    r = og.grads(inp, do, ds)
    rng = np.random.default_rng(5)
    if inp.cu_seqlens is None:
        n, row, a, e = 0, 0, 0, inp.T
    else:
        n, row, a, e = 1, 0, int(inp.cu_seqlens[1]), int(inp.cu_seqlens[2])
    c = 1
    t0 = a + 64 * c
    assert t0 < e
    sl = lambda x, lo, hi: np.ascontiguousarray(x[row:row + 1, lo:hi])
    s0 = None if inp.initial_state is None else inp.initial_state[n:n + 1]
    head = gi.GdnInputs(**{**inp.__dict__, "B": 1, "T": t0 - a, "q": sl(inp.q, a, t0), "k": sl(inp.k, a, t0),
                           "v": sl(inp.v, a, t0), "g": sl(inp.g, a, t0), "beta": sl(inp.beta, a, t0),
                           "initial_state": s0, "cu_seqlens": None})
    _, s_c = oracle.recur(head)
    tail = gi.GdnInputs(**{**inp.__dict__, "B": 1, "T": e - t0, "q": sl(inp.q, t0, e), "k": sl(inp.k, t0, e),
                           "v": sl(inp.v, t0, e), "g": sl(inp.g, t0, e), "beta": sl(inp.beta, t0, e),
                           "initial_state": s_c, "cu_seqlens": None})
    do_t = np.ascontiguousarray(do[row:row + 1, t0:e])
    ds_t = ds[n:n + 1]
    d = rng.standard_normal(s_c.shape)
    diff = og.loss_value(tail, do_t, ds_t, overrides={"initial_state": s_c + d}) - og.loss_value(tail, do_t, ds_t)
    an = float((r["dh"][n][c] * d[0]).sum())
    assert abs(diff - an) <= 1e-9 * max(1.0, abs(an))
    # the state entering chunk 0 is S_0
    assert np.array_equal(r["dh"][n][0], r["ds0"][n])


def test_beta_zero_closed_form():
    """beta = 0 (no sigmoid): S_t = exp(G_t) S_0, o_t = scale exp(G_t) S_0^T qn_t,
    so dS_0 = sum_t scale exp(G_t) qn_t dO_t^T + exp(G_T) dS_T, dv = 0 and
    dk = 0 (the keys only enter through beta)."""
    rng = np.random.default_rng(11)
    inp = gi.random_problem(rng, 1, 50, 2, 128, 128, gate_scale=0.2, with_initial_state=True,
                            flags=gi.FLAG_L2NORM_QK | gi.FLAG_OUTPUT_FINAL_STATE)
    inp = gi.GdnInputs(**{**inp.__dict__, "beta": np.zeros_like(inp.beta)})
    do, ds = _cot(inp, 12)
    r = og.grads(inp, do, ds)
    q = decode_bf16(inp.q)[0]
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6)
    G = np.cumsum(inp.g[0].astype(np.float64), axis=0)          # [T,H]
    ref = np.einsum("th,thk,thv->hkv", inp.scale * np.exp(G), qn, do[0]) + np.exp(G[-1])[:, None, None] * ds[0]
    assert np.abs(r["ds0"][0] - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.abs(r["dv"]).max() == 0.0
    assert np.abs(r["dk"]).max() == 0.0


@pytest.mark.parametrize("kda", [False, True])
def test_gate_chain_rule_matches_finite_differences(kda):
    """Loss as a function of the raw gate x and the gate parameters (A_log,
    dt_bias), through oracle.gate: central differences along random directions
    equal <grad, D> for the gradients of grads() chained by gate_grads()."""
    from oracle import gate as ogate
    rng = np.random.default_rng(21 + kda)
    inp = gi.random_problem(rng, 1, 70, 2, 128, 128, kda=kda, with_initial_state=True)
    H, K = inp.H, inp.K
    x = rng.standard_normal(inp.g.shape)
    a_log = rng.uniform(0, np.log(16), H)
    dt = rng.standard_normal((H, K) if kda else (H,)) * 0.1
    gate = ogate.kda_gate if kda else ogate.gdn_gate
    inp = gi.GdnInputs(**{**inp.__dict__, "g": gate(x, a_log, dt)})
    do, ds = _cot(inp, 22)
    r = og.grads(inp, do, ds)
    gg = og.gate_grads(kda, x, a_log, dt, r["dg"])
    eps = 1e-6
    for key, val, grad in (("x", x, gg["dx"]), ("a_log", a_log, gg["da_log"]), ("dt", dt, gg["ddt_bias"])):
        d = rng.standard_normal(val.shape)
        args = lambda s: {"x": x, "a_log": a_log, "dt": dt, key: val + s * eps * d}
        lp = og.loss_value(inp, do, ds, overrides={"g": gate(*args(1).values())})
        lm = og.loss_value(inp, do, ds, overrides={"g": gate(*args(-1).values())})
        fd = (lp - lm) / (2 * eps)
        an = float((grad * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (key, fd, an)


def _host_normalised(rng, T, H, kda):
    """No in-kernel flags: q, k of unit norm and beta in (0, 1) given directly."""
    base = gi.random_problem(rng, 1, T, H, 128, 128, kda=kda, gate_scale=0.3, with_initial_state=True,
                             flags=gi.FLAG_OUTPUT_FINAL_STATE)
    out = {}
    for name in ("q", "k"):
        x = decode_bf16(getattr(base, name))
        out[name] = gi.f32_to_bf16_bits((x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32))
    b = 1.0 / (1.0 + np.exp(-decode_bf16(base.beta)))
    out["beta"] = gi.f32_to_bf16_bits(b.astype(np.float32))
    return gi.GdnInputs(**{**base.__dict__, **out})


def _chunk_form_cases():
    rng = np.random.default_rng(131)
    return {
        "gdn_dense": PROBLEMS["gdn_dense"],
        "gdn_packed": PROBLEMS["gdn_packed"],
        "kda_dense": PROBLEMS["kda_dense"],
        "kda_packed": gi.random_problem(rng, 1, 90, 2, 128, 128, kda=True, gate_scale=0.3, with_initial_state=True,
                                        cu_seqlens=np.array([0, 1, 66, 90])),
        "kda_host_normalised": _host_normalised(rng, 70, 2, True),
        "kda_reset": (lambda p: gi.GdnInputs(**{**p.__dict__, "g": np.where(
            np.arange(p.T)[None, :, None, None] == 37, -1000.0, p.g).astype(np.float32)}))(
            gi.random_problem(rng, 1, 80, 1, 128, 128, kda=True, gate_scale=0.3, with_initial_state=True)),
    }


CHUNK_FORM = _chunk_form_cases()


@pytest.mark.parametrize("chunk", [4, 16, 64])
@pytest.mark.parametrize("name", list(CHUNK_FORM))
def test_chunk_form_gradients_equal_autograd(name, chunk):
    """oracle.grad_chunk (the chunked reverse pass, step by step) equals the
    reverse-mode derivative of the token recurrence: every input gradient, the
    gradient of the state entering every chunk, and the forward it runs."""
    from oracle import grad_chunk as gc
    inp = CHUNK_FORM[name]
    do, ds = _cot(inp, 132)
    ref = og.grads(inp, do, ds, chunk_size=chunk)
    got = gc.grads_chunk(inp, do, ds, chunk_size=chunk)
    for key in ("dq", "dk", "dv", "dbeta", "dg", "ds0", "o", "s_final"):
        err = np.abs(got[key] - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30)
        assert err <= 1e-9, (key, err)
    for a, b in zip(got["dh"], ref["dh"]):
        assert np.abs(a - b).max() <= 1e-9 * max(np.abs(b).max(), 1e-30)
