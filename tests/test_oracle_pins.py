"""Pins of the oracle against facts fixed by the mathematics, not by itself.

Each test names the part of the oracle it pins and the plausible mistake it
would catch. Both oracle functions are covered: ``oracle.recur`` (C token
recurrence) and ``oracle.chunk`` (numpy chunk form derived from it).
"""
import glob
import json
import math
import os

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _from_json(d):
    B, T, H, K, V = d["B"], d["T"], d["H"], d["K"], d["V"]
    q = np.asarray(d["q"], dtype=np.float32).reshape(B, T, H, K)
    k = np.asarray(d["k"], dtype=np.float32).reshape(B, T, H, K)
    v = np.asarray(d["v"], dtype=np.float32).reshape(B, T, H, V)
    beta = np.asarray(d["beta"], dtype=np.float32).reshape(B, T, H)
    g = np.asarray(d["g"], dtype=np.float32).reshape((B, T, H, K) if d["kda"] else (B, T, H))
    cu = d.get("cu_seqlens")
    N = B if cu is None else len(cu) - 1
    s0 = d.get("initial_state")
    if s0 is not None:
        s0 = np.asarray(s0, dtype=np.float32).reshape(N, H, K, V)
    for name, arr in (("q", q), ("k", k), ("v", v), ("beta", beta)):
        assert np.array_equal(gi.bf16_bits_to_f32(gi.f32_to_bf16_bits(arr)), arr), name + " not bf16-exact"
    return gi.GdnInputs(name="golden", B=B, T=T, H=H, K=K, V=V, kda=d["kda"], flags=d["flags"],
                        scale=d["scale"], q=gi.f32_to_bf16_bits(q), k=gi.f32_to_bf16_bits(k),
                        v=gi.f32_to_bf16_bits(v), g=g, beta=gi.f32_to_bf16_bits(beta), initial_state=s0,
                        cu_seqlens=None if cu is None else np.asarray(cu, dtype=np.int32))


def _rel(a, b):
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(GOLDEN, "*.json"))), ids=os.path.basename)
@pytest.mark.parametrize("method", ["recur", "chunk2", "chunk64"])
def test_golden_hand_derived(oracle_lib, path, method):
    """Hand-derived values of tiny problems (decay, delta rule ordering, scale,
    sigmoid(0)=1/2, per-document states). Catches a wrong sign, a transposed
    state, decay applied after the update, or documents leaking into each other."""
    d = json.load(open(path))
    inp = _from_json(d)
    if method == "recur":
        o, fs = oracle.recur(inp)
    else:
        o, fs, _ = oracle.chunk(inp, chunk_size=int(method[5:]))
    N = inp.num_seqs
    np.testing.assert_allclose(o.reshape(inp.B * inp.T, inp.V), np.asarray(d["o"]).reshape(-1, inp.V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(fs.reshape(N, inp.K, inp.V), np.asarray(d["final_state"]).reshape(N, inp.K, inp.V),
                               rtol=0, atol=1e-12)


CASES = [
    # T, C, K, kda, flags, init
    (1, 4, 8, False, 7, True), (3, 4, 8, False, 4, True), (17, 4, 8, True, 7, True),
    (63, 16, 8, False, 7, False), (64, 16, 8, True, 5, True), (65, 16, 8, False, 6, True),
    (200, 64, 16, False, 7, True), (200, 64, 16, True, 7, True), (130, 64, 128, False, 7, True),
    (129, 64, 128, True, 7, False), (64, 64, 128, False, 4, False), (17, 64, 128, True, 7, True),
]


@pytest.mark.parametrize("T,C,K,kda,flags,init", CASES)
def test_chunk_form_equals_recurrence(oracle_lib, T, C, K, kda, flags, init):
    """The chunk form and the token recurrence are two independent codes;
    they must agree to rounding. Catches a dropped term in the WY terms, a
    wrong mask (diagonal in A or missing in the QK term), a wrong decay
    exponent, a wrong triangular system for T, partial-chunk padding."""
    rng = np.random.default_rng(T * 1000 + C + K + kda)
    inp = gi.random_problem(rng, 2, T, 3, K, K, kda=kda, with_initial_state=init, flags=flags)
    o1, s1 = oracle.recur(inp)
    o2, s2, _ = oracle.chunk(inp, chunk_size=C)
    assert _rel(o2, o1) < 1e-10
    assert _rel(s2, s1) < 1e-10


@pytest.mark.parametrize("kda", [False, True])
def test_beta_zero_closed_form(oracle_lib, kda):
    """beta = 0: the state only decays, S_T = e^{sum g} S0 (per channel for
    KDA), and o_t = scale * (decayed S0)^T q^_t. Catches an error in the decay
    or in the output contraction, independently of the delta rule."""
    rng = np.random.default_rng(11)
    T, H, K, V = 37, 2, 16, 8
    inp = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True,
                            flags=gi.FLAG_L2NORM_QK, gate_scale=0.3)
    inp.beta[:] = 0
    s0 = inp.initial_state.astype(np.float64)
    g = inp.g.astype(np.float64)
    qh = oracle.l2norm(oracle.decode_bf16(inp.q))
    if kda:
        G = np.cumsum(g[0], axis=0)                         # [T,H,K]
        dec = np.exp2(G)                                    # [T,H,K]
        S_t = dec[:, :, :, None] * s0[0][None]              # [T,H,K,V]
    else:
        G = np.cumsum(g[0], axis=0)                         # [T,H]
        S_t = np.exp(G)[:, :, None, None] * s0[0][None]
    o_exp = inp.scale * np.einsum("thkv,thk->thv", S_t, qh[0])
    for fn in ("recur", "chunk"):
        if fn == "recur":
            o, fs = oracle.recur(inp)
        else:
            o, fs, _ = oracle.chunk(inp, chunk_size=16)
        assert _rel(fs[0], S_t[-1]) < 1e-12
        assert _rel(o[0], o_exp) < 1e-12


@pytest.mark.parametrize("kda", [False, True])
def test_retrieval(oracle_lib, kda):
    """With ||k|| = 1 and beta = 1 the delta rule stores v exactly under k:
    S_t^T k_t = v_t, whatever the decay and the earlier state. With q = k and
    scale s, o_t = s v_t. Catches decay applied after the update, a wrong sign
    in (v - S^T k), or beta applied to the wrong factor."""
    rng = np.random.default_rng(5)
    T, H, K, V = 50, 2, 16, 8
    inp = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True, flags=0, scale=0.75)
    k = np.zeros((1, T, H, K), dtype=np.float32)
    for t in range(T):
        for h in range(H):
            idx = rng.choice(K, 4, replace=False)
            k[0, t, h, idx] = rng.choice([-0.5, 0.5], 4)
    inp.k = gi.f32_to_bf16_bits(k)
    inp.q = inp.k.copy()
    inp.beta[:] = gi.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    v = oracle.decode_bf16(inp.v)
    for fn in ("recur", "chunk"):
        o = oracle.recur(inp)[0] if fn == "recur" else oracle.chunk(inp, chunk_size=16)[0]
        np.testing.assert_allclose(o, 0.75 * v, rtol=0, atol=1e-12)


def test_l2norm_epsilon_placement(oracle_lib):
    """In-kernel normalisation is x / sqrt(sum(x^2) + 1e-6). One token, g=0,
    beta=1, q=k, S0=0 gives o = scale * ||k^||^2 v = scale * s/(s+1e-6) v with
    s = sum(k^2). With s = 4 * 2^-16 the factor is visibly below 1, so a
    missing or misplaced epsilon (or no normalisation) fails."""
    K, V = 8, 4
    k = np.zeros((1, 1, 1, K), np.float32)
    k[0, 0, 0, :4] = [2.0 ** -8, -(2.0 ** -8), 2.0 ** -8, 2.0 ** -8]
    v = np.arange(1, V + 1, dtype=np.float32).reshape(1, 1, 1, V)
    kb = gi.f32_to_bf16_bits(k)
    inp = gi.GdnInputs(name="eps", B=1, T=1, H=1, K=K, V=V, kda=False, flags=gi.FLAG_L2NORM_QK, scale=1.0,
                       q=kb.copy(), k=kb, v=gi.f32_to_bf16_bits(v), g=np.zeros((1, 1, 1), np.float32),
                       beta=gi.f32_to_bf16_bits(np.ones((1, 1, 1), np.float32)), initial_state=None, cu_seqlens=None)
    s = 4 * 2.0 ** -16
    expect = s / (s + 1e-6) * v.astype(np.float64)
    for fn in ("recur", "chunk"):
        o = oracle.recur(inp)[0] if fn == "recur" else oracle.chunk(inp, chunk_size=4)[0]
        np.testing.assert_allclose(o, expect, rtol=1e-13, atol=0)
    x = np.random.default_rng(0).standard_normal((5, 16))
    ss = (x * x).sum(-1)
    np.testing.assert_allclose((oracle.l2norm(x) ** 2).sum(-1), ss / (ss + 1e-6), rtol=1e-14)


@pytest.mark.parametrize("kda", [False, True])
def test_reset_by_large_negative_gate(oracle_lib, kda):
    """g = -1000 at token t0 multiplies the old state by e^-1000 = 0: outputs
    from t0 on and the final state are independent of S0 and of every earlier
    token. The chunk form must also survive it (mask before exp: an exp of a
    positive difference would overflow to inf and give NaN)."""
    rng = np.random.default_rng(9)
    T, H, K, V, t0 = 90, 2, 16, 16, 41
    a = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True)
    if kda:
        a.g[0, t0] = -1000.0
    else:
        a.g[0, t0] = -1000.0
    b = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True)
    for name in ("q", "k", "v", "g", "beta"):
        getattr(b, name)[0, t0:] = getattr(a, name)[0, t0:]
    for fn in ("recur", "chunk"):
        if fn == "recur":
            oa, sa = oracle.recur(a)
            ob, sb = oracle.recur(b)
        else:
            oa, sa, _ = oracle.chunk(a, chunk_size=16)
            ob, sb, _ = oracle.chunk(b, chunk_size=16)
        assert np.isfinite(oa).all() and np.isfinite(sa).all()
        assert _rel(ob[0, t0:], oa[0, t0:]) < 1e-12
        assert _rel(sb, sa) < 1e-12
        assert _rel(ob[0, :t0], oa[0, :t0]) > 1e-3   # the prefix does differ


@pytest.mark.parametrize("kda", [False, True])
def test_affine_state_summary(oracle_lib, kda):
    """The final state is affine in S0: S_T(S0) = M S0 + S_T(0), with M the
    product of per-chunk transitions e^{G_last} I - (k * e^{G_last - G})^T W
    (the state summary of _compute_gdn_state_summary_from_prepared on the
    2026-09-10 page; per-channel decays for KDA). M is built from the chunk
    form's W and keys, S_T from the token recurrence: a wrong W, a wrong key
    decay or a wrong decay of the carried state fails here."""
    rng = np.random.default_rng(21)
    T, H, K, V, C = 100, 2, 16, 8, 16
    inp = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True, gate_scale=0.01)
    _, _, inters = oracle.chunk(inp, chunk_size=C, keep=True)
    it = inters[0]
    G, W, kk = it["G"], it["W"], it["k"]          # [1,H,NC,C(,K)], [1,H,NC,C,K], [1,H,NC,C,K]
    NC = G.shape[2]
    M = np.broadcast_to(np.eye(K), (1, H, K, K)).copy()
    for c in range(NC):
        if kda:
            Gc = G[:, :, c]
            kd = kk[:, :, c] * np.exp2(Gc[:, :, -1:, :] - Gc)
            trans = np.eye(K) * np.exp2(Gc[:, :, -1, :])[..., None, :] - np.swapaxes(kd, -1, -2) @ W[:, :, c]
        else:
            Gc = G[:, :, c]
            kd = kk[:, :, c] * np.exp(Gc[..., -1:] - Gc)[..., None]
            trans = np.exp(Gc[..., -1])[..., None, None] * np.eye(K) - np.swapaxes(kd, -1, -2) @ W[:, :, c]
        M = trans @ M
    _, s_with = oracle.recur(inp)
    zero = gi.GdnInputs(**{**inp.__dict__, "initial_state": None})
    _, s_zero = oracle.recur(zero)
    lhs = s_with - s_zero
    rhs = M @ inp.initial_state.astype(np.float64)
    assert _rel(lhs, rhs) < 1e-10
    assert np.abs(lhs).max() > 1e-3 * np.abs(s_with).max()


@pytest.mark.parametrize("kda", [False, True])
def test_packed_equals_per_document_dense(oracle_lib, kda):
    """cu_seqlens: the packed run equals separate dense runs of every document,
    each with its own initial state (lengths 1 and 17 included)."""
    rng = np.random.default_rng(3)
    lengths = [17, 1, 64, 30, 65]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, K, V = int(cu[-1]), 2, 16, 8
    inp = gi.random_problem(rng, 1, T, H, K, V, kda=kda, with_initial_state=True, cu_seqlens=cu)
    o_p, s_p = oracle.recur(inp)
    o_c, s_c, _ = oracle.chunk(inp, chunk_size=16)
    assert _rel(o_c, o_p) < 1e-10 and _rel(s_c, s_p) < 1e-10
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        sl = lambda x: np.ascontiguousarray(x[:, a:b])
        doc = gi.GdnInputs(name="doc", B=1, T=int(b - a), H=H, K=K, V=V, kda=kda, flags=inp.flags, scale=inp.scale,
                           q=sl(inp.q), k=sl(inp.k), v=sl(inp.v), g=sl(inp.g), beta=sl(inp.beta),
                           initial_state=inp.initial_state[n:n + 1].copy(), cu_seqlens=None)
        o_d, s_d = oracle.recur(doc)
        np.testing.assert_array_equal(o_p[:, a:b], o_d)
        np.testing.assert_array_equal(s_p[n], s_d[0])


def test_kda_with_channel_constant_gate_is_gdn(oracle_lib):
    """A KDA gate equal on every channel, c (log2), is GDN with g = c ln 2.
    Pins the KDA decay against the GDN decay (the GDN decay is pinned by the
    beta = 0 closed form)."""
    rng = np.random.default_rng(4)
    T, H, K, V = 70, 2, 16, 8
    kda = gi.random_problem(rng, 1, T, H, K, V, kda=True, with_initial_state=True)
    c = -np.abs(rng.standard_normal((1, T, H))).astype(np.float32)
    kda.g = np.ascontiguousarray(np.repeat(c[..., None], K, axis=-1))
    gdn = gi.GdnInputs(**{**kda.__dict__, "kda": False, "g": (c.astype(np.float64) * math.log(2.0)).astype(np.float32)})
    o1, s1 = oracle.recur(kda)
    o2, s2 = oracle.recur(gdn)
    assert _rel(o1, o2) < 1e-5 and _rel(s1, s2) < 1e-5
    kda.g[:] = 0.0
    gdn.g[:] = 0.0
    o1, s1 = oracle.recur(kda)
    o2, s2 = oracle.recur(gdn)
    assert _rel(o1, o2) < 1e-14 and _rel(s1, s2) < 1e-14


def test_unit_subset_matches_full_run(oracle_lib):
    """Restricting the recurrence to a list of (sequence, head) units computes
    exactly those rows (used for sampled parity at full size)."""
    rng = np.random.default_rng(8)
    inp = gi.random_problem(rng, 3, 40, 4, 16, 8, with_initial_state=True)
    o, s = oracle.recur(inp)
    units = [(2, 1), (0, 3)]
    ou, su = oracle.recur(inp, units=units)
    for n, h in units:
        np.testing.assert_array_equal(ou[n, :, h], o[n, :, h])
        np.testing.assert_array_equal(su[n, h], s[n, h])
    assert np.abs(ou[1]).max() == 0.0


def _segment(inp, a, b):
    """Tokens a..b-1 of a dense single-sequence problem, no initial state."""
    sl = lambda x: np.ascontiguousarray(x[:, a:b])
    return gi.GdnInputs(**{**inp.__dict__, "T": b - a, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v),
                           "g": sl(inp.g), "beta": sl(inp.beta), "initial_state": None})


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("packed", [False, True])
def test_state_summary_against_recurrence(oracle_lib, kda, packed):
    """oracle.state_summary (``_compute_gdn_state_summary_from_prepared``): S
    equals the token recurrence's final state from a zero state, and
    M S0 + S its final state from S0 (so M is the exact transition); the apply
    step reproduces the latter. A wrong transition term (decay, key decay, W)
    or a wrong chunk order fails one of them."""
    rng = np.random.default_rng(31 + kda + 2 * packed)
    H, K, V, C = 2, 16, 8, 16
    cu = np.asarray([0, 7, 40, 100], dtype=np.int32) if packed else None
    inp = gi.random_problem(rng, 1, 100, H, K, V, kda=kda, with_initial_state=True, gate_scale=0.05,
                            cu_seqlens=cu)
    M, S = oracle.state_summary(inp, chunk_size=C)
    zero = gi.GdnInputs(**{**inp.__dict__, "initial_state": None})
    _, s_zero = oracle.recur(zero)
    _, s_with = oracle.recur(inp)
    assert _rel(S, s_zero) < 1e-10
    assert _rel(M @ inp.initial_state.astype(np.float64) + S, s_with) < 1e-10
    assert _rel(oracle.apply_state_summary(M, S, inp.initial_state), s_with) < 1e-10
    assert np.abs(M - np.eye(K)).max() > 1e-2      # not trivially the identity


@pytest.mark.parametrize("kda", [False, True])
def test_state_summary_composes_over_segments(oracle_lib, kda):
    """Sequence-parallel use of the summary: the final state of a sequence
    equals the second segment's summary applied to the first segment's final
    state (segments split at a chunk boundary and mid-chunk)."""
    rng = np.random.default_rng(41 + kda)
    H, K, V, C = 2, 16, 8, 16
    inp = gi.random_problem(rng, 1, 90, H, K, V, kda=kda, gate_scale=0.05)
    _, s_full = oracle.recur(inp)
    for t0 in (32, 45):
        _, s_a = oracle.recur(_segment(inp, 0, t0))
        M, S = oracle.state_summary(_segment(inp, t0, 90), chunk_size=C)
        assert _rel(oracle.apply_state_summary(M, S, s_a), s_full) < 1e-10
