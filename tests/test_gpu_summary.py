"""GPU parity of the affine state summary and its apply step (through the C ABI).

``gdn_state_summary`` / ``kda_state_summary`` against ``oracle.state_summary``
(the summary of ``_compute_gdn_state_summary_from_prepared``):
max |X - X_ref| / max |X_ref| <= 1e-3 for both the transition M and the
zero-state final state S. ``gdn_state_summary_apply`` against the token
recurrence's final state from the same initial state, and the two-segment
composition against the recurrence over the whole sequence.
"""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import S_RTOL, run_gpu, s_err, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_gated_delta_03_amd as m
    return m


def _summary_gpu(gdn, inp):
    d = to_device(inp)
    M, S = gdn.state_summary(d["k"], d["v"], d["g"], d["beta"], q=d["q"], cu_seqlens=inp.cu_seqlens, kda=inp.kda,
                             l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2))
    torch.cuda.synchronize()
    return M, S


def _mild(seed, B, T, H, kda=False, cu=None):
    """Gates ~ -0.02 softplus(N(0,1)): the transition stays of order one."""
    rng = np.random.default_rng(seed)
    return gi.random_problem(rng, B, T, H, 128, 128, kda=kda, gate_scale=0.02,
                             cu_seqlens=None if cu is None else np.asarray(cu, dtype=np.int32))


# the workload recipes (strong gates: M decays to ~0 over a few chunks) and
# mild gates (M of order one), dense and packed, both gate kinds
CASES = [
    ("gdn_B2_T300_H3", lambda: gi.make_inputs("gdn", B=2, T=300, H=3)),
    ("gdn_T1", lambda: gi.make_inputs("gdn", B=2, T=1, H=2)),
    ("gdn_T2048_H2", lambda: gi.make_inputs("long", T=2048, H=2)),
    ("varlen_docs", lambda: gi.make_inputs("varlen", H=3, doc_lengths=[1, 17, 64, 65, 200])),
    ("wide_B4_T130_H16", lambda: gi.make_inputs("gdn", B=4, T=130, H=16)),
    ("kda_B1_T200_H2", lambda: gi.make_inputs("kda", B=1, T=200, H=2)),
    ("mild_B2_T300_H3", lambda: _mild(1, 2, 300, 3)),
    ("mild_varlen", lambda: _mild(2, 1, 400, 2, cu=[0, 1, 65, 200, 400])),
    ("mild_kda_B1_T200_H2", lambda: _mild(3, 1, 200, 2, kda=True)),
    ("mild_kda_varlen", lambda: _mild(4, 1, 150, 2, kda=True, cu=[0, 40, 150])),
]


@pytest.mark.parametrize("name,make", CASES, ids=[n for n, _ in CASES])
def test_state_summary_parity(gdn, name, make):
    """S: relative to max |S_ref|. M: relative to max(max |M_ref|, 0.1) (under
    the workload gates M vanishes; the floor keeps the bound meaningful)."""
    inp = make()
    _say("summary case", name, "B,T,H =", inp.B, inp.T, inp.H, "kda", inp.kda,
         "docs", None if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1)
    M, S = _summary_gpu(gdn, inp)
    M_ref, S_ref = oracle.state_summary(inp)
    M, S = M.cpu().numpy(), S.cpu().numpy()
    assert np.isfinite(M).all() and np.isfinite(S).all()
    em = float(np.abs(M - M_ref).max() / max(np.abs(M_ref).max(), 0.1))
    es = s_err(S, S_ref)
    _say("  transition err %.3e (max |M_ref| %.2e)   state rel err %.3e" % (em, np.abs(M_ref).max(), es))
    assert em <= S_RTOL
    assert es <= S_RTOL


@pytest.mark.parametrize("kda", [False, True])
def test_summary_apply_matches_recurrence(gdn, kda):
    """M S0 + S from the GPU summary equals the token recurrence from S0, and
    the whole-pass entry's final state; a NULL state_in gives S itself."""
    rng = np.random.default_rng(5 + kda)
    inp = gi.random_problem(rng, 2, 190, 2, 128, 128, kda=kda, gate_scale=0.02, with_initial_state=True)
    M, S = _summary_gpu(gdn, inp)
    s0 = torch.from_numpy(inp.initial_state).cuda()
    out = gdn.state_summary_apply(M, S, s0)
    zero = gdn.state_summary_apply(M, S, None)
    torch.cuda.synchronize()
    _, s_ref = oracle.recur(inp)
    _, fs = run_gpu(inp)
    e1, e2 = s_err(out.cpu().numpy(), s_ref), s_err(out.cpu().numpy(), fs)
    _say("  apply vs recurrence %.3e   vs whole pass %.3e" % (e1, e2))
    assert e1 <= S_RTOL and e2 <= S_RTOL
    assert torch.equal(zero, S)


@pytest.mark.parametrize("kda", [False, True])
def test_summary_composes_two_segments(gdn, kda):
    """Sequence-parallel use: whole pass over tokens [0, t0), summary of
    [t0, T) applied to its final state, against the recurrence over [0, T)
    (t0 in the middle of a chunk)."""
    T, t0 = 300, 150
    inp = _mild(9 + kda, 1, T, 2, kda=kda)
    sl = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    seg = lambda a, b: gi.GdnInputs(**{**inp.__dict__, "T": b - a, "q": sl(inp.q, a, b), "k": sl(inp.k, a, b),
                                       "v": sl(inp.v, a, b), "g": sl(inp.g, a, b), "beta": sl(inp.beta, a, b),
                                       "initial_state": None})
    _, s_a = run_gpu(seg(0, t0))
    M, S = _summary_gpu(gdn, seg(t0, T))
    out = gdn.state_summary_apply(M, S, torch.from_numpy(np.ascontiguousarray(s_a, dtype=np.float32)).cuda())
    torch.cuda.synchronize()
    _, s_ref = oracle.recur(inp)
    e = s_err(out.cpu().numpy(), s_ref)
    _say("  two-segment composition rel err %.3e" % e)
    assert e <= S_RTOL


@pytest.mark.parametrize("name", ["gdn", "varlen", "kda"])
def test_state_summary_gated(gdn, name):
    """gdn_state_summary_gated: the gate formed in the kernel from the raw
    values, against the oracle's summary on the oracle's gate."""
    import dataclasses
    from oracle import gate as ogate
    inp = {"gdn": lambda: gi.make_inputs("gdn", B=2, T=200, H=2),
           "varlen": lambda: gi.make_inputs("varlen", H=2, doc_lengths=[1, 64, 130]),
           "kda": lambda: gi.make_inputs("kda", B=1, T=150, H=2)}[name]()
    fn = ogate.kda_gate if inp.kda else ogate.gdn_gate
    ref_inp = dataclasses.replace(inp, g=fn(inp.gate_raw, inp.A_log, inp.dt_bias).astype(np.float32))
    M_ref, S_ref = oracle.state_summary(ref_inp)
    d = to_device(inp)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    M, S = gdn.state_summary(d["k"], d["v"], t(inp.gate_raw), d["beta"], q=d["q"], cu_seqlens=inp.cu_seqlens,
                             kda=inp.kda, l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2),
                             A_log=t(inp.A_log), dt_bias=t(inp.dt_bias))
    torch.cuda.synchronize()
    M, S = M.cpu().numpy(), S.cpu().numpy()
    em = float(np.abs(M - M_ref).max() / max(np.abs(M_ref).max(), 0.1))
    es = s_err(S, S_ref)
    _say("  gated summary %s: transition err %.3e   state rel err %.3e" % (name, em, es))
    assert em <= S_RTOL and es <= S_RTOL
