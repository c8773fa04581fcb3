"""GPU parity of the GDN backward pass (gdn_chunk_bwd, through the C ABI)
against the fp64 gradient oracle (``oracle.grad``), element by element.

Bar, per gradient tensor X in (dq, dk, dv, dg, dbeta, d_initial_state):
max |X - X_ref| <= G_RTOL * max |X_ref|. The kernels compute in fp32
throughout, but they reuse the forward's operands: the intra-chunk output
matrix Aqk is stored in bf16 (relative rounding 2^-9) and T as a bf16 hi + lo
pair (about 2^-16), so a gradient carries errors of a few 1e-3 of its scale;
the bar is 1e-2 of the largest element.
"""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
from oracle import grad as og
from gpu_util import to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

G_RTOL = 1e-2
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "ds0")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_gated_delta_03_amd as m
    return m


def _cotangents(inp, seed, with_dsf=True):
    rng = np.random.default_rng(seed)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32) if with_dsf else None
    return do_bits, dsf


def _run_bwd(gdn, inp, do_bits, dsf):
    d = to_device(inp)
    do = torch.from_numpy(np.ascontiguousarray(do_bits)).view(torch.bfloat16).cuda()
    dsf_t = None if dsf is None else torch.from_numpy(dsf).cuda()
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=dsf_t, cu_seqlens=inp.cu_seqlens,
                            l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2))
    torch.cuda.synchronize()
    return {n: t.cpu().numpy().astype(np.float64) for n, t in zip(NAMES, out)}


def _compare(got, ref, names=NAMES):
    errs = {}
    for n in names:
        r = ref[n]
        assert np.isfinite(got[n]).all(), n
        errs[n] = float(np.abs(got[n] - r).max() / max(np.abs(r).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % (n, e) for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= G_RTOL, (n, e)


def _reset_problem():
    rng = np.random.default_rng(41)
    inp = gi.random_problem(rng, 1, 150, 2, 128, 128, gate_scale=0.3, with_initial_state=True)
    g = inp.g.copy()
    g[0, 77, :] = -1000.0
    return gi.GdnInputs(**{**inp.__dict__, "g": g})


def _noflag_problem():
    """q, k L2-normalised on the host, beta in (0, 1), no in-kernel flags."""
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 140, 2, 128)).astype(np.float32)
    k = rng.standard_normal((1, 140, 2, 128)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((1, 140, 2))))).astype(np.float32)
    base = gi.random_problem(rng, 1, 140, 2, 128, 128, gate_scale=0.3, with_initial_state=True,
                             flags=gi.FLAG_OUTPUT_FINAL_STATE)
    return gi.GdnInputs(**{**base.__dict__, "q": gi.f32_to_bf16_bits(q), "k": gi.f32_to_bf16_bits(k),
                           "beta": gi.f32_to_bf16_bits(beta)})


CASES = [
    ("B2_T150_H2", lambda: gi.random_problem(np.random.default_rng(31), 2, 150, 2, 128, 128, gate_scale=0.3,
                                             with_initial_state=True), True),
    ("packed_docs", lambda: gi.random_problem(np.random.default_rng(32), 1, 277, 2, 128, 128, gate_scale=0.3,
                                              with_initial_state=True,
                                              cu_seqlens=np.array([0, 1, 18, 82, 147, 277])), True),
    ("T1", lambda: gi.random_problem(np.random.default_rng(33), 2, 1, 2, 128, 128, with_initial_state=True), True),
    ("T64_exact_chunk", lambda: gi.random_problem(np.random.default_rng(34), 1, 64, 3, 128, 128, gate_scale=0.3),
     True),
    ("workload_gates_no_dsf", lambda: gi.make_inputs("gdn", B=1, T=200, H=2), False),
    ("reset_at_77", _reset_problem, True),
    ("host_normalised_no_flags", _noflag_problem, True),
    ("l2norm_only", lambda: gi.random_problem(np.random.default_rng(35), 1, 100, 2, 128, 128, gate_scale=0.3,
                                              with_initial_state=True,
                                              flags=gi.FLAG_L2NORM_QK | gi.FLAG_OUTPUT_FINAL_STATE), True),
    ("long_T2048_H2", lambda: gi.make_inputs("long", T=2048, H=2), True),
]


@pytest.mark.parametrize("name,make,with_dsf", CASES, ids=[c[0] for c in CASES])
def test_gdn_bwd_parity(gdn, name, make, with_dsf):
    inp = make()
    _say("bwd case", name, "B,T,H =", inp.B, inp.T, inp.H, "flags", inp.flags,
         "docs", None if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1)
    do_bits, dsf = _cotangents(inp, 7, with_dsf)
    got = _run_bwd(gdn, inp, do_bits, dsf)
    ref = og.grads(inp, gi.bf16_bits_to_f32(do_bits).astype(np.float64),
                   None if dsf is None else dsf.astype(np.float64))
    _compare(got, ref)


def test_gdn_bwd_full_size_sampled(gdn):
    """The benchmark shape (B=4, T=4096, H=16, workload gates and flags): the
    whole backward on the GPU, then one (batch row, head) pair against the
    oracle run on that slice alone (heads and rows are independent)."""
    inp = gi.make_inputs("gdn")
    _say("bwd full size B,T,H =", inp.B, inp.T, inp.H)
    do_bits, dsf = _cotangents(inp, 8)
    got = _run_bwd(gdn, inp, do_bits, dsf)
    for b, h in ((3, 14),):
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        one = gi.GdnInputs(**{**inp.__dict__, "B": 1, "H": 1, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v),
                              "g": sl(inp.g), "beta": sl(inp.beta), "initial_state": None})
        ref = og.grads(one, gi.bf16_bits_to_f32(sl(do_bits)).astype(np.float64),
                       dsf[b:b + 1, h:h + 1].astype(np.float64))
        sub = {n: (got[n][b:b + 1, h:h + 1] if n == "ds0" else got[n][b:b + 1, :, h:h + 1]) for n in NAMES}
        _say("  slice b=%d h=%d" % (b, h))
        _compare(sub, ref)


def test_gdn_bwd_sigmoid_only(gdn):
    """beta through the in-kernel sigmoid, q and k normalised on the host."""
    base = _noflag_problem()
    rng = np.random.default_rng(44)
    logits = gi.f32_to_bf16_bits(rng.standard_normal((base.B, base.T, base.H)).astype(np.float32))
    inp = gi.GdnInputs(**{**base.__dict__, "beta": logits,
                          "flags": gi.FLAG_BETA_SIGMOID | gi.FLAG_OUTPUT_FINAL_STATE})
    do_bits, dsf = _cotangents(inp, 9)
    got = _run_bwd(gdn, inp, do_bits, dsf)
    ref = og.grads(inp, gi.bf16_bits_to_f32(do_bits).astype(np.float64), dsf.astype(np.float64))
    _compare(got, ref)


def test_gdn_bwd_packed_full_size_sampled(gdn):
    """The packed workload (T=32768, H=16, documents of 17..8192 tokens, initial
    states): the whole backward on the GPU, then the shortest document and one
    head against the oracle run on that slice alone."""
    inp = gi.make_inputs("varlen")
    cu = [int(x) for x in inp.cu_seqlens]
    n = int(np.argmin(np.diff(cu)))
    a, e, h = cu[n], cu[n + 1], 5
    _say("bwd packed full size: %d documents, checking document %d (%d tokens), head %d" % (len(cu) - 1, n, e - a, h))
    do_bits, dsf = _cotangents(inp, 10)
    got = _run_bwd(gdn, inp, do_bits, dsf)
    sl = lambda x: np.ascontiguousarray(x[:, a:e, h:h + 1])
    one = gi.GdnInputs(**{**inp.__dict__, "T": e - a, "H": 1, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v),
                          "g": sl(inp.g), "beta": sl(inp.beta), "cu_seqlens": None,
                          "initial_state": np.ascontiguousarray(inp.initial_state[n:n + 1, h:h + 1])})
    ref = og.grads(one, gi.bf16_bits_to_f32(sl(do_bits)).astype(np.float64),
                   dsf[n:n + 1, h:h + 1].astype(np.float64))
    sub = {k: (got[k][n:n + 1, h:h + 1] if k == "ds0" else got[k][:, a:e, h:h + 1]) for k in NAMES}
    _compare(sub, ref)


def test_gdn_bwd_deterministic_with_caller_workspace(gdn):
    """No atomics: two calls, the second with a caller-provided workspace,
    give bitwise-equal gradients."""
    inp = gi.random_problem(np.random.default_rng(36), 1, 300, 3, 128, 128, gate_scale=0.3,
                            with_initial_state=True, cu_seqlens=np.array([0, 10, 300]))
    do_bits, dsf = _cotangents(inp, 11)
    first = _run_bwd(gdn, inp, do_bits, dsf)
    need = gdn.lib.gdn_chunk_bwd_workspace_bytes(1, 300, 3, 128, 128, 2,
                                                 np.ascontiguousarray(inp.cu_seqlens, dtype=np.int32)
                                                 .ctypes.data_as(__import__("ctypes").c_void_p), 3)
    ws = torch.empty(int(need), dtype=torch.uint8, device="cuda")
    d = to_device(inp)
    do = torch.from_numpy(np.ascontiguousarray(do_bits)).view(torch.bfloat16).cuda()
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do, scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=torch.from_numpy(dsf).cuda(),
                            cu_seqlens=inp.cu_seqlens, l2norm_qk=True, beta_sigmoid=True, workspace=ws)
    torch.cuda.synchronize()
    for name, t in zip(NAMES, out):
        assert np.array_equal(t.cpu().numpy().astype(np.float64), first[name]), name


# ---------------------------------------------------------------------------
# Backward of the in-kernel gate (gdn_chunk_bwd_gated): the oracle's gradient
# w.r.t. the gate, chained through the gate by oracle.grad.gate_grads.
# ---------------------------------------------------------------------------
def _gated_cases():
    import dataclasses
    big = gi.make_inputs("gdn", B=1, T=5000, H=2)   # three token blocks of the gate reduction, ragged
    docs = gi.make_inputs("varlen", H=2, doc_lengths=[1, 17, 64, 65, 130])
    docs = dataclasses.replace(docs, gate_raw=(np.random.default_rng(5).standard_normal((1, docs.T, 2))
                                               .astype(np.float32)),
                               A_log=np.array([0.3, 2.0], np.float32), dt_bias=np.array([0.05, -0.1], np.float32))
    return [("gdn_B2_T300_H3", gi.make_inputs("gdn", B=2, T=300, H=3)), ("gdn_T5000_H2", big),
            ("varlen_docs", docs)]


GATED = _gated_cases()


def _run_bwd_gated(gdn, inp, do_bits, dsf):
    d = to_device(inp)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    do = torch.from_numpy(np.ascontiguousarray(do_bits)).view(torch.bfloat16).cuda()
    dsf_t = None if dsf is None else torch.from_numpy(dsf).cuda()
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], t(inp.gate_raw), d["beta"], do, scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=dsf_t, cu_seqlens=inp.cu_seqlens,
                            l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2),
                            A_log=t(inp.A_log), dt_bias=t(inp.dt_bias))
    torch.cuda.synchronize()
    return {n: x.cpu().numpy().astype(np.float64) for n, x in zip(NAMES + ("da_log", "ddt_bias"), out)}


@pytest.mark.parametrize("name,inp", GATED, ids=[c[0] for c in GATED])
def test_gdn_bwd_gated_parity(gdn, name, inp):
    import dataclasses
    from oracle import gate as ogate
    _say("gated bwd case", name, "B,T,H =", inp.B, inp.T, inp.H)
    do_bits, dsf = _cotangents(inp, 9)
    got = _run_bwd_gated(gdn, inp, do_bits, dsf)
    g64 = ogate.gdn_gate(inp.gate_raw, inp.A_log, inp.dt_bias)
    ref = og.grads(dataclasses.replace(inp, g=g64), gi.bf16_bits_to_f32(do_bits).astype(np.float64),
                   dsf.astype(np.float64))
    gg = og.gate_grads(False, inp.gate_raw, inp.A_log, inp.dt_bias, ref["dg"])
    ref = {**ref, "dg": gg["dx"], "da_log": gg["da_log"], "ddt_bias": gg["ddt_bias"]}
    _compare(got, ref, NAMES + ("da_log", "ddt_bias"))
    again = _run_bwd_gated(gdn, inp, do_bits, dsf)
    for n in ("dg", "da_log", "ddt_bias"):
        assert np.array_equal(again[n], got[n]), n
