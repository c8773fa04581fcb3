"""GPU parity of the KDA backward's reverse state pass (kda_bwd_state_pass,
through the C ABI) against the chunk-form reverse pass oracle
(``oracle.grad_chunk``): per chunk the gradient w.r.t. the state leaving it and
w.r.t. v_new, and the initial-state gradient. Bar: max |X - X_ref| <= 1e-2 *
max |X_ref| per tensor (fp32 arithmetic on the prepare kernel's bf16 T hi + lo
and bf16 Aqk)."""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
from gpu_util import to_device
from oracle import grad_chunk as gc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL = 1e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_gated_delta_03_amd as m
    return m


def _cases():
    rng = np.random.default_rng(211)
    return [
        ("kda_B2_T150_H2", gi.make_inputs("kda", B=2, T=150, H=2)),
        ("kda_T64", gi.make_inputs("kda", B=1, T=64, H=3)),
        ("kda_T1", gi.make_inputs("kda", B=2, T=1, H=2)),
        ("kda_mild_B1_T300_H2", gi.random_problem(rng, 1, 300, 2, 128, 128, kda=True, gate_scale=0.05)),
        ("kda_packed", gi.random_problem(rng, 1, 277, 2, 128, 128, kda=True, gate_scale=0.3,
                                         cu_seqlens=np.array([0, 1, 18, 82, 147, 277]))),
    ]


CASES = _cases()


@pytest.mark.parametrize("name,inp", CASES, ids=[c[0] for c in CASES])
def test_kda_reverse_state_pass(gdn, name, inp):
    _say("kda reverse pass", name, inp.B, inp.T, inp.H, "docs",
         None if inp.cu_seqlens is None else list(np.diff(inp.cu_seqlens)))
    rng = np.random.default_rng(5)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    d = to_device(inp)
    dh, dvn, ds0 = gdn.kda_bwd_state_pass(d["q"], d["k"], d["g"], d["beta"],
                                          torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                                          d_final_state=torch.from_numpy(dsf).cuda(), cu_seqlens=inp.cu_seqlens,
                                          l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2))
    torch.cuda.synchronize()
    dh, dvn, ds0 = (x.cpu().numpy().astype(np.float64) for x in (dh, dvn, ds0))
    ref = gc.grads_chunk(inp, gi.bf16_bits_to_f32(do_bits).astype(np.float64), dsf.astype(np.float64))
    # the chunk table: sequences in order, chunks of each in order
    lens = [inp.T] * inp.B if inp.cu_seqlens is None else list(np.diff(inp.cu_seqlens))
    ref_dh = np.zeros_like(dh)
    ref_dvn = np.zeros_like(dvn)
    c = 0
    for n, ln in enumerate(lens):
        nch = (int(ln) + 63) // 64
        for j in range(nch):
            ref_dh[:, c] = ref["dh"][n][j + 1] if j + 1 < nch else dsf[n]
            ref_dvn[:, c] = ref["dvn"][n][j]
            c += 1
    assert c == dh.shape[1]
    errs = {}
    for key, got, r in (("dh_next", dh, ref_dh), ("dv_new", dvn, ref_dvn), ("ds0", ds0, ref["ds0"])):
        assert np.isfinite(got).all(), key
        errs[key] = float(np.abs(got - r).max() / max(np.abs(r).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for key, e in errs.items():
        assert e <= RTOL, (key, e)


def test_kda_reverse_state_pass_full_size_sampled(gdn):
    """The benchmark shape (B=2, T=8192, H=32, 128 chunks per sequence): the
    whole pass on the GPU, then one (sequence, head) against the oracle run on
    that slice alone (heads and sequences are independent)."""
    inp = gi.make_inputs("kda")
    _say("kda reverse pass full size B,T,H =", inp.B, inp.T, inp.H)
    rng = np.random.default_rng(6)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    d = to_device(inp)
    dh, dvn, ds0 = gdn.kda_bwd_state_pass(d["q"], d["k"], d["g"], d["beta"],
                                          torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                                          d_final_state=torch.from_numpy(dsf).cuda(), l2norm_qk=True,
                                          beta_sigmoid=True)
    torch.cuda.synchronize()
    b, h = 1, 29
    nch = inp.T // 64
    sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
    one = gi.GdnInputs(**{**inp.__dict__, "B": 1, "H": 1, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v),
                          "g": sl(inp.g), "beta": sl(inp.beta), "initial_state": None})
    ref = gc.grads_chunk(one, gi.bf16_bits_to_f32(sl(do_bits)).astype(np.float64),
                         dsf[b:b + 1, h:h + 1].astype(np.float64))
    got_dh = dh[h, b * nch:(b + 1) * nch].cpu().numpy().astype(np.float64)
    ref_dh = np.concatenate([ref["dh"][0][1:, 0], dsf[b:b + 1, h]], 0)
    got_dv = dvn[h, b * nch:(b + 1) * nch].cpu().numpy().astype(np.float64)
    errs = {"dh_next": float(np.abs(got_dh - ref_dh).max() / np.abs(ref_dh).max()),
            "dv_new": float(np.abs(got_dv - ref["dvn"][0][:, 0]).max() / np.abs(ref["dvn"][0]).max()),
            "ds0": float(np.abs(ds0[b, h].cpu().numpy() - ref["ds0"][0, 0]).max() / np.abs(ref["ds0"]).max())}
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for key, e in errs.items():
        assert e <= RTOL, (key, e)


# ---------------------------------------------------------------------------
# Whole KDA backward (kda_chunk_bwd) against the fp64 autograd oracle.
# ---------------------------------------------------------------------------
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "ds0")


def _whole_cases():
    rng = np.random.default_rng(221)
    return [
        ("kda_B2_T150_H2", gi.make_inputs("kda", B=2, T=150, H=2)),
        # with an initial state: from a zero one the gate's gradient at T = 1 is exactly zero
        ("kda_T1_init", gi.random_problem(rng, 2, 1, 2, 128, 128, kda=True, with_initial_state=True)),
        ("kda_T64", gi.make_inputs("kda", B=1, T=64, H=3)),
        ("kda_mild_init", gi.random_problem(rng, 1, 200, 2, 128, 128, kda=True, gate_scale=0.05,
                                            with_initial_state=True)),
        ("kda_packed", gi.random_problem(rng, 1, 277, 2, 128, 128, kda=True, gate_scale=0.3, with_initial_state=True,
                                         cu_seqlens=np.array([0, 1, 18, 82, 147, 277]))),
        ("kda_l2norm_only", gi.random_problem(rng, 1, 100, 2, 128, 128, kda=True, gate_scale=0.3,
                                              with_initial_state=True,
                                              flags=gi.FLAG_L2NORM_QK | gi.FLAG_OUTPUT_FINAL_STATE)),
    ]


WHOLE = _whole_cases()


@pytest.mark.parametrize("name,inp", WHOLE, ids=[c[0] for c in WHOLE])
def test_kda_chunk_bwd_parity(gdn, name, inp):
    from oracle import grad as og
    _say("kda bwd", name, inp.B, inp.T, inp.H, "flags", inp.flags)
    rng = np.random.default_rng(8)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    d = to_device(inp)
    out = gdn.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=torch.from_numpy(dsf).cuda(),
                            cu_seqlens=inp.cu_seqlens, l2norm_qk=bool(inp.flags & 1),
                            beta_sigmoid=bool(inp.flags & 2))
    torch.cuda.synchronize()
    ref = og.grads(inp, gi.bf16_bits_to_f32(do_bits).astype(np.float64), dsf.astype(np.float64))
    errs = {}
    for key, t in zip(NAMES, out):
        x = t.cpu().numpy().astype(np.float64)
        assert np.isfinite(x).all(), key
        errs[key] = float(np.abs(x - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for key, e in errs.items():
        assert e <= RTOL, (key, e)


def test_kda_chunk_bwd_full_size_sampled(gdn):
    """The benchmark shape (B=2, T=8192, H=32): the whole backward on the GPU,
    then one (sequence, head) against the autograd oracle run on that slice."""
    from oracle import grad as og
    inp = gi.make_inputs("kda")
    _say("kda bwd full size B,T,H =", inp.B, inp.T, inp.H)
    rng = np.random.default_rng(9)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    d = to_device(inp)
    out = gdn.kda_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                            d_final_state=torch.from_numpy(dsf).cuda(), l2norm_qk=True, beta_sigmoid=True)
    torch.cuda.synchronize()
    b, h = 0, 17
    sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
    one = gi.GdnInputs(**{**inp.__dict__, "B": 1, "H": 1, "q": sl(inp.q), "k": sl(inp.k), "v": sl(inp.v),
                          "g": sl(inp.g), "beta": sl(inp.beta), "initial_state": None})
    ref = og.grads(one, gi.bf16_bits_to_f32(sl(do_bits)).astype(np.float64), dsf[b:b + 1, h:h + 1].astype(np.float64))
    errs = {}
    for key, t in zip(NAMES, out):
        x = t.cpu().numpy().astype(np.float64)
        x = x[b:b + 1, h:h + 1] if key == "ds0" else x[b:b + 1, :, h:h + 1]
        errs[key] = float(np.abs(x - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for key, e in errs.items():
        assert e <= RTOL, (key, e)


# ---------------------------------------------------------------------------
# Backward of the in-kernel KDA gate (kda_chunk_bwd_gated): the oracle's
# gradient w.r.t. the per-channel gate, chained through the gate by
# oracle.grad.gate_grads; the gate's sums are bitwise reproducible.
# ---------------------------------------------------------------------------
def _gated_cases():
    import dataclasses
    packed = gi.make_inputs("kda", B=1, T=277, H=2)
    packed = dataclasses.replace(packed, cu_seqlens=np.array([0, 1, 18, 82, 147, 277], np.int32))
    return [("kda_gated_B1_T600_H2", gi.make_inputs("kda", B=1, T=600, H=2)),  # three gate blocks, ragged
            ("kda_gated_B2_T150_H3", gi.make_inputs("kda", B=2, T=150, H=3)),
            ("kda_gated_packed", packed)]


GATED = _gated_cases()


def _run_kda_bwd_gated(gdn, inp, do_bits, dsf):
    d = to_device(inp)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    out = gdn.kda_chunk_bwd(d["q"], d["k"], d["v"], t(inp.gate_raw), d["beta"],
                            torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=torch.from_numpy(dsf).cuda(),
                            cu_seqlens=inp.cu_seqlens, l2norm_qk=bool(inp.flags & 1),
                            beta_sigmoid=bool(inp.flags & 2), A_log=t(inp.A_log), dt_bias=t(inp.dt_bias))
    torch.cuda.synchronize()
    return {n: x.cpu().numpy().astype(np.float64) for n, x in zip(NAMES + ("da_log", "ddt_bias"), out)}


@pytest.mark.parametrize("name,inp", GATED, ids=[c[0] for c in GATED])
def test_kda_chunk_bwd_gated_parity(gdn, name, inp):
    import dataclasses
    from oracle import gate as ogate
    from oracle import grad as og
    _say("kda gated bwd", name, inp.B, inp.T, inp.H, "seqs", inp.num_seqs)
    rng = np.random.default_rng(12)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    got = _run_kda_bwd_gated(gdn, inp, do_bits, dsf)
    g64 = ogate.kda_gate(inp.gate_raw, inp.A_log, inp.dt_bias)
    ref = og.grads(dataclasses.replace(inp, g=g64), gi.bf16_bits_to_f32(do_bits).astype(np.float64),
                   dsf.astype(np.float64))
    gg = og.gate_grads(True, inp.gate_raw, inp.A_log, inp.dt_bias, ref["dg"])
    ref = {**ref, "dg": gg["dx"], "da_log": gg["da_log"], "ddt_bias": gg["ddt_bias"]}
    errs = {}
    for key in NAMES + ("da_log", "ddt_bias"):
        x = got[key]
        assert np.isfinite(x).all(), key
        assert x.shape == ref[key].shape, (key, x.shape, ref[key].shape)
        errs[key] = float(np.abs(x - ref[key]).max() / max(np.abs(ref[key]).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for key, e in errs.items():
        assert e <= RTOL, (key, e)
    again = _run_kda_bwd_gated(gdn, inp, do_bits, dsf)
    for n in ("dg", "da_log", "ddt_bias"):
        assert np.array_equal(again[n], got[n]), n
