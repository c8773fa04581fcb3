"""GPU parity of the forward entries with the gate formed in the kernel
(gdn_chunk_fwd_gated, kda_chunk_fwd_gated) against the oracle.

The expected result is the token recurrence (``oracle.recur``) run on the
gate of ``oracle.gate`` (fp64, then stored as the fp32 gate the recurrence
takes), so the kernel's fp32 softplus is checked through the whole pass at
the method's bars: max |o - o_ref| <= 2e-2, max |S - S_ref| / max |S_ref|
<= 1e-3.
"""
import dataclasses
import sys

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import O_ATOL, S_RTOL, check_all_units, o_err, run_gpu, s_err, to_device
from oracle import gate as ogate

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


def _oracle_gate(inp):
    fn = ogate.kda_gate if inp.kda else ogate.gdn_gate
    return fn(inp.gate_raw, inp.A_log, inp.dt_bias).astype(np.float32)


def _run_gated(gdn, inp):
    d = to_device(inp)
    dev = d["q"].device
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    fn = gdn.kda_chunk_fwd_gated if inp.kda else gdn.gdn_chunk_fwd_gated
    o, fs = fn(d["q"], d["k"], d["v"], t(inp.gate_raw), t(inp.A_log), t(inp.dt_bias), d["beta"], scale=inp.scale,
               initial_state=d["initial_state"], cu_seqlens=inp.cu_seqlens, l2norm_qk=bool(inp.flags & 1),
               beta_sigmoid=bool(inp.flags & 2), output_final_state=bool(inp.flags & 4))
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def _with_raw(inp, raw):
    return dataclasses.replace(inp, gate_raw=np.ascontiguousarray(raw, dtype=np.float32))


def _problems():
    gdn_small = gi.make_inputs("gdn", B=2, T=300, H=3)
    kda_small = gi.make_inputs("kda", B=1, T=200, H=4)
    rng = np.random.default_rng(91)
    # raw values far out on both sides of softplus (its linear branch and the
    # branch where 1 + e^-|y| rounds to 1), and next to -dt_bias (softplus(0))
    wide = gdn_small.gate_raw * np.float32(12.0)
    near0 = -np.broadcast_to(gdn_small.dt_bias, gdn_small.gate_raw.shape) + \
        rng.standard_normal(gdn_small.gate_raw.shape).astype(np.float32) * np.float32(1e-3)
    kda_wide = kda_small.gate_raw * np.float32(12.0)
    return [
        ("gdn_B2_T300_H3", gdn_small),
        ("gdn_T1", gi.make_inputs("gdn", B=3, T=1, H=2)),
        ("gdn_T65", gi.make_inputs("gdn", B=1, T=65, H=2)),
        ("gdn_wide_raw", _with_raw(gdn_small, wide)),
        ("gdn_raw_near_minus_bias", _with_raw(gdn_small, near0)),
        ("varlen_docs", gi.make_inputs("varlen", H=3, doc_lengths=[1, 17, 63, 64, 65, 130, 200])),
        ("wide_B4_T200_H16", gi.make_inputs("gdn", B=4, T=200, H=16)),
        ("kda_B1_T200_H4", kda_small),
        ("kda_wide_raw", _with_raw(kda_small, kda_wide)),
        ("kda_varlen", dataclasses.replace(
            gi.make_inputs("kda", B=1, T=150, H=2),
            cu_seqlens=np.array([0, 1, 64, 150], dtype=np.int32))),
    ]


PROBLEMS = _problems()


@pytest.mark.parametrize("name,inp", PROBLEMS, ids=[p[0] for p in PROBLEMS])
def test_gated_matches_recurrence(gdn, name, inp):
    _say("gated parity", name, inp.B, inp.T, inp.H, "kda" if inp.kda else "gdn")
    ref_inp = dataclasses.replace(inp, g=_oracle_gate(inp))
    o_ref, s_ref = oracle.recur(ref_inp)
    o, fs = _run_gated(gdn, inp)
    eo, es = o_err(o, o_ref), s_err(fs, s_ref)
    _say("  o err %.3e  S rel err %.3e" % (eo, es))
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    assert eo <= O_ATOL and es <= S_RTOL


@pytest.mark.parametrize("name,inp", PROBLEMS[:2] + PROBLEMS[7:8], ids=["gdn_B2_T300_H3", "gdn_T1", "kda_B1_T200_H4"])
def test_gated_equals_plain_entry_with_oracle_gate(gdn, name, inp):
    """The gated entry and the plain entry given the oracle's gate differ only
    by the fp32 rounding of the gate: both are held to the bars against each
    other's common reference, and to a tight bound against each other."""
    ref_inp = dataclasses.replace(inp, g=_oracle_gate(inp))
    o_p, s_p = run_gpu(ref_inp)
    o_g, s_g = _run_gated(gdn, inp)
    _say("  gated vs plain: o %.3e  S %.3e" % (o_err(o_g, o_p), s_err(s_g, s_p)))
    assert o_err(o_g, o_p) <= 2e-3 and s_err(s_g, s_p) <= 1e-4


@pytest.mark.parametrize("name", ["gdn", "kda"])
def test_full_size_gated(gdn, name):
    """The benchmark shapes (GDN B=4 T=4096 H=16; KDA B=2 T=8192 H=32) with the
    gate formed in the kernel: every output and every final state."""
    inp = gi.make_inputs(name)
    _say("full-size gated", name)
    o, fs = _run_gated(gdn, inp)
    o_ref, s_ref = oracle.recur(dataclasses.replace(inp, g=_oracle_gate(inp)))
    check_all_units(o, fs, o_ref, s_ref, _say)
