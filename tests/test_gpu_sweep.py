"""Seeded randomized parity sweep over small problems (through the C ABI):
gate kind, dense or packed input, every flag subset, with and without an
initial state, sequence and document lengths across every chunk remainder.
Forward: o and the final state against the token recurrence at the method's
bars. Backward (GDN): every gradient against the autograd oracle at the
backward bar."""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import O_ATOL, S_RTOL, o_err, run_gpu, s_err, to_device

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


def _random_case(seed):
    rng = np.random.default_rng(seed)
    kda = bool(rng.integers(2))
    packed = bool(rng.integers(2))
    flags = int(rng.integers(8)) | gi.FLAG_OUTPUT_FINAL_STATE
    H = int(rng.integers(1, 5))
    gate_scale = float(rng.choice([0.01, 0.3, 1.0]))
    init = bool(rng.integers(2))
    if packed:
        n = int(rng.integers(1, 6))
        lens = rng.integers(1, 200, size=n)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        B, T = 1, int(cu[-1])
    else:
        cu = None
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 300))
    inp = gi.random_problem(rng, B, T, H, 128, 128, kda=kda, gate_scale=gate_scale, with_initial_state=init,
                            cu_seqlens=cu, flags=flags)
    if not flags & gi.FLAG_L2NORM_QK:
        # without the in-kernel norm, keep q, k at unit scale as the layer would
        for name in ("q", "k"):
            x = gi.bf16_bits_to_f32(getattr(inp, name)).astype(np.float64)
            x /= np.sqrt((x * x).sum(-1, keepdims=True)) + 1e-12
            setattr(inp, name, gi.f32_to_bf16_bits(x.astype(np.float32)))
    if not flags & gi.FLAG_BETA_SIGMOID:
        b = 1.0 / (1.0 + np.exp(-gi.bf16_bits_to_f32(inp.beta).astype(np.float64)))
        inp.beta = gi.f32_to_bf16_bits(b.astype(np.float32))
    return inp


SEEDS = list(range(5000, 5040))


@pytest.mark.parametrize("seed", SEEDS)
def test_forward_sweep(gdn, seed):
    inp = _random_case(seed)
    _say("sweep seed %d: %s B=%d T=%d H=%d flags=%d docs=%s init=%s" % (
        seed, "kda" if inp.kda else "gdn", inp.B, inp.T, inp.H, inp.flags,
        None if inp.cu_seqlens is None else list(np.diff(inp.cu_seqlens)), inp.initial_state is not None))
    o, fs = run_gpu(inp)
    o_ref, s_ref = oracle.recur(inp)
    eo, es = o_err(o, o_ref), s_err(fs, s_ref)
    _say("  o err %.3e  S rel err %.3e" % (eo, es))
    assert eo <= O_ATOL and es <= S_RTOL


@pytest.mark.parametrize("seed", [6000, 6001, 6002, 6003, 6004, 6005])
def test_backward_sweep(gdn, seed):
    from oracle import grad as og
    inp = _random_case(seed)
    if inp.kda:  # the backward covers the GDN gate
        inp = gi.random_problem(np.random.default_rng(seed), 1, 150, 2, 128, 128, gate_scale=0.3,
                                with_initial_state=True)
    _say("bwd sweep seed %d: B=%d T=%d H=%d flags=%d docs=%s" % (
        seed, inp.B, inp.T, inp.H, inp.flags, None if inp.cu_seqlens is None else list(np.diff(inp.cu_seqlens))))
    rng = np.random.default_rng(seed + 1)
    do_bits = gi.f32_to_bf16_bits(rng.standard_normal((inp.B, inp.T, inp.H, inp.V), dtype=np.float32))
    dsf = (rng.standard_normal((inp.num_seqs, inp.H, inp.K, inp.V)) * 0.1).astype(np.float32)
    d = to_device(inp)
    out = gdn.gdn_chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            torch.from_numpy(do_bits).view(torch.bfloat16).cuda(), scale=inp.scale,
                            initial_state=d["initial_state"], d_final_state=torch.from_numpy(dsf).cuda(),
                            cu_seqlens=inp.cu_seqlens, l2norm_qk=bool(inp.flags & 1),
                            beta_sigmoid=bool(inp.flags & 2))
    torch.cuda.synchronize()
    ref = og.grads(inp, gi.bf16_bits_to_f32(do_bits).astype(np.float64), dsf.astype(np.float64))
    errs = {}
    for name, t in zip(("dq", "dk", "dv", "dg", "dbeta", "ds0"), out):
        x = t.cpu().numpy().astype(np.float64)
        errs[name] = float(np.abs(x - ref[name]).max() / max(np.abs(ref[name]).max(), 1e-30))
    _say("  " + "  ".join("%s %.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e <= 1e-2, (name, e)
