"""GPU parity of the causal depthwise Conv1d + SiLU (gdn_short_conv, through
the C ABI) against ``oracle.short_conv`` (fp64), element by element:
|y - y_ref| <= 2^-8 |y_ref| + 1e-5 (the output is bf16, rounded to nearest:
at most 2^-9 relative, the rest is fp32 accumulation)."""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RTOL = 2.0 ** -8
ATOL = 1e-5


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunked_gated_delta_03_amd as m
    return m


def _run(gdn, inp):
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).cuda()
    x = bf(inp.x)
    w = torch.from_numpy(inp.weight).cuda()
    b = None if inp.bias is None else torch.from_numpy(inp.bias).cuda()
    h = None if inp.halo is None else bf(inp.halo)
    y = gdn.short_conv(x, w, bias=b, halo=h, cu_seqlens=inp.cu_seqlens, dilation=inp.dilation, silu=inp.silu)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


CASES = [
    ("B2_T100_D64_W4", dict(B=2, T=100, D=64, W=4)),
    ("bias_halo", dict(B=2, T=77, D=64, W=4, bias=True, halo=True)),
    ("no_silu", dict(B=1, T=50, D=32, W=4, silu=False, bias=True)),
    ("W1", dict(B=1, T=40, D=16, W=1, bias=True)),
    ("W2", dict(B=1, T=40, D=16, W=2)),
    ("W3_dil2_halo", dict(B=2, T=45, D=24, W=3, dilation=2, halo=True)),
    ("W5_dil3", dict(B=1, T=70, D=16, W=5, dilation=3, bias=True)),
    ("W8", dict(B=1, T=70, D=16, W=8, halo=True)),
    ("T1", dict(B=3, T=1, D=64, W=4, halo=True)),
    ("packed_docs_halo", dict(B=1, T=0, D=64, W=4, bias=True, halo=True, doc_lengths=[1, 3, 17, 40, 64, 100])),
    ("packed_one_token_docs", dict(B=1, T=0, D=16, W=4, doc_lengths=[1, 1, 1, 2, 1])),
    ("wide_D6144_T257", dict(B=1, T=257, D=6144, W=4)),
]


@pytest.mark.parametrize("name,kw", CASES, ids=[n for n, _ in CASES])
def test_short_conv_parity(gdn, name, kw):
    inp = gi.make_conv_inputs(seed=sum(map(ord, name)), **kw)
    _say("conv case", name, "B,T,D,W,dil =", inp.B, inp.T, inp.D, inp.W, inp.dilation)
    y = _run(gdn, inp)
    ref = oracle.short_conv(inp)
    bad = np.abs(y - ref) > RTOL * np.abs(ref) + ATOL
    _say("  max abs err %.3e, violations %d" % (np.abs(y - ref).max(), int(bad.sum())))
    assert not bad.any()


def test_short_conv_full_size(gdn):
    """The GDN layer shape of the benchmark workload: B=4, T=4096, D = 3 * 16 *
    128 = 6144 channels (q, k, v of 16 heads), W = 4; every element."""
    inp = gi.make_conv_inputs(4, 4096, 6144, W=4, seed=2001)
    _say("conv full size B=4 T=4096 D=6144 W=4")
    y = _run(gdn, inp)
    ref = oracle.short_conv(inp)
    bad = np.abs(y - ref) > RTOL * np.abs(ref) + ATOL
    _say("  max abs err %.3e, violations %d" % (np.abs(y - ref).max(), int(bad.sum())))
    assert not bad.any()


def test_short_conv_halo_continuation(gdn):
    """Two halves of a sequence, the second with the first's last rows as
    halo, equal the whole run (the sequence-parallel split of the page)."""
    inp = gi.make_conv_inputs(2, 200, 64, W=4, dilation=2, bias=True, seed=17)
    full = _run(gdn, inp)
    t0, hw = 90, 6
    tail = gi.ConvInputs(**{**inp.__dict__, "T": 200 - t0, "x": np.ascontiguousarray(inp.x[:, t0:]),
                            "halo": np.ascontiguousarray(inp.x[:, t0 - hw:t0])})
    assert np.array_equal(_run(gdn, tail), full[:, t0:])


def test_conv_feeds_gdn_forward(gdn):
    """The layer order of the pages: the mixed projections go through the
    ShortConv + SiLU, are split into q, k, v (16 heads each) and run through
    the GDN forward; against the conv oracle followed by the token recurrence
    on the same bf16 q, k, v."""
    B, T, H = 1, 300, 4
    D = 3 * H * 128
    cin = gi.make_conv_inputs(B, T, D, W=4, seed=23)
    y = _run(gdn, cin)                                   # fp64 view of the bf16 GPU output
    y_ref = oracle.short_conv(cin)
    assert not (np.abs(y - y_ref) > RTOL * np.abs(y_ref) + ATOL).any()
    bits = gi.f32_to_bf16_bits(y.astype(np.float32))     # exactly the GPU's bf16 values
    q, k, v = (np.ascontiguousarray(bits[:, :, i * H * 128:(i + 1) * H * 128]).reshape(B, T, H, 128)
               for i in range(3))
    base = gi.make_inputs("gdn", B=B, T=T, H=H)
    inp = gi.GdnInputs(**{**base.__dict__, "q": q, "k": k, "v": v})
    from gpu_util import O_ATOL, S_RTOL, o_err, run_gpu, s_err
    o, fs = run_gpu(inp)
    o_ref, s_ref = oracle.recur(inp)
    eo, es = o_err(o, o_ref), s_err(fs, s_ref)
    _say("  conv -> GDN: o err %.3e  S rel err %.3e" % (eo, es))
    assert eo <= O_ATOL and es <= S_RTOL
