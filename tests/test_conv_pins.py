"""Pins of the ShortConv oracle (``oracle.short_conv``) against facts fixed by
the definition of a causal depthwise cross-correlation, not by itself."""
import numpy as np
import pytest

import gdn_inputs as gi
import oracle


def _with(inp, **kw):
    return gi.ConvInputs(**{**inp.__dict__, **kw})


def _silu(z):
    return z / (1.0 + np.exp(-z))


def test_kernel_one_is_elementwise():
    """W = 1: y = silu(w x + b) per channel (no time mixing)."""
    inp = gi.make_conv_inputs(2, 30, 8, W=1, bias=True, seed=1)
    x = oracle.decode_bf16(inp.x)
    ref = _silu(x * inp.weight[:, 0].astype(np.float64) + inp.bias.astype(np.float64))
    assert np.abs(oracle.short_conv(inp) - ref).max() < 1e-12


@pytest.mark.parametrize("W,dil", [(4, 1), (3, 2)])
def test_impulse_response_gives_taps_in_order(W, dil):
    """A unit impulse at token t0 of channel c: without the activation, the
    output at t0 + m d is w[c, W-1-m] (tap order, causality, dilation) and zero
    elsewhere, including before t0."""
    inp = gi.make_conv_inputs(1, 40, 4, W=W, dilation=dil, silu=False, seed=2)
    xf = np.zeros((1, 40, 4), dtype=np.float32)
    t0 = 11
    xf[0, t0, 2] = 1.0
    y = oracle.short_conv(_with(inp, x=gi.f32_to_bf16_bits(xf)))
    expect = np.zeros((1, 40, 4))
    for m in range(W):
        expect[0, t0 + m * dil, 2] = inp.weight[2, W - 1 - m]
    assert np.abs(y - expect).max() < 1e-15


def test_equals_numpy_convolve():
    """Per channel, the causal output is np.convolve (a true convolution, so
    the reversed taps) truncated to the first T samples."""
    inp = gi.make_conv_inputs(2, 57, 6, W=4, silu=False, seed=3)
    x = oracle.decode_bf16(inp.x)
    y = oracle.short_conv(inp)
    for b in range(2):
        for c in range(6):
            ref = np.convolve(x[b, :, c], inp.weight[c, ::-1].astype(np.float64))[:57]
            assert np.abs(y[b, :, c] - ref).max() < 1e-12


def test_packed_equals_per_document_dense():
    """Packed: each document is filtered on its own (no leakage across the
    boundary), the halo precedes the first document only."""
    lens = [1, 3, 17, 40]
    inp = gi.make_conv_inputs(1, 0, 8, W=4, bias=True, halo=True, seed=4, doc_lengths=lens)
    y = oracle.short_conv(inp)
    cu = inp.cu_seqlens
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        one = _with(inp, T=b - a, x=np.ascontiguousarray(inp.x[:, a:b]), cu_seqlens=None,
                    halo=inp.halo if n == 0 else None)
        assert np.abs(y[:, a:b] - oracle.short_conv(one)).max() < 1e-15


def test_halo_continues_the_previous_segment():
    """Running on tokens [t0, T) with the last (W-1) d rows before t0 as the
    halo equals the tail of the run over [0, T) (the sequence-parallel split)."""
    inp = gi.make_conv_inputs(2, 60, 8, W=4, dilation=2, bias=True, seed=5)
    y = oracle.short_conv(inp)
    t0, hw = 25, 6
    tail = _with(inp, T=60 - t0, x=np.ascontiguousarray(inp.x[:, t0:]),
                 halo=np.ascontiguousarray(inp.x[:, t0 - hw:t0]))
    assert np.abs(oracle.short_conv(tail) - y[:, t0:]).max() < 1e-15
