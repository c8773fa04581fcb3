"""Causal depthwise Conv1d + SiLU in fp64 numpy (TEST INFRASTRUCTURE ONLY).

The ShortConv that forms q, k, v from the projections on the hyper-parallel
"Diff Coverage" page of the 2026-09-10 gate build (``_causal_conv1d_with_cp_halo``):
a depthwise ``F.conv1d`` (cross-correlation, one filter per channel, kernel
W, dilation d) over the sequence left-padded with (W-1) d rows -- zeros, or
the preceding rank's last rows (the halo) -- keeping the first T outputs,
then ``F.silu``. Per channel c and token t:

    y[t, c] = silu(bias[c] + sum_{j<W} w[c, j] x[t - (W-1-j) d, c])

with rows before the start of the sequence taken from the halo or zero. For
packed input each document is its own sequence; a halo precedes the first
document only. Pinned by tests/test_conv_pins.py.
"""
from __future__ import annotations

import numpy as np

from .chunk import decode_bf16


def short_conv(inp) -> np.ndarray:
    """fp64 [B,T,D] output of :class:`gdn_inputs.ConvInputs`."""
    x = decode_bf16(inp.x)
    w = np.asarray(inp.weight, dtype=np.float64)
    b = None if inp.bias is None else np.asarray(inp.bias, dtype=np.float64)
    halo = None if inp.halo is None else decode_bf16(inp.halo)
    W, d = inp.W, inp.dilation
    hw = (W - 1) * d
    y = np.zeros(x.shape)

    def one(seq, pre):
        """seq [t, D]; pre [hw, D] rows before it."""
        xp = np.concatenate([pre, seq], axis=0)
        out = np.zeros(seq.shape)
        for j in range(W):
            out += w[:, j] * xp[j * d: j * d + seq.shape[0]]
        if b is not None:
            out += b
        if inp.silu:
            out = out / (1.0 + np.exp(-out))
        return out

    for bi in range(inp.B):
        if inp.cu_seqlens is None:
            pre = halo[bi] if halo is not None else np.zeros((hw, x.shape[2]))
            y[bi] = one(x[bi], pre)
        else:
            cu = [int(v) for v in inp.cu_seqlens]
            for n in range(len(cu) - 1):
                pre = halo[bi] if (halo is not None and n == 0) else np.zeros((hw, x.shape[2]))
                y[bi, cu[n]:cu[n + 1]] = one(x[bi, cu[n]:cu[n + 1]], pre)
    return y
