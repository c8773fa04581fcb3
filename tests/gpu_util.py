"""Helpers for the GPU parity tests: move a gdn_inputs problem to the device,
run the HIP path through the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import gdn_inputs as gi

# Bars of the method's accuracy statement: max-abs error on o, relative
# (to max |S_ref|) max error on the fp32 final state.
O_ATOL = 2e-2
S_RTOL = 1e-3


def to_device(inp: gi.GdnInputs, device="cuda"):
    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(device)
    d = dict(q=bf(inp.q), k=bf(inp.k), v=bf(inp.v), beta=bf(inp.beta),
             g=torch.from_numpy(np.ascontiguousarray(inp.g)).to(device))
    d["initial_state"] = None if inp.initial_state is None else torch.from_numpy(inp.initial_state).to(device)
    return d


def run_gpu(inp: gi.GdnInputs, device="cuda", workspace=None):
    import chunked_gated_delta_03_amd as m
    d = to_device(inp, device)
    fn = m.kda_chunk_fwd if inp.kda else m.gdn_chunk_fwd
    o, fs = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale, initial_state=d["initial_state"],
               cu_seqlens=inp.cu_seqlens, l2norm_qk=bool(inp.flags & 1), beta_sigmoid=bool(inp.flags & 2),
               output_final_state=bool(inp.flags & 4), workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), None if fs is None else fs.cpu().numpy().astype(np.float64)


def o_err(o_gpu, o_ref):
    return float(np.abs(o_gpu - o_ref).max())


def s_err(s_gpu, s_ref):
    return float(np.abs(s_gpu - s_ref).max() / max(np.abs(s_ref).max(), 1e-30))


def check_all_units(o, fs, o_ref, s_ref, say=print):
    """Every element of o (max-abs <= O_ATOL) and the final state of every
    (sequence, head) unit (max |S - S_ref| / max |S_ref| of the unit <=
    S_RTOL, which implies the whole-tensor bar). Returns (o error, worst unit
    relative state error)."""
    N, H = fs.shape[:2]
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    eo = o_err(o, o_ref)
    diff = np.abs(fs - s_ref).reshape(N, H, -1).max(-1)
    ref = np.maximum(np.abs(s_ref).reshape(N, H, -1).max(-1), 1e-30)
    rel = diff / ref
    worst = np.unravel_index(int(np.argmax(rel)), rel.shape)
    say("  all %d x %d units: o max-abs err %.3e; final state: worst unit %s rel err %.3e, whole tensor %.3e"
        % (N, H, eo, tuple(int(x) for x in worst), float(rel.max()), s_err(fs, s_ref)))
    assert eo <= O_ATOL
    assert float(rel.max()) <= S_RTOL
    return eo, float(rel.max())


def hm_chunks(arr_list, dense: bool):
    """Oracle per-batch/per-document [B,H,NC,...] intermediates -> GPU layout [H,NT,...]."""
    parts = []
    for a in arr_list:
        B, H, NC = a.shape[:3]
        parts.append(np.moveaxis(a, 1, 0).reshape(H, B * NC, *a.shape[3:]))
    return np.concatenate(parts, axis=1)


# Column order of the stage outputs tmat and aqk: column 32s + 16h + 4g + e is
# stored at position 32s + 8g + 4h + e (the layout the stage entry documents).
_POS = np.arange(64)
_COL_AT_POS = (_POS & ~31) | ((_POS & 4) << 2) | ((_POS & 24) >> 1) | (_POS & 3)


def unpermute_cols(x):
    out = np.empty_like(x)
    out[..., _COL_AT_POS] = x
    return out


def decode_tmat(tmat):
    """Stage tmat (bf16 [H,NT,64,128], hi | lo, permuted) -> fp64 T [H,NT,64,64]."""
    t = tmat.float().cpu().numpy().astype(np.float64)
    return unpermute_cols(t[..., :64]) + unpermute_cols(t[..., 64:])


def decode_aqk(aqk):
    """Stage aqk (bf16 [H,NT,64,64], permuted columns) -> fp64 [H,NT,64,64]."""
    return unpermute_cols(aqk.float().cpu().numpy().astype(np.float64))
