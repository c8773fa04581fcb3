"""gdn_chunk_fwd_noalloc (the entry that allocates nothing: intermediates in
the library's fixed device scratch) against gdn_chunk_fwd with a workspace,
through the C ABI: two no-allocation calls in a row, the second on a smaller
problem, each bit-identical to the workspace entry's result (same kernels, same
inputs) and within the accuracy bars of the fp64 recurrence."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from gpu_util import O_ATOL, S_RTOL, o_err, s_err, to_device

pytestmark = pytest.mark.gpu


def _problems():
    big = gi.make_inputs("gdn", B=2, T=1000, H=4)             # 2 x 16 chunks x 4 heads, ragged tail of 40 rows
    small = gi.make_inputs("gdn", B=1, T=300, H=2, seed=77)   # smaller than the first: 5 chunks x 2 heads
    rng = np.random.default_rng(78)
    small.initial_state = (rng.standard_normal((1, 2, 128, 128), dtype=np.float32) * np.float32(0.02))
    return big, small


def _kw(inp, d):
    return dict(scale=inp.scale, initial_state=d["initial_state"], l2norm_qk=bool(inp.flags & 1),
                beta_sigmoid=bool(inp.flags & 2), output_final_state=True)


def test_noalloc_equals_workspace_entry_on_two_calls(oracle_lib):
    import chunked_gated_delta_03_amd as m
    probs = _problems()
    devs = [to_device(inp) for inp in probs]
    refs = []
    for inp, d in zip(probs, devs):
        refs.append(m.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **_kw(inp, d)))
    torch.cuda.synchronize()
    outs = []
    for inp, d in zip(probs, devs):  # two no-allocation calls in a row, the second smaller
        outs.append(m.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], **_kw(inp, d)))
    torch.cuda.synchronize()
    for inp, (o_ws, s_ws), (o_na, s_na) in zip(probs, refs, outs):
        print("noalloc case B=%d T=%d H=%d" % (inp.B, inp.T, inp.H), flush=True)
        assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16))
        assert torch.equal(s_na.view(torch.int32), s_ws.view(torch.int32))
        o_ref, s_ref = oracle_lib.recur(inp)
        o64 = o_na.float().cpu().numpy().astype(np.float64)
        s64 = s_na.cpu().numpy().astype(np.float64)
        assert o_err(o64, o_ref) <= O_ATOL
        assert s_err(s64, s_ref) <= S_RTOL


def test_noalloc_into_caller_outputs_and_without_final_state(oracle_lib):
    import chunked_gated_delta_03_amd as m
    inp = gi.make_inputs("gdn", B=1, T=129, H=3, seed=79)
    d = to_device(inp)
    o = torch.empty((1, 129, 3, 128), dtype=torch.bfloat16, device="cuda")
    kw = _kw(inp, d)
    kw["output_final_state"] = False
    o2, fs = m.gdn_chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], out=(o, None), **kw)
    torch.cuda.synchronize()
    assert fs is None and o2.data_ptr() == o.data_ptr()
    o_ref, _ = oracle_lib.recur(inp)
    assert o_err(o.float().cpu().numpy().astype(np.float64), o_ref) <= O_ATOL
