"""C-ABI checks that need no GPU: the library loads, exports every function
that include/gdn.h declares, and rejects invalid arguments before any HIP call
(status code + message, nothing launched)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def gdn():
    import chunked_gated_delta_03_amd as m
    return m


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", src, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    for must in ("gdn_chunk_fwd", "kda_chunk_fwd", "gdn_last_error", "gdn_chunk_fwd_workspace_bytes",
                 "gdn_stage_prepare", "gdn_stage_fwd_h", "gdn_stage_finalize", "gdn_num_chunks",
                 "gdn_state_summary", "kda_state_summary", "gdn_state_summary_workspace_bytes",
                 "gdn_state_summary_apply", "gdn_short_conv", "gdn_short_conv_workspace_bytes",
                 "gdn_chunk_bwd", "gdn_chunk_bwd_workspace_bytes", "gdn_chunk_fwd_gated", "kda_chunk_fwd_gated",
                 "gdn_chunk_bwd_gated", "gdn_state_summary_gated", "kda_bwd_state_pass"):
        assert must in names


def test_library_exports_every_declared_symbol(gdn):
    lib = ctypes.CDLL(gdn.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(gdn.EXPORTED) <= set(_declared_functions())


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced by the validation paths


def _call_fwd(gdn, B=1, T=64, H=2, K=128, V=128, cu=None, num_seqs=None, scale=0.1, flags=4, q=FAKE, o=FAKE,
              fs=FAKE, kda=False):
    cu_arr = None if cu is None else np.asarray(cu, dtype=np.int32)
    n = (B if cu is None else len(cu) - 1) if num_seqs is None else num_seqs
    fn = gdn.lib.kda_chunk_fwd if kda else gdn.lib.gdn_chunk_fwd
    return fn(q, FAKE, FAKE, FAKE, FAKE, None, None if cu_arr is None else cu_arr.ctypes.data_as(ctypes.c_void_p),
              n, B, T, H, K, V, scale, flags, o, fs, None, 0, None)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(B=0), 1, "B, T and H"),
    (dict(T=0), 1, "B, T and H"),
    (dict(H=0), 1, "B, T and H"),
    (dict(H=70000), 1, "at most 65535 heads"),
    (dict(K=64), 2, "K = V = 128"),
    (dict(V=256), 2, "K = V = 128"),
    (dict(scale=0.0), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(flags=8), 1, "unknown flag"),
    (dict(q=None), 1, "non-NULL"),
    (dict(q=ctypes.c_void_p(0x100002)), 1, "aligned"),
    (dict(o=None), 1, "o must be non-NULL"),
    (dict(fs=None), 1, "final_state is NULL"),
    (dict(B=2, num_seqs=3), 1, "num_seqs == B"),
    (dict(B=2, T=10, cu=[0, 4, 10]), 1, "B == 1"),
    (dict(T=10, cu=[1, 4, 10]), 1, "cu_seqlens[0]"),
    (dict(T=10, cu=[0, 4, 4, 10]), 1, "strictly increasing"),
    (dict(T=10, cu=[0, 6, 4, 10]), 1, "strictly increasing"),
    (dict(T=10, cu=[0, 4, 9]), 1, "must equal T"),
    (dict(T=10, cu=[0, 4, 10], num_seqs=0), 1, "num_seqs"),
])
def test_invalid_arguments_rejected(gdn, kw, code, msg, kda):
    rc = _call_fwd(gdn, kda=kda, **kw)
    assert rc == code
    assert msg in gdn.last_error()


def _call_fwd_gated(gdn, kda=False, a_log=FAKE, dt_bias=FAKE, g=FAKE, B=1, T=64, H=2, K=128, scale=0.1, flags=4):
    fn = gdn.lib.kda_chunk_fwd_gated if kda else gdn.lib.gdn_chunk_fwd_gated
    return fn(FAKE, FAKE, FAKE, g, a_log, dt_bias, FAKE, None, None, B, B, T, H, K, 128, scale, flags,
              FAKE, FAKE, None, 0, None)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(a_log=None), 1, "A_log and dt_bias"),
    (dict(dt_bias=None), 1, "A_log and dt_bias"),
    (dict(g=None), 1, "non-NULL"),
    (dict(K=64), 2, "K = V = 128"),
    (dict(scale=0.0), 1, "scale"),
])
def test_gated_entries_validate_before_device(gdn, kw, code, msg, kda):
    rc = _call_fwd_gated(gdn, kda=kda, **kw)
    assert rc == code
    assert msg in gdn.last_error()


def test_kda_gated_requires_aligned_gate_operands(gdn):
    rc = _call_fwd_gated(gdn, kda=True, dt_bias=ctypes.c_void_p(0x100004))
    assert rc == 1 and "16-byte aligned" in gdn.last_error()
    rc = _call_fwd_gated(gdn, kda=True, g=ctypes.c_void_p(0x100008))
    assert rc == 1 and "16-byte aligned" in gdn.last_error()


@pytest.mark.parametrize("missing", ["a_log", "dt_bias", "da_log", "ddt_bias"])
def test_gated_bwd_validates_before_device(gdn, missing):
    ptr = {n: (None if n == missing else FAKE) for n in ("a_log", "dt_bias", "da_log", "ddt_bias")}
    rc = gdn.lib.gdn_chunk_bwd_gated(FAKE, FAKE, FAKE, FAKE, ptr["a_log"], ptr["dt_bias"], FAKE, None, None, 1, 1, 64,
                                     2, 128, 128, 0.1, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE, ptr["da_log"],
                                     ptr["ddt_bias"], FAKE, None, None, 0, None)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "dA_log" in gdn.last_error()


def test_gated_summary_validates_before_device(gdn):
    rc = gdn.lib.gdn_state_summary_gated(0, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 1, 64, 2, 128, 128, 0,
                                         FAKE, FAKE, None, 0, None)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT and "A_log" in gdn.last_error()
    rc = gdn.lib.gdn_state_summary_gated(1, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_void_p(0x100004), FAKE, None, 1, 1,
                                         64, 2, 128, 128, 0, FAKE, FAKE, None, 0, None)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT and "16-byte aligned" in gdn.last_error()


def test_kda_bwd_state_pass_validates_before_device(gdn):
    call = lambda **kw: gdn.lib.kda_bwd_state_pass(
        FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 2, kw.get("K", 128), 128, 0.1, 0, kw.get("do", FAKE), None,
        FAKE, kw.get("dvn", FAKE), None, None, 0, None)
    assert call(do=None) == gdn.GDN_ERR_INVALID_ARGUMENT and "non-NULL" in gdn.last_error()
    assert call(dvn=ctypes.c_void_p(0x100004)) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "16-byte aligned" in gdn.last_error()
    assert call(K=64) == gdn.GDN_ERR_UNSUPPORTED
    assert gdn.lib.kda_bwd_state_pass_workspace_bytes(1, 64, 2, 128, 128, 1, None, 0) > 0


def test_num_chunks(gdn):
    assert gdn.num_chunks(1, 1) == 1
    assert gdn.num_chunks(3, 64) == 3
    assert gdn.num_chunks(3, 65) == 6
    assert gdn.num_chunks(1, 150, [0, 1, 18, 82, 150]) == 1 + 1 + 1 + 2
    with pytest.raises(gdn.GdnError):
        gdn.num_chunks(1, 150, [0, 100, 90, 150])


def test_workspace_bytes(gdn):
    # per (chunk, head): T bf16 hi | lo, Aqk bf16, 8 fp32 row vectors
    a = gdn.workspace_bytes(4, 4096, 16)
    nt = 4 * 64
    per = 64 * 64 * 4 + 64 * 64 * 2 + 8 * 64 * 4
    assert a >= 16 * nt * per
    assert a % 256 == 0
    b = gdn.workspace_bytes(1, 150, 16, cu_seqlens=[0, 1, 18, 82, 150])
    assert b >= 16 * 5 * per + 16 * (5 + 4)
    per_kda = 64 * 64 * 4 + 64 * 64 * 2 + 8 * 64 * 4
    k = gdn.workspace_bytes(2, 8192, 32, kda=True)
    assert k >= 32 * 2 * 128 * (per_kda + 64 * 128 * 4)
    with pytest.raises(gdn.GdnError):
        gdn.workspace_bytes(1, 10, 4, cu_seqlens=[0, 11])


def test_stage_entries_validate_before_device(gdn):
    rc = gdn.lib.gdn_stage_prepare(0, FAKE, FAKE, FAKE, FAKE, None, 1, 1, 64, 2, 128, 128, 0.1, 0,
                                   None, FAKE, FAKE, None, None)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT
    rc = gdn.lib.gdn_stage_fwd_h(0, FAKE, FAKE, FAKE, FAKE, None, None, None, 1, 1, 64, 2, 128, 128, 4,
                                 FAKE, FAKE, None, None)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT and "final_state" in gdn.last_error()
    rc = gdn.lib.gdn_stage_finalize(0, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, 1, 1, 64, 2, 64, 64, FAKE, None)
    assert rc == gdn.GDN_ERR_UNSUPPORTED


def test_python_wrapper_checks_shapes(gdn):
    import torch
    q = torch.zeros((1, 8, 2, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gdn.gdn_chunk_fwd(q, q, q, torch.zeros((1, 8, 2)), torch.zeros((1, 8, 2), dtype=torch.bfloat16))


def test_stage_column_order_decoder():
    """The test-side decoder of the stage outputs' column order follows the
    documented mapping 32s+16h+4g+e -> 32s+8g+4h+e and is a permutation."""
    import numpy as np
    from gpu_util import unpermute_cols
    stored = np.zeros(64)
    for s in range(2):
        for h in range(2):
            for g in range(4):
                for e in range(4):
                    stored[32 * s + 8 * g + 4 * h + e] = 32 * s + 16 * h + 4 * g + e
    np.testing.assert_array_equal(unpermute_cols(stored), np.arange(64))


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(K=64), 2, "K = V = 128"),
    (dict(B=0), 1, "B, T and H"),
    (dict(flags=8), 1, "unknown flag"),
    (dict(k=None), 1, "non-NULL"),
    (dict(M=None), 1, "transition and state_ext"),
    (dict(S=None), 1, "transition and state_ext"),
    (dict(T=10, cu=[0, 4, 9]), 1, "must equal T"),
])
def test_state_summary_validates_before_device(gdn, kw, code, msg, kda):
    a = dict(B=1, T=64, H=2, K=128, V=128, flags=3, k=FAKE, M=FAKE, S=FAKE, cu=None)
    a.update(kw)
    cu = None if a["cu"] is None else np.asarray(a["cu"], dtype=np.int32)
    n = a["B"] if cu is None else len(cu) - 1
    fn = gdn.lib.kda_state_summary if kda else gdn.lib.gdn_state_summary
    rc = fn(None, a["k"], FAKE, FAKE, FAKE, None if cu is None else cu.ctypes.data_as(ctypes.c_void_p), n,
            a["B"], a["T"], a["H"], a["K"], a["V"], a["flags"], a["M"], a["S"], None, 0, None)
    assert rc == code
    assert msg in gdn.last_error()


def test_state_summary_workspace_and_apply_validation(gdn):
    ws = gdn.lib.gdn_state_summary_workspace_bytes
    a = ws(0, 1, 8192, 32, 128, 128, 1, None)
    k = ws(1, 1, 8192, 32, 128, 128, 1, None)
    per = 64 * 64 * 4 + 64 * 64 * 2 + 8 * 64 * 4        # GDN: T hi | lo
    assert a >= 32 * 128 * per and a % 256 == 0
    per_kda = 64 * 64 * 4 + 64 * 64 * 2 + 8 * 64 * 4    # KDA: T hi | lo, plus the cumulative gate
    assert k >= 32 * 128 * (per_kda + 64 * 128 * 4)
    assert ws(0, 1, 10, 4, 64, 128, 1, None) == 0
    ap = gdn.lib.gdn_state_summary_apply
    assert ap(None, FAKE, FAKE, FAKE, 1, 2, 128, 128, None) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert ap(FAKE, FAKE, FAKE, ctypes.c_void_p(0x200000), 1, 2, 64, 128, None) == gdn.GDN_ERR_UNSUPPORTED
    assert ap(FAKE, FAKE, ctypes.c_void_p(0x200000), ctypes.c_void_p(0x200000), 1, 2, 128, 128, None) \
        == gdn.GDN_ERR_INVALID_ARGUMENT and "alias" in gdn.last_error()
    assert ap(FAKE, FAKE, FAKE, ctypes.c_void_p(0x200008), 1, 2, 128, 128, None) == gdn.GDN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,code,msg", [
    (dict(D=12), 2, "multiple of 8"),
    (dict(W=9), 2, "1..8"),
    (dict(W=0), 2, "1..8"),
    (dict(dil=0), 1, "dilation"),
    (dict(x=None), 1, "non-NULL"),
    (dict(y=None), 1, "non-NULL"),
    (dict(y=FAKE), 1, "alias"),
    (dict(halo=ctypes.c_void_p(0x100008)), 1, "aligned"),
    (dict(B=2, cu=[0, 4, 10], T=10), 1, "B == 1"),
    (dict(T=10, cu=[0, 4, 9]), 1, "must equal T"),
])
def test_short_conv_validates_before_device(gdn, kw, code, msg):
    a = dict(B=1, T=64, D=64, W=4, dil=1, x=FAKE, y=ctypes.c_void_p(0x200000), halo=None, cu=None)
    a.update(kw)
    cu = None if a["cu"] is None else np.asarray(a["cu"], dtype=np.int32)
    n = a["B"] if cu is None else len(cu) - 1
    rc = gdn.lib.gdn_short_conv(a["x"], FAKE, None, a["halo"], None if cu is None else cu.ctypes.data_as(ctypes.c_void_p),
                                n, a["B"], a["T"], a["D"], a["W"], a["dil"], 1, a["y"], None, 0, None)
    assert rc == code
    assert msg in gdn.last_error()
    cu2 = np.asarray([0, 5, 9], dtype=np.int32)
    assert gdn.lib.gdn_short_conv_workspace_bytes(2, cu2.ctypes.data_as(ctypes.c_void_p)) == 256
    assert gdn.lib.gdn_short_conv_workspace_bytes(2, None) == 0


@pytest.mark.parametrize("kw,code,msg", [
    (dict(K=64), 2, "K = V = 128"),
    (dict(B=0), 1, "B, T and H"),
    (dict(flags=8), 1, "unknown flag"),
    (dict(scale=0.0), 1, "scale"),
    (dict(q=None), 1, "non-NULL"),
    (dict(do=None), 1, "d_o, dq"),
    (dict(dg=None), 1, "d_o, dq"),
    (dict(dq=ctypes.c_void_p(0x100008)), 1, "aligned"),
    (dict(B=2, cu=[0, 4, 10], T=10), 1, "B == 1"),
    (dict(T=10, cu=[0, 4, 9]), 1, "must equal T"),
])
def test_chunk_bwd_validates_before_device(gdn, kw, code, msg):
    a = dict(B=1, T=64, H=2, K=128, V=128, flags=3, scale=0.1, q=FAKE, do=FAKE, dq=FAKE, dg=FAKE, cu=None)
    a.update(kw)
    cu = None if a["cu"] is None else np.asarray(a["cu"], dtype=np.int32)
    n = a["B"] if cu is None else len(cu) - 1
    rc = gdn.lib.gdn_chunk_bwd(a["q"], FAKE, FAKE, FAKE, FAKE, None,
                               None if cu is None else cu.ctypes.data_as(ctypes.c_void_p), n, a["B"], a["T"], a["H"],
                               a["K"], a["V"], a["scale"], a["flags"], a["do"], None, a["dq"], FAKE, FAKE, a["dg"],
                               FAKE, None, None, 0, None)
    assert rc == code
    assert msg in gdn.last_error()


def test_chunk_bwd_workspace_bytes(gdn):
    ws = gdn.lib.gdn_chunk_bwd_workspace_bytes
    fwd = gdn.lib.gdn_chunk_fwd_workspace_bytes(4, 4096, 16, 128, 128, 4, None, 3)
    b = ws(4, 4096, 16, 128, 128, 4, None, 3)
    cmh = 4 * 64 * 16
    assert b >= fwd + cmh * (2 * 128 * 128 * 4 + 5 * 64 * 128 * 4 + 4) and b % 256 == 0
    assert ws(4, 4096, 16, 64, 128, 4, None, 3) == 0
    assert ws(4, 4096, 16, 128, 128, 4, None, 8) == 0


def _header_define(name):
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    m = re.search(r"#define\s+%s\s+\((\d+)u\s*<<\s*(\d+)\)" % name, src)
    return int(m.group(1)) << int(m.group(2))


def _call_noalloc(gdn, B=1, T=64, H=2, K=128, V=128, cu=None, num_seqs=None, scale=0.1, flags=4, q=FAKE, o=FAKE,
                  fs=FAKE):
    cu_arr = None if cu is None else np.asarray(cu, dtype=np.int32)
    n = (B if cu is None else len(cu) - 1) if num_seqs is None else num_seqs
    return gdn.lib.gdn_chunk_fwd_noalloc(q, FAKE, FAKE, FAKE, FAKE, None,
                                         None if cu_arr is None else cu_arr.ctypes.data_as(ctypes.c_void_p),
                                         n, B, T, H, K, V, scale, flags, o, fs, None)


def test_noalloc_scratch_size_matches_binding(gdn):
    assert _header_define("GDN_NOALLOC_SCRATCH_BYTES") == gdn.NOALLOC_SCRATCH_BYTES == 128 << 20


@pytest.mark.parametrize("kw,code,msg", [
    (dict(T=10, cu=[0, 4, 10]), 2, "dense input only"),
    (dict(B=0), 1, "B, T and H"),
    (dict(K=64), 2, "K = V = 128"),
    (dict(scale=0.0), 1, "scale"),
    (dict(q=None), 1, "non-NULL"),
    (dict(o=None), 1, "o must be non-NULL"),
    (dict(fs=None), 1, "final_state is NULL"),
    (dict(B=2, num_seqs=3), 1, "num_seqs == B"),
])
def test_noalloc_invalid_arguments_rejected(gdn, kw, code, msg):
    rc = _call_noalloc(gdn, **kw)
    assert rc == code
    assert msg in gdn.last_error()


def test_noalloc_rejects_problems_beyond_its_scratch(gdn):
    limit = gdn.NOALLOC_SCRATCH_BYTES
    # the largest dense H that fits at B=4, T=4096 by the library's own workspace count, then one more head
    per_head = gdn.lib.gdn_chunk_fwd_workspace_bytes(4, 4096, 1, 128, 128, 4, None, 7)
    assert per_head > 0
    h_fit = limit // per_head
    assert gdn.lib.gdn_chunk_fwd_workspace_bytes(4, 4096, h_fit, 128, 128, 4, None, 7) <= limit
    rc = _call_noalloc(gdn, B=4, T=4096, H=h_fit + 1)
    assert rc == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "scratch" in gdn.last_error()
    # the benchmark shape fits
    assert gdn.lib.gdn_chunk_fwd_workspace_bytes(4, 4096, 16, 128, 128, 4, None, 7) <= limit


def test_documented_size_limits_are_the_enforced_ones(gdn):
    """The header allows B*T < 2^30 and 1 <= H <= 65535; both edges are checked
    before any device call."""
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert "1 <= H <= 65535, B*T < 2^30" in src
    assert _call_fwd(gdn, H=65536) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call_fwd(gdn, B=1, T=1 << 30) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert _call_fwd(gdn, B=2, T=1 << 29) == gdn.GDN_ERR_INVALID_ARGUMENT
    assert "exceeds the supported range" in gdn.last_error()
    # sizes at the edges pass the shape checks: the workspace count (pure host
    # arithmetic) accepts them
    assert gdn.lib.gdn_chunk_fwd_workspace_bytes(1, (1 << 30) - 1, 1, 128, 128, 1, None, 0) > 0
    assert gdn.lib.gdn_chunk_fwd_workspace_bytes(1, 64, 65535, 128, 128, 1, None, 0) > 0
    assert gdn.lib.kda_chunk_fwd_workspace_bytes(1, (1 << 30) - 1, 1, 128, 128, 1, None, 0) > 0
