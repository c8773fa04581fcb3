"""GPU parity: the HIP path (through the C ABI) against the oracle.

Stage tests compare each kernel's output with the chunk-form intermediates of
``oracle.chunk``; end-to-end tests compare o and the final state with the
token recurrence ``oracle.recur`` (max |o - o_ref| <= 2e-2, max |S - S_ref| /
max |S_ref| <= 1e-3). Full-size workloads are checked on (sequence, head)
units sampled from the same launch the benchmark times.
"""
import sys

import numpy as np
import pytest

import gdn_inputs as gi
import oracle
from gpu_util import (O_ATOL, S_RTOL, check_all_units, decode_aqk, decode_tmat, hm_chunks, o_err, run_gpu,
                      s_err, to_device)

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


def _problems_reduced():
    rng = np.random.default_rng(77)
    out = [
        ("tiny", gi.make_inputs("tiny")),
        ("gdn_B2_T300_H3", gi.make_inputs("gdn", B=2, T=300, H=3)),
        ("gdn_T1", gi.make_inputs("gdn", B=3, T=1, H=2)),
        ("gdn_T63", gi.make_inputs("gdn", B=1, T=63, H=2)),
        ("gdn_T64", gi.make_inputs("gdn", B=2, T=64, H=2)),
        ("gdn_T65", gi.make_inputs("gdn", B=1, T=65, H=2)),
        ("gdn_T127", gi.make_inputs("gdn", B=1, T=127, H=3)),
        ("varlen_docs", gi.make_inputs("varlen", H=3, doc_lengths=[1, 17, 63, 64, 65, 130, 200])),
        ("varlen_one_doc", gi.make_inputs("varlen", H=2, doc_lengths=[333])),
        ("long_T2048_H2", gi.make_inputs("long", T=2048, H=2)),
        ("mild_gate_init", gi.random_problem(rng, 2, 250, 2, 128, 128, gate_scale=0.01, with_initial_state=True)),
        ("host_normalised_B2_T300_H3", gi.make_inputs("tiny", B=2, T=300, H=3)),
        # 64+ (sequence, head) units: the state kernel's four-compute-wave form
        ("wide_B4_T200_H16", gi.make_inputs("gdn", B=4, T=200, H=16)),
        ("wide_varlen_H16", gi.make_inputs("varlen", H=16, doc_lengths=[1, 64, 65, 130, 7])),
        # 65 units: the four-compute-wave form with padding workgroups (the
        # grid rounds the units up to groups of 8), ragged last chunk
        ("wide_pad_B5_T130_H13", gi.make_inputs("gdn", B=5, T=130, H=13)),
        # gates that barely decay (or not at all) over 64 chunks: rounding errors
        # written into the state persist, so the state operands must keep
        # about 16 significant bits (single bf16 there gives 1.4e-3 .. 1.7e-3)
        ("slow_gate_T4096_H2", gi.random_problem(rng, 1, 4096, 2, 128, 128, gate_scale=0.001)),
        ("no_decay_T4096_H2", gi.random_problem(rng, 1, 4096, 2, 128, 128, gate_scale=0.0)),
        ("kda_slow_gate_T4096_H2", gi.random_problem(rng, 1, 4096, 2, 128, 128, kda=True, gate_scale=0.001,
                                                     with_initial_state=True)),
    ]
    return out


REDUCED = _problems_reduced()


@pytest.mark.parametrize("name,inp", REDUCED, ids=[n for n, _ in REDUCED])
def test_end_to_end_reduced(gdn, name, inp):
    _say("case", name, "B,T,H =", inp.B, inp.T, inp.H, "docs", None if inp.cu_seqlens is None else len(inp.cu_seqlens) - 1)
    o_ref, s_ref = oracle.recur(inp)
    o, fs = run_gpu(inp)
    assert np.isfinite(o).all()
    eo = o_err(o, o_ref)
    es = s_err(fs, s_ref)
    _say("  o max-abs err %.3e   final-state rel err %.3e" % (eo, es))
    assert eo <= O_ATOL
    assert es <= S_RTOL


def test_stage_parity(gdn):
    """Each stage against the chunk-form intermediates of the oracle."""
    # gdn_B4_T1024_H16 has 1,024 (chunk, head) items, more than the prepare
    # kernel's persistent grid (three workgroups per compute unit), so each
    # workgroup takes several items and the next item's loads overlap the
    # previous item's deferred stores
    for name, inp in [("tiny", gi.make_inputs("tiny")),
                      ("gdn_B2_T200_H2", gi.make_inputs("gdn", B=2, T=200, H=2)),
                      ("varlen", gi.make_inputs("varlen", H=2, doc_lengths=[17, 64, 100])),
                      ("gdn_B4_T1024_H16", gi.make_inputs("gdn", B=4, T=1024, H=16))]:
        _say("stage case", name)
        d = to_device(inp)
        l2, sig = bool(inp.flags & 1), bool(inp.flags & 2)
        tmat, aqk, vec, _ = gdn.gdn_stage_prepare(d["q"], d["k"], d["g"], d["beta"], scale=inp.scale,
                                                  cu_seqlens=inp.cu_seqlens, l2norm_qk=l2, beta_sigmoid=sig)
        torch.cuda.synchronize()
        _, _, inters = oracle.chunk(inp, keep=True)
        dense = inp.cu_seqlens is None
        T_ref = hm_chunks([it["T"] for it in inters], dense)
        A_ref = hm_chunks([it["Aqk"] for it in inters], dense)
        G_ref = hm_chunks([it["G"] for it in inters], dense)
        b_ref = hm_chunks([it["beta"] for it in inters], dense)
        rq_ref = hm_chunks([it["rq"] for it in inters], dense)
        rk_ref = hm_chunks([it["rk"] for it in inters], dense)
        tm = decode_tmat(tmat)
        assert np.abs(tm - T_ref).max() <= 1e-4 * max(1.0, np.abs(T_ref).max())
        aq = decode_aqk(aqk)
        assert np.abs(aq - A_ref).max() <= 1e-2 * max(1e-3, np.abs(A_ref).max())
        vc = vec.cpu().numpy().astype(np.float64)
        np.testing.assert_allclose(vc[:, :, 4], G_ref, rtol=1e-5, atol=1e-4)
        np.testing.assert_allclose(vc[:, :, 0], b_ref, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(vc[:, :, 5], rq_ref, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(vc[:, :, 6], rk_ref, rtol=1e-5, atol=1e-6)

        s0 = d["initial_state"]
        h, v_new, fs = gdn.gdn_stage_fwd_h(d["k"], d["v"], tmat, vec, initial_state=s0, cu_seqlens=inp.cu_seqlens)
        torch.cuda.synchronize()
        h_ref = hm_chunks([it["h"] for it in inters], dense)
        vn_ref = hm_chunks([it["v_new"] for it in inters], dense)
        hh = h.cpu().numpy().astype(np.float64)
        vn = v_new.cpu().numpy().astype(np.float64)
        eh = np.abs(hh - h_ref).max() / max(np.abs(h_ref).max(), 1e-30)
        ev = np.abs(vn - vn_ref).max() / max(np.abs(vn_ref).max(), 1e-30)
        _say("  h rel err %.3e  v_new rel err %.3e" % (eh, ev))
        assert eh <= 1e-3 and ev <= 1e-3
        _, s_ref = oracle.recur(inp)
        assert s_err(fs.cpu().numpy().astype(np.float64), s_ref) <= S_RTOL

        # finalize alone, fed the oracle's h and v_new
        o = gdn.gdn_stage_finalize(d["q"], aqk, vec, torch.from_numpy(h_ref.astype(np.float32)).cuda(),
                                   torch.from_numpy(vn_ref.astype(np.float32)).cuda(), cu_seqlens=inp.cu_seqlens)
        torch.cuda.synchronize()
        o_ref, _ = oracle.recur(inp)
        assert o_err(o.float().cpu().numpy().astype(np.float64), o_ref) <= O_ATOL


def test_fused_matches_stage_path(gdn):
    inp = gi.make_inputs("gdn", B=2, T=500, H=4)
    d = to_device(inp)
    tmat, aqk, vec, _ = gdn.gdn_stage_prepare(d["q"], d["k"], d["g"], d["beta"], scale=inp.scale,
                                              l2norm_qk=True, beta_sigmoid=True)
    h, v_new, fs1 = gdn.gdn_stage_fwd_h(d["k"], d["v"], tmat, vec)
    o1 = gdn.gdn_stage_finalize(d["q"], aqk, vec, h, v_new)
    o2, fs2 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=inp.scale, l2norm_qk=True,
                                beta_sigmoid=True)
    torch.cuda.synchronize()
    assert torch.equal(fs1, fs2)
    assert (o1.float() - o2.float()).abs().max().item() <= 1e-2


def test_deterministic(gdn):
    inp = gi.make_inputs("varlen", H=4, doc_lengths=[100, 1, 300, 64])
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_concurrent_streams_match_sequential(gdn):
    """Calls enqueued on two streams at once (packed inputs, whose chunk
    tables go through the library's pinned staging ring, and dense KDA
    inputs, stream-ordered workspaces) give the same bits as one at a time."""
    probs = [gi.make_inputs("varlen", H=3, doc_lengths=[70, 1, 200, 64]),
             gi.make_inputs("kda", B=1, T=150, H=2),
             gi.make_inputs("varlen", H=2, doc_lengths=[5, 130]),
             gi.make_inputs("gdn", B=2, T=100, H=2)]
    ref = [run_gpu(p) for p in probs]
    devs = [to_device(p) for p in probs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        for i, (p, d) in enumerate(zip(probs, devs)):
            fn = gdn.kda_chunk_fwd if p.kda else gdn.gdn_chunk_fwd
            s = streams[i % 2]
            with torch.cuda.stream(s):
                outs.append((i, fn(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=p.scale,
                                   initial_state=d["initial_state"], cu_seqlens=p.cu_seqlens,
                                   l2norm_qk=bool(p.flags & 1), beta_sigmoid=bool(p.flags & 2),
                                   output_final_state=True, stream=s)))
    torch.cuda.synchronize()
    for i, (o, fs) in outs:
        assert np.array_equal(o.float().cpu().numpy().astype(np.float64), ref[i][0]), i
        assert np.array_equal(fs.cpu().numpy().astype(np.float64), ref[i][1]), i


def test_no_final_state_flag(gdn):
    inp = gi.make_inputs("gdn", B=1, T=130, H=2)
    inp.flags &= ~gi.FLAG_OUTPUT_FINAL_STATE
    o, fs = run_gpu(inp)
    assert fs is None
    o_ref, _ = oracle.recur(inp)
    assert o_err(o, o_ref) <= O_ATOL


def test_caller_workspace_and_errors(gdn):
    inp = gi.make_inputs("gdn", B=1, T=100, H=2)
    need = gdn.workspace_bytes(1, 100, 2)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o, fs = run_gpu(inp, workspace=ws)
    o_ref, s_ref = oracle.recur(inp)
    assert o_err(o, o_ref) <= O_ATOL and s_err(fs, s_ref) <= S_RTOL
    d = to_device(inp)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=-1.0)
    assert e.value.code == gdn.GDN_ERR_INVALID_ARGUMENT
    q64 = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd(q64, q64, q64, torch.zeros((1, 8, 2), device="cuda"),
                          torch.zeros((1, 8, 2), dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == gdn.GDN_ERR_UNSUPPORTED


def _kda_problems():
    rng = np.random.default_rng(91)
    return [
        ("kda_B1_T300_H2", gi.make_inputs("kda", B=1, T=300, H=2)),
        ("kda_B2_T64_H3", gi.make_inputs("kda", B=2, T=64, H=3)),
        ("kda_T1", gi.make_inputs("kda", B=2, T=1, H=2)),
        ("kda_T65", gi.make_inputs("kda", B=1, T=65, H=2)),
        ("kda_mild_init", gi.random_problem(rng, 2, 200, 2, 128, 128, kda=True, gate_scale=0.02,
                                            with_initial_state=True)),
        ("kda_packed", gi.random_problem(rng, 1, 317, 2, 128, 128, kda=True, with_initial_state=True,
                                         cu_seqlens=[0, 1, 18, 82, 147, 317])),
        # 64+ (sequence, head) units: the four-compute-wave form of the state kernel
        ("kda_wide_B2_T130_H32", gi.make_inputs("kda", B=2, T=130, H=32)),
        ("kda_wide_pad_B5_T70_H13", gi.make_inputs("kda", B=5, T=70, H=13)),
    ]


KDA = _kda_problems()


@pytest.mark.parametrize("name,inp", KDA, ids=[n for n, _ in KDA])
def test_kda_end_to_end_reduced(gdn, name, inp):
    _say("kda case", name, "B,T,H =", inp.B, inp.T, inp.H)
    o_ref, s_ref = oracle.recur(inp)
    o, fs = run_gpu(inp)
    assert np.isfinite(o).all()
    eo, es = o_err(o, o_ref), s_err(fs, s_ref)
    _say("  o max-abs err %.3e   final-state rel err %.3e" % (eo, es))
    assert eo <= O_ATOL and es <= S_RTOL


def test_kda_stage_parity(gdn):
    for name, inp in [("kda_B1_T200_H2", gi.make_inputs("kda", B=1, T=200, H=2)),
                      ("kda_packed", gi.random_problem(np.random.default_rng(5), 1, 150, 2, 128, 128, kda=True,
                                                       with_initial_state=True, cu_seqlens=[0, 17, 81, 150]))]:
        _say("kda stage case", name)
        d = to_device(inp)
        tmat, aqk, vec, gk = gdn.gdn_stage_prepare(d["q"], d["k"], d["g"], d["beta"], scale=inp.scale,
                                                   cu_seqlens=inp.cu_seqlens, kda=True, l2norm_qk=True,
                                                   beta_sigmoid=True)
        torch.cuda.synchronize()
        _, _, inters = oracle.chunk(inp, keep=True)
        dense = inp.cu_seqlens is None
        T_ref = hm_chunks([it["T"] for it in inters], dense)
        A_ref = hm_chunks([it["Aqk"] for it in inters], dense)
        G_ref = hm_chunks([it["G"] for it in inters], dense)
        tm = decode_tmat(tmat)
        et = np.abs(tm - T_ref).max() / max(1.0, np.abs(T_ref).max())
        aq = decode_aqk(aqk)
        ea = np.abs(aq - A_ref).max() / max(1e-3, np.abs(A_ref).max())
        gg = gk.cpu().numpy().astype(np.float64)
        eg = np.abs(gg - G_ref).max() / max(1.0, np.abs(G_ref).max())
        _say("  T err %.3e  Aqk err %.3e  G err %.3e" % (et, ea, eg))
        assert et <= 1e-4 and ea <= 1e-2 and eg <= 1e-5
        h, v_new, fs = gdn.gdn_stage_fwd_h(d["k"], d["v"], tmat, vec, gk=gk, initial_state=d["initial_state"],
                                           cu_seqlens=inp.cu_seqlens, kda=True)
        torch.cuda.synchronize()
        h_ref = hm_chunks([it["h"] for it in inters], dense)
        vn_ref = hm_chunks([it["v_new"] for it in inters], dense)
        eh = np.abs(h.cpu().numpy() - h_ref).max() / max(np.abs(h_ref).max(), 1e-30)
        ev = np.abs(v_new.cpu().numpy() - vn_ref).max() / max(np.abs(vn_ref).max(), 1e-30)
        _say("  h rel err %.3e  v_new rel err %.3e" % (eh, ev))
        assert eh <= 1e-3 and ev <= 1e-3
        o = gdn.gdn_stage_finalize(d["q"], aqk, vec, torch.from_numpy(h_ref.astype(np.float32)).cuda(),
                                   torch.from_numpy(vn_ref.astype(np.float32)).cuda(), gk=gk,
                                   cu_seqlens=inp.cu_seqlens, kda=True)
        torch.cuda.synchronize()
        o_ref, _ = oracle.recur(inp)
        assert o_err(o.float().cpu().numpy().astype(np.float64), o_ref) <= O_ATOL


def _full_size(name):
    inp = gi.make_inputs(name)
    _say("full-size %s: inputs ready (%d sequences)" % (name, inp.num_seqs))
    o, fs = run_gpu(inp)
    _say("full-size %s: GPU done" % name)
    o_ref, s_ref = oracle.recur(inp)
    _say("full-size %s: oracle done" % name)
    check_all_units(o, fs, o_ref, s_ref, _say)


def test_full_size_gdn(gdn):
    """B=4 T=4096 H=16, the benchmarked launch: every output and final state."""
    _full_size("gdn")


def test_full_size_varlen(gdn):
    """Packed T=32768 H=16, documents ~U[17,8192] with per-document initial
    states: every output and every document's final state."""
    _full_size("varlen")


def test_full_size_long(gdn):
    """B=1 T=131072 H=32 (2048 sequential chunks): every output and final state."""
    _full_size("long")


def test_full_size_kda(gdn):
    """KDA B=2 T=8192 H=32 per-channel gate: every output and final state."""
    _full_size("kda")


def _degenerate_cases():
    """The method's degenerate inputs, on both gate kinds: a gate of -1000 at
    one token (the carried state and earlier tokens are forgotten: every decay
    path underflows to exactly 0), beta = 0 (the state only decays), k = 0
    (no writes), and a run whose gate is -1000 at every token."""
    out = []
    for kda in (False, True):
        tag = "kda" if kda else "gdn"
        rng = np.random.default_rng(300 + kda)
        base = gi.random_problem(rng, 2, 200, 2, 128, 128, kda=kda, gate_scale=0.05, with_initial_state=True)
        g = base.g.copy()
        g[:, 77] = -1000.0
        out.append((tag + "_reset_at_77", gi.GdnInputs(**{**base.__dict__, "g": g})))
        beta0 = gi.f32_to_bf16_bits(np.zeros(base.beta.shape, dtype=np.float32))
        out.append((tag + "_beta_zero", gi.GdnInputs(**{**base.__dict__, "beta": beta0,
                                                         "flags": gi.FLAG_L2NORM_QK | gi.FLAG_OUTPUT_FINAL_STATE})))
        k0 = gi.f32_to_bf16_bits(np.zeros(gi.bf16_bits_to_f32(base.k).shape, dtype=np.float32))
        out.append((tag + "_k_zero", gi.GdnInputs(**{**base.__dict__, "k": k0,
                                                      "flags": gi.FLAG_BETA_SIGMOID | gi.FLAG_OUTPUT_FINAL_STATE})))
        out.append((tag + "_gate_all_reset", gi.GdnInputs(**{**base.__dict__, "g": np.full_like(base.g, -1000.0)})))
    return out


DEGENERATE = _degenerate_cases()


@pytest.mark.parametrize("name,inp", DEGENERATE, ids=[n for n, _ in DEGENERATE])
def test_degenerate_inputs(gdn, name, inp):
    _say("degenerate case", name)
    o_ref, s_ref = oracle.recur(inp)
    o, fs = run_gpu(inp)
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    eo = o_err(o, o_ref)
    es = float(np.abs(fs - s_ref).max() / max(np.abs(s_ref).max(), 1e-3))
    _say("  o max-abs err %.3e   final-state err %.3e (max |S_ref| %.2e)" % (eo, es, np.abs(s_ref).max()))
    assert eo <= O_ATOL
    assert es <= S_RTOL
