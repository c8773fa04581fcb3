"""Pins of the gate oracle (``oracle.gate``) against closed forms and an
independent library routine."""
import numpy as np

from oracle import gate as og


def test_softplus_against_logaddexp():
    x = np.concatenate([np.linspace(-60, 60, 241), np.random.default_rng(1).standard_normal(1000) * 8])
    assert np.allclose(og._softplus(x), np.logaddexp(0.0, x), rtol=1e-14, atol=1e-300)


def test_gdn_gate_closed_forms():
    a_log = np.array([0.0, np.log(3.0)])
    dt_bias = np.array([0.25, -1.5])
    # a = -dt_bias: softplus(0) = ln 2, so g = -exp(A_log) ln 2
    a = np.broadcast_to(-dt_bias, (1, 4, 2))
    g = og.gdn_gate(a, a_log, dt_bias)
    assert np.allclose(g, -np.exp(a_log) * np.log(2.0), rtol=1e-15)
    # large argument: softplus(y) = y + log1p(e^-y) -> y
    a = np.full((1, 1, 2), 40.0)
    assert np.allclose(og.gdn_gate(a, a_log, dt_bias), -np.exp(a_log) * (40.0 + dt_bias), rtol=1e-15)
    # very negative argument: g -> 0 from below
    g = og.gdn_gate(np.full((1, 1, 2), -80.0), a_log, dt_bias)
    assert (g < 0).all() and (np.abs(g) < 1e-30).all()


def test_kda_gate_closed_forms():
    rng = np.random.default_rng(2)
    H, K = 3, 128
    a_log = rng.uniform(0, np.log(16), H)
    dt_bias = rng.standard_normal((H, K)) * 0.1
    # x = -dt_bias: g = -exp(A_log) ln 2 / ln 2 = -exp(A_log), exactly one power of two per step
    x = np.broadcast_to(-dt_bias, (1, 5, H, K))
    assert np.allclose(og.kda_gate(x, a_log, dt_bias), -np.exp(a_log)[:, None], rtol=1e-15)
    # per-channel log2 gate equals the GDN gate of the same logits divided by ln 2
    x = rng.standard_normal((1, 4, H, K))
    g_gdn = np.stack([og.gdn_gate(x[..., d], a_log, dt_bias[:, d]) for d in range(K)], -1)
    assert np.allclose(og.kda_gate(x, a_log, dt_bias), g_gdn / np.log(2.0), rtol=1e-14)
