"""In-kernel gate of the forward entry, fp64 (TEST INFRASTRUCTURE ONLY).

The pages' native entries take the gate either as a ready per-token log
decay or as raw logits with the parameters ``A_log`` (per head) and
``dt_bias`` (per head, or per head and key channel for KDA) and a
``use_gate_in_kernel`` switch (the fla-npu forward contract on the
hyper-parallel "Diff Coverage" page of the 2026-11-06 gate build;
``_prepare_kda`` on the kimi_delta_attention_ascendc.py coverage page); they
do not print the formula. The reading taken here is the gate of the GDN and
KDA layers that the workloads use:

  GDN:  g = -exp(A_log[h]) * softplus(a + dt_bias[h])           (natural log)
  KDA:  g = -exp(A_log[h]) * softplus(x + dt_bias[h, d]) / ln 2   (log2)

with softplus(x) = log(1 + e^x). The safe-gate variant with a lower bound
(KDA ``safe_gate``, ``lower_bound``) is not covered: no formula for it is
given.

Pinned by tests/test_gate_pins.py (softplus(0) = ln 2 closed forms, the
linear asymptote, numpy's logaddexp).
"""
from __future__ import annotations

import numpy as np


def _softplus(x: np.ndarray) -> np.ndarray:
    # log(1 + e^x) without overflow: max(x, 0) + log1p(e^-|x|)
    x = np.asarray(x, dtype=np.float64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def gdn_gate(a: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """a [B,T,H] (or [T,H]), a_log [H], dt_bias [H] -> g, same shape as a, fp64."""
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(a_log) * _softplus(np.asarray(a, dtype=np.float64) + dt_bias)


def kda_gate(x: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """x [B,T,H,K], a_log [H], dt_bias [H,K] -> g (log2 units), fp64."""
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(a_log)[:, None] * _softplus(np.asarray(x, dtype=np.float64) + dt_bias) / np.log(2.0)
