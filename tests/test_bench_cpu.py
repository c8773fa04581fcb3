"""Host-side contract of bench.py that needs no GPU: one GPU only, and the
roofline bookkeeping (algorithmic bytes per token-head, counter lookup)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_hash_follows_the_workloads_sources():
    assert "kda_bwd.hip" not in bench.sources_for("gdn")
    assert "kda_bwd.hip" in bench.sources_for("bwd_kda")
    assert "gdn_bwd.hip" in bench.sources_for("bwd_gdn")
    assert bench.sources_for("conv") == ("gdn_common.h", "gdn_kernels.h", "short_conv.hip")


def test_algorithmic_bytes_per_token_head():
    # q, k, v bf16 (768) + gate (GDN 4 / KDA 512) + beta (2) + o bf16 (256)
    assert bench.GDN_PREP_BYTES + bench.STATE_BYTES == 1030
    assert bench.KDA_PREP_BYTES + bench.STATE_BYTES == 1538


def test_recorded_traffic_requires_matching_sources(tmp_path, monkeypatch):
    """A counter summary counts only for the kernel sources it was taken on."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    rec = {"workload": "gdn", "kernel_source_hash": bench.kernel_source_hash("gdn"),
           "kernels": {"void gdn::gdn_state_kernel<2, false, true>(gdn::FwdArgs)": {"hbm_bytes_scaled": 123.0}}}
    (prof / "x_hbm_counters.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w=None: rec["kernel_source_hash"])
    assert bench.recorded_traffic("gdn", "gdn_state_kernel") == 123.0
    assert bench.recorded_traffic("kda", "gdn_state_kernel") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda w=None: "other")
    assert bench.recorded_traffic("gdn", "gdn_state_kernel") is None
