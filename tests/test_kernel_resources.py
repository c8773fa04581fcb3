"""Build-level guard on the gfx950 code (CPU only: hipcc cross-compiles).

Every kernel of the library is compiled to assembly with the build's own
flags and checked for two things that have given wrong results or slow code
with no error:
  * indexed register moves (s_set_gpr_idx_on, v_movrels/v_movreld): a
    register-array index that depends on the wave compiles to them, and such a
    move can read an MFMA result before the MFMA has written it;
  * private (scratch) memory: a kernel whose registers spill, or whose
    register array is indexed at run time, keeps it in scratch.
The kernels index register arrays with compile-time indices only, so both
counts must be zero."""
import concurrent.futures
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "chunked_gated_delta_03_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_gdn_build_for_guard", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _assembly(b, src):
    cmd = [b._hipcc(), *b.HIPCC_FLAGS, "--cuda-device-only", "-S", "-o", "-", "-x", "hip", os.path.join(b.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


@pytest.fixture(scope="module")
def assemblies():
    b = _build_module()
    if not os.path.exists(b._hipcc()) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    srcs = [s for s in b.SOURCES if s.endswith(".hip")]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        return dict(zip(srcs, ex.map(lambda s: _assembly(b, s), srcs)))


def _kernels(asm):
    """(name, private segment bytes) of every kernel in the code object metadata."""
    out = []
    for block in asm.split("  - .")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block)
        priv = re.search(r"\.private_segment_fixed_size:\s+(\d+)", block)
        if name and priv:
            out.append((name.group(1), int(priv.group(1))))
    return out


def test_every_source_has_kernels(assemblies):
    for src, asm in assemblies.items():
        assert _kernels(asm), src


def test_no_kernel_uses_scratch(assemblies):
    bad = [(src, k, p) for src, asm in assemblies.items() for k, p in _kernels(asm) if p != 0]
    assert not bad, bad
    for src, asm in assemblies.items():
        assert not re.search(r"^\s+scratch_(load|store)", asm, flags=re.M), src


def test_no_indexed_register_moves(assemblies):
    for src, asm in assemblies.items():
        assert not re.search(r"^\s+(s_set_gpr_idx_on|v_movrels|v_movreld|v_movrelsd)", asm, flags=re.M), src
