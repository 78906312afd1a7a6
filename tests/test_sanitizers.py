"""The oracle and the host library's validation code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: tests/sanitize/oracle_check.c runs every oracle
entry point on small inputs (gcc), and tests/sanitize/abi_check.c calls every C-ABI entry
point with arguments validation must reject, linked against the host code of api.hip and
graph.hip built with the sanitizers on the host side only (the kernels' objects are the
regular ones; nothing reaches a GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "bidirectional_mamba_state_amd", "csrc")
OBJ = os.path.join(ROOT, "bidirectional_mamba_state_amd", "_build")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "bdssm_oracle.c"), "-lm"])
    r = _run([exe], env=ENV)
    assert "ok" in r.stdout


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")
def test_host_validation_under_sanitizers(tmp_path):
    others = [os.path.join(OBJ, f + ".o") for f in ("scan_valu", "block_step_mfma", "block_step_lat",
                                                     "block_step_bw", "prefix_mfma", "conv")]
    if not all(os.path.exists(o) for o in others):
        from bidirectional_mamba_state_amd import build
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    objs = []
    for src in ("api", "graph"):
        o = str(tmp_path / (src + ".o"))
        _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san,
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-I", os.path.join(ROOT, "include"), "-c", "-o", o, os.path.join(CSRC, src + ".hip")])
        objs.append(o)
    exe = str(tmp_path / "abi_check")
    _run(["hipcc", "--offload-arch=gfx950", "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"),
          "-x", "c++", os.path.join(SAN, "abi_check.c"), "-x", "none", *objs, *others, "-o", exe])
    r = _run([exe], env=ENV)
    assert "ok" in r.stdout
