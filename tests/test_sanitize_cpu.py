"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers, each built in a temporary directory and run as a child process:

- tests/sanitize/oracle_driver.c, linked with oracle/ddtree_oracle.c: every
  oracle function on ragged, degenerate and malformed inputs (ties, NaN and
  infinite logits, whole -inf rows, K = V, N = 1024, requests whose KV range
  lies outside the caches or overflows 64 bits, malformed commit requests),
  one and several threads.
- tests/sanitize/abi_driver.cpp, linked with the library's sources compiled
  with host-side sanitizers: every C-ABI entry point called with arguments
  it must reject, each returning its documented status, and the workspace
  size queries over extreme shapes (INT_MAX sizes, out-of-range dtypes).
  No call passes validation, so nothing is launched.

A sanitizer report ends the child with a non-zero status (recovery is off).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
LIB_SOURCES = ["abi", "k_build", "k_tree", "k_attn", "k_accept", "k_commit", "k_probe"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    if r.returncode != 0:
        raise AssertionError("command failed (%d): %s\n%s%s" % (r.returncode, " ".join(cmd),
                                                                r.stdout[-4000:], r.stderr[-4000:]))
    return r.stdout


def _child_env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1:detect_leaks=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "ddtree_oracle.c"),
          "-lm", "-o", exe])
    out = _run([exe], env=_child_env())
    assert "all paths ran clean" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                    reason="ROCm compilers not available")
@pytest.mark.skipif(os.path.exists("/dev/kfd"),
                    reason="host-only check: run where no GPU is visible")
def test_abi_validation_under_asan_ubsan(tmp_path):
    # device code as usual; every host-side part with the sanitizers
    flags = ["--offload-arch=gfx950", "-O1", "-std=c++17", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I" + os.path.join(ROOT, "include"),
             "-I" + os.path.join(ROOT, "draft_tree_build_amd", "csrc")]
    objs, procs = [], []
    for s in LIB_SOURCES:
        obj = str(tmp_path / (s + ".o"))
        objs.append(obj)
        cmd = [HIPCC] + flags + ["-c", os.path.join(ROOT, "draft_tree_build_amd", "csrc",
                                                     s + ".hip"), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                                            text=True)))
    for cmd, p in procs:
        out, err = p.communicate(timeout=600)
        assert p.returncode == 0, "compile failed: %s\n%s" % (" ".join(cmd), err[-4000:])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
          os.path.join(SAN, "abi_driver.cpp")] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = _run([exe], env=_child_env())
    assert "every rejected call returned its status" in out
