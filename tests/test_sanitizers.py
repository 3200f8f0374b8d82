"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The fp64 oracle (oracle/oracle.c) is compiled with gcc and
  -fsanitize=address,undefined together with tests/sanitize/oracle_edges.c,
  which runs it on edge shapes (N = 1, d = 1, empty and full lengths, empty
  row sets, dropout at p8 = 0 and 255, argument errors) with buffers of exactly
  the size its layout needs; leaks are checked too.
- The C ABI's host side (fa_api.hip, fa_debug.hip) is compiled by hipcc with
  the sanitizers on the host side only (-Xarch_host before each option; device
  code is built as usual) and linked with tests/sanitize/abi_host.cpp, whose
  stub launchers launch nothing.  It drives every entry point through its
  argument checks and planners with extreme sizes (INT_MAX, INT_MIN, the
  largest head), misaligned and null pointers, non-finite scales and
  dropout probabilities, short workspaces, also in debug mode.

Either program stops at the first sanitizer report (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "exact_attention_21_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    return r.returncode, r.stdout, err


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env.pop("FA_DEBUG", None)
    env.pop("FLASH_ATTENTION_DEBUG", None)
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_edges")
    rc, _, err = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                       "-fno-omit-frame-pointer", "-o", exe, os.path.join(HERE, "oracle_edges.c"),
                       os.path.join(ROOT, "oracle", "oracle.c"), "-lm", "-lpthread"])
    assert rc == 0, err
    env = _env()
    env["ASAN_OPTIONS"] += ":detect_leaks=1"
    rc, out, err = _run([exe], env=env, timeout=300)
    assert rc == 0, err[-4000:]
    assert "all passed" in out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not found")
def test_abi_host_code_under_asan_ubsan(tmp_path):
    san = []
    for opt in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
                "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", opt]
    common = ["-O1", "-g", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC, *san]
    objs = []
    for src in (os.path.join(CSRC, "fa_api.hip"), os.path.join(CSRC, "fa_debug.hip"),
                os.path.join(HERE, "abi_host.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        extra = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] \
            if src.endswith(".hip") else []
        rc, _, err = _run([HIPCC, *extra, *common, "-c", src, "-o", obj])
        assert rc == 0, err
        objs.append(obj)
    exe = str(tmp_path / "abi_host")
    # host link with the sanitizer runtimes (no device code is compiled here)
    rc, _, err = _run([CLANG, "-fsanitize=address,undefined", "-o", exe, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                       "-Wl,-rpath,/opt/rocm/lib"])
    assert rc == 0, err
    env = _env()
    # the HIP runtime keeps allocations until exit; leaks are not this test's question
    env["ASAN_OPTIONS"] += ":detect_leaks=0"
    rc, out, err = _run([exe], env=env, timeout=300)
    assert rc == 0, err[-4000:]
    assert "ABI host checks:" in out and "passed" in out
    # the debug-mode pass printed plan lines for the valid calls
    assert "[FA_DEBUG] fa_fwd: " in err and "[FA_DEBUG] fa_bwd: " in err
