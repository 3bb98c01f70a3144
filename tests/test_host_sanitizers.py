"""Host code under AddressSanitizer, UndefinedBehaviorSanitizer and (the
oracle's threads) ThreadSanitizer (no GPU).

The CPU oracle (oracle/oracle.c) is built with a C driver that calls every
entry point on small seeded inputs; the C ABI layer (capi.cpp: argument
validation, the split and workspace planners) is built with its host side
instrumented, linked with stand-ins for the kernel launchers, and driven over
a grid of shapes up to the documented limits and through every rejection
path.  Any out-of-bounds access, use after free, leak (oracle) or undefined
operation (signed overflow, misaligned access, ...) fails the test with the
sanitizer's report.  Built with gcc (the oracle) and with hipcc's host pass
only (the ABI layer: the sanitizer flags go to the host compiler alone), in a
temporary directory."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["address", "undefined"]


def _run(cmd, cwd, env=None, timeout=600):
    r = subprocess.run(cmd, cwd=cwd, env=env, capture_output=True, text=True, timeout=timeout)
    if r.returncode != 0:
        raise AssertionError("%s failed (%d):\n%s\n%s" % (cmd[0], r.returncode, r.stdout[-4000:], r.stderr[-4000:]))
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    flags = ["-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    flags += ["-fsanitize=" + s for s in SAN]
    _run(["gcc", *flags, os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-lm", "-lpthread", "-o", exe], str(tmp_path))
    env = dict(os.environ, UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = _run([exe], str(tmp_path), env=env, timeout=300)
    assert out.strip().endswith("ok")


def test_oracle_threads_under_thread_sanitizer(tmp_path):
    # the oracle splits rows and sequences over POSIX threads that write
    # disjoint outputs; ThreadSanitizer checks that no two of them race
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_tsan")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=thread", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread", "-o", exe], str(tmp_path))
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    out = _run([exe], str(tmp_path), env=env, timeout=300)
    assert out.strip().endswith("ok")


def test_abi_host_code_under_sanitizers(tmp_path):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    sys.path.insert(0, os.path.join(ROOT, "speculative_decoding_verify_attn_amd"))
    import build as B  # the library's own compile flags
    host_san = []
    for s in SAN:
        host_san += ["-Xarch_host", "-fsanitize=" + s]
    host_san += ["-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in B.COMPILE_FLAGS if f != "-O3"] + ["-O1", "-g"]
    objs = []
    for src in (os.path.join(ROOT, "speculative_decoding_verify_attn_amd", "csrc", "capi.cpp"),
                os.path.join(HERE, "launch_stubs.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run(["hipcc", *flags, *host_san, "-c", "-x", "hip", src, "-o", obj], str(tmp_path))
        objs.append(obj)
    drv = str(tmp_path / "capi_driver.o")
    _run(["hipcc", "-O1", "-g", "-std=c++17", *host_san, "-c", os.path.join(HERE, "capi_driver.cpp"), "-o", drv],
         str(tmp_path))
    exe = str(tmp_path / "capi_san")
    _run(["hipcc", "--offload-arch=" + B.ARCH, *host_san, drv, *objs, "-o", exe], str(tmp_path))
    # the HIP runtime (not instrumented) keeps allocations until exit: no leak check here
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = _run([exe], str(tmp_path), env=env, timeout=300)
    assert out.strip().split()[0] == "ok"
