"""Host sanitizer builds (CPU only): the fp64 oracle and the C ABI's host code
under AddressSanitizer and UndefinedBehaviorSanitizer.

* oracle: oracle/gdn_oracle.c with tests/sanitize/oracle_main.c, built by gcc;
  several shapes (with and without an initial state and outputs, T = 0) and the
  one-token closed form.
* C ABI: every library source compiled by hipcc with the sanitizers on the host
  side only (-Xarch_host before each flag; device code is built as usual),
  linked with tests/sanitize/abi_main.cpp by the ROCm clang++.  The driver makes
  only calls that the host checks reject, so no GPU is needed, and sweeps the
  workspace-size queries over the size range.

A sanitizer report makes the program exit non-zero (-fno-sanitize-recover)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CSRC = os.path.join(ROOT, "linear_attention_sequence_deltanet_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, "%s\n%s\n%s" % (" ".join(cmd), r.stdout[-3000:], r.stderr[-3000:])
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), os.path.join(SAN, "oracle_main.c"),
          "-lm", "-o", exe])
    out = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle sanitizer run: ok" in out, out


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "bin", "hipcc")), reason="hipcc not found")
def test_c_abi_host_checks_under_asan_ubsan(tmp_path):
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_gdn_build", os.path.join(ROOT, "linear_attention_sequence_deltanet_amd", "build.py"))
    bld = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bld)
    host_san = []
    for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer"):
        host_san += ["-Xarch_host", f]
    flags = [x if x != "-O3" else "-O1" for x in bld.flags()] + ["-g"] + host_san
    objs = []
    for src in bld.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([bld.hipcc()] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    drv = str(tmp_path / "abi_main.o")
    clangxx = os.path.join(ROCM, "llvm", "bin", "clang++")
    _run([clangxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"), "-c",
          os.path.join(SAN, "abi_main.cpp"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([clangxx, "-fsanitize=address,undefined", drv] + objs +
         ["-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
          "-o", exe])
    out = _run([exe], env=ENV)
    assert "abi sanitizer run: ok" in out, out
