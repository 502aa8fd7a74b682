"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The float64 oracle (plain C) is built with gcc and both sanitizers and run
  by a C driver that compares its two forms (tests/native/oracle_sanitize.c).
* libgdr's host side (argument validation, dispatch, launch setup) is built
  host-only (no device code) with both sanitizers and driven through the C
  ABI by tests/native/abi_sanitize.c: every entry point with invalid
  arguments, and -- on a host without a GPU -- with valid ones, which must
  return GDR_ERR_HIP rather than crash.  Without device code each object's
  fat binary is an empty offload bundle (enough where no GPU is visible; the
  driver skips itself where one is).

Sanitizers apply to host code only: the HIP compile lines pass each
-fsanitize option behind -Xarch_host and build no device code at all.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "gated_delta_rule_08_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _tool(*cands):
    for c in cands:
        p = shutil.which(c) if not os.path.isabs(c) else (c if os.path.exists(c) else None)
        if p:
            return p
    pytest.skip("none of %s found" % (cands,))


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = _tool("gcc")
    exe = str(tmp_path / "oracle_sanitize")
    rc, out = _run([gcc, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-Wall", "-o", exe, os.path.join(NATIVE, "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "gdr_oracle.c"), "-lm", "-pthread"])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=120)
    assert rc == 0 and "all checks passed" in out, out


def test_abi_host_side_under_asan_ubsan(tmp_path):
    hipcc = _tool(os.environ.get("HIPCC", "hipcc"), "/opt/rocm/bin/hipcc")
    clang = _tool("/opt/rocm/llvm/bin/clang", "clang")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined"]
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = _run([hipcc, "--offload-host-only", "-O1", "-g", "-fPIC", "-std=c++17",
                        "-fno-omit-frame-pointer"] + san +
                       ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-c", src, "-o", obj])
        assert rc == 0, out
        objs.append(obj)
    # Without device code, each object still names its (absent) fat binary.
    # An empty offload bundle stands in for each: registration accepts it,
    # and with no GPU every launch fails at runtime start-up anyway.
    names = set()
    for obj in objs:
        rc, out = _run(["nm", "-u", obj])
        assert rc == 0, out
        names |= {ln.split()[-1] for ln in out.splitlines() if "__hip_fatbin_" in ln}
    stub = tmp_path / "fatbin_stub.c"
    stub.write_text("".join('const char %s[32] __attribute__((aligned(4096))) = '
                            '"__CLANG_OFFLOAD_BUNDLE__";\n' % n for n in sorted(names)))
    rc, out = _run([clang, "-c", "-fPIC", str(stub), "-o", str(tmp_path / "fatbin_stub.o")])
    assert rc == 0, out
    lib = str(tmp_path / "libgdr_san.so")
    rc, out = _run([hipcc, "--offload-host-only", "-shared", "-fPIC"] + san + ["-o", lib] + objs +
                   [str(tmp_path / "fatbin_stub.o")])
    assert rc == 0, out
    exe = str(tmp_path / "abi_sanitize")
    rc, out = _run([clang, "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-I" + os.path.join(ROOT, "include"), "-o", exe,
                    os.path.join(NATIVE, "abi_sanitize.c"), lib, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath," + str(tmp_path)])
    assert rc == 0, out
    rc, out = _run([exe], env=ENV, timeout=120)
    if rc == 77:
        pytest.skip("a GPU is visible; the valid-call checks run only without one")
    assert rc == 0 and "all checks passed" in out, out
