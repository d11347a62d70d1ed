"""CPU builds of the oracle and of the library's host-only code under
AddressSanitizer and UndefinedBehaviorSanitizer, each driven by a small
program in tests/sanitize/ (no GPU).

* oracle_check: every oracle entry point on seeded inputs, round trips of
  every layout and escape form, each byte of small containers damaged in
  turn, random headers, and GEMV on ragged shapes.
* host_check: the library's container header check against the oracle's
  reader on every one-bit change of real headers and on random headers, the
  CRC-32 against a bit-at-a-time one, artifact round trips, and every byte of
  an artifact file changed in turn (each must read as corrupt).

Any out-of-bounds access, use after free, leak or undefined operation ends the
program with a sanitizer report and a non-zero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ORACLE = os.path.join(ROOT, "oracle")
CSRC = os.path.join(ROOT, "decode_gemv_sign_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CHECKS = ["address", "undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _host_flags():
    # host-side sanitizers only: each flag goes to the host compilation
    out = []
    for f in [f"-fsanitize={c}" for c in CHECKS] + ["-fno-sanitize-recover=all",
                                                     "-fno-omit-frame-pointer"]:
        out += ["-Xarch_host", f]
    return out


@pytest.fixture(scope="module")
def bindir(tmp_path_factory):
    return tmp_path_factory.mktemp("sanitize")


def test_oracle_under_sanitizers(bindir):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(bindir / "oracle_check")
    _run(["gcc", "-std=c99", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
          "-fsanitize=" + ",".join(CHECKS), "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-I", ORACLE, os.path.join(ORACLE, "wc_oracle.c"), os.path.join(SAN, "oracle_check.c"),
          "-o", exe])
    r = _run([exe], env=_env(), timeout=300)
    assert r.stdout.strip().splitlines()[-1].startswith("ok"), r.stdout
    assert "runtime error" not in r.stderr, r.stderr


def test_host_code_under_sanitizers(bindir):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("ROCm compilers not found")
    objs = []
    # the library's host-only source and the driver: host compilation only
    for src in (os.path.join(CSRC, "wc_artifact.hip"), os.path.join(SAN, "host_check.cpp")):
        obj = str(bindir / (os.path.basename(src) + ".o"))
        _run([HIPCC, "-x", "hip", "--cuda-host-only", "-std=c++17", "-O1", "-g", "-Wall",
              "-I", os.path.join(ROOT, "include"), "-I", ORACLE, "-I", CSRC, *_host_flags(),
              "-c", src, "-o", obj])
        objs.append(obj)
    # the oracle, for the containers and the second header reader
    obj = str(bindir / "wc_oracle.o")
    _run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=" + ",".join(CHECKS),
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", ORACLE, "-c",
          os.path.join(ORACLE, "wc_oracle.c"), "-o", obj])
    objs.append(obj)
    exe = str(bindir / "host_check")
    _run([CLANG + "++", "-fsanitize=" + ",".join(CHECKS), *objs, "-o", exe])
    work = bindir / "files"
    work.mkdir(exist_ok=True)
    r = _run([exe, str(work)], env=_env(), timeout=300)
    out = r.stdout.strip().splitlines()
    assert out[-1].startswith("ok"), r.stdout
    assert any("0 undetected" in l for l in out), r.stdout
    assert "runtime error" not in r.stderr, r.stderr
