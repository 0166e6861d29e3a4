"""The library's host code and the oracle under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

* The HIP sources are compiled for the host only (no device code) with ASan and
  UBSan and linked with tests/sanitize/hip_stub.cpp in place of the HIP runtime: the
  checks in tests/sanitize/lib_host_checks.cpp sweep the planners over shapes, call
  every entry point (nothing reaches a device; the stub checks and records each
  launch: grid, block, LDS against 160 KB) and its refusal paths.
* oracle.c is compiled with ASan and UBSan and run by tests/sanitize/oracle_checks.c on
  small inputs, including every refusal.
No GPU is used.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "selective_state_space_79_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"   # the host compiler hipcc drives (one sanitizer runtime)
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm compilers not installed")
def test_library_host_code_under_sanitizers(tmp_path):
    # host-only objects of the library; every sanitizer flag is for the host pass
    host = ["--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", "-I",
            os.path.join(ROOT, "include")]
    for flag in SAN:
        host += ["-Xarch_host", flag]
    objs, procs = [], []
    for name in ("scan_fwd", "scan_bwd", "ssd_fwd", "scan_chunked"):
        obj = str(tmp_path / f"{name}.o")
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, *host, "-c", "-o", obj, os.path.join(CSRC, f"{name}.hip")],
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for pr in procs:
        out, err = pr.communicate(timeout=600)
        assert pr.returncode == 0, err[-3000:]
    # the fat-binary symbols the host objects reference (their device code is not built)
    syms = set()
    for obj in objs:
        r = _run(["nm", "-u", obj])
        syms |= set(re.findall(r"\b(__hip_fatbin_[0-9a-f]+)\b", r.stdout))
    (tmp_path / "fatbin_symbols.inc").write_text("".join(f"SSM_STUB_FATBIN({s})\n" for s in sorted(syms)))
    exe = str(tmp_path / "lib_host_checks")
    _run([CLANG, "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
          "-I", str(tmp_path), "-D__HIP_PLATFORM_AMD__", "-o", exe, os.path.join(HERE, "lib_host_checks.cpp"),
          os.path.join(HERE, "hip_stub.cpp"), *objs, "-lpthread"], timeout=600)
    r = _run([exe], env=ENV, timeout=600)
    print(r.stdout)
    assert "0 failed" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", *SAN, "-o", exe, os.path.join(HERE, "oracle_checks.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"], timeout=300)
    r = _run([exe], env=ENV, timeout=300)
    print(r.stdout)
    assert "0 failed" in r.stdout
