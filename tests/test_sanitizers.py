"""Host-side sanitizers (no GPU): the reference and the C ABI's host code, built with
AddressSanitizer and UndefinedBehaviorSanitizer, run small drivers (tests/sanitize/) that
exercise every reference function and every entry point's validation.  Any invalid memory
access, leak (reference) or undefined operation aborts the driver."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, "%s\n%s" % (" ".join(cmd), r.stdout[-4000:])
    return r.stdout


def test_reference_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe])
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert "oracle driver: ok" in out


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from sparse_moe_transformer_wave_amd import build as b
    objs = [os.path.join(b.BUILD_DIR, "moe_%s.o" % n) for n in ("route", "permute", "gemv", "gemm", "decode1", "decode_few")]
    if not all(os.path.exists(o) for o in objs):
        b.build_moe()
    api = str(tmp_path / "api_san.o")
    # the sanitizers instrument the host code only (-Xarch_host); the device code is as shipped
    _run([HIPCC] + [f for f in b.HIP_FLAGS if f != "-O3"] +
         ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-c", os.path.join(ROOT, "sparse_moe_transformer_wave_amd", "csrc", "api.hip"), "-o", api])
    drv = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-std=c11", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c",
          os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([CLANG + "++", "-fsanitize=address,undefined", drv, api] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    out = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert "abi driver: ok" in out
