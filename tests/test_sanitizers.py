"""The oracle and the C ABI's host side under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; any sanitizer finding aborts the
driver).  The library's sources are compiled for the host only (no GPU code;
kernel launches then fail with NVFP4_EHIP, which the driver expects)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def run(cmd, sanitized=False):
    env = dict(os.environ, **SAN_ENV) if sanitized else None
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (cmd, r.stdout[-2000:], r.stderr[-4000:])
    return r


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", *SAN,
         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
         os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), "-o", exe, "-lm"])
    assert "oracle ok" in run([exe], sanitized=True).stdout


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not installed")
def test_c_abi_host_side_under_sanitizers(tmp_path):
    csrc = os.path.join(ROOT, "nvfp4_bit_quantization_amd", "csrc")
    objs = []
    empty = str(tmp_path / "empty.bin")
    open(empty, "wb").close()
    for src in ("quantize.hip", "kv.hip", "gemm.hip", "attn.hip", "capi.cpp", "profile.cpp",
                os.path.join("..", "..", "tests", "sanitize", "abi_driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        # host-only compilation (-Xarch_host before each sanitizer flag); an
        # empty device image stands in for the GPU code
        run([CLANG, "-x", "hip", "--cuda-host-only", "-nogpulib", "-Xclang",
             "-fcuda-include-gpubinary", "-Xclang", empty, "-O1", "-g", "-std=c++17",
             "-Xarch_host", SAN[0], "-Xarch_host", SAN[1], "-Xarch_host", SAN[2],
             f"-I{os.path.join(ROOT, 'include')}", f"-I{ROCM}/include", "-c",
             os.path.join(csrc, src), "-o", obj])
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    run([CLANG, *SAN, *objs, "-o", exe, f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib"])
    r = run([exe], sanitized=True)
    assert "abi ok" in r.stdout
