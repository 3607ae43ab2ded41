"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

 - the CPU oracle (gcc, with float-to-integer conversion overflow checks as
   well), driven through every entry point on ragged lengths, both head dims,
   smooth_k, causal and the log-sum-exp, on ordinary inputs, on BF16
   subnormals (blocks and channels whose 127/a and 448/a overflow a float)
   and on key channels mixing 2^60 and 2^-60 (tests/sanitize/oracle_driver.c);
 - the library's C ABI with its host code instrumented (hipcc; the device code
   is built as usual), driven with 20 000 seeded random descriptors and the
   documented error cases without a GPU (tests/sanitize/abi_driver.cpp).
Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined,float-cast-overflow",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/lib/llvm/bin/clang++"


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="needs the ROCm toolchain")
def test_c_abi_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("drives the validation paths without a GPU")
    csrc = os.path.join(ROOT, "quantized_attention_prepare_amd", "csrc")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", csrc]
    objs = []
    for src, lang in (("prologue.hip", []), ("attention.hip", []), ("sage_api.cpp", ["-x", "hip"])):
        obj = tmp_path / (src + ".o")
        subprocess.run([HIPCC, *lang, *flags, "-c", os.path.join(csrc, src), "-o", str(obj)], check=True,
                       capture_output=True, text=True)
        objs.append(str(obj))
    drv = tmp_path / "abi_driver.o"
    subprocess.run([HIPCC, "-x", "hip", *flags, "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
                    "-o", str(drv)], check=True, capture_output=True, text=True)
    exe = tmp_path / "abi_driver"
    subprocess.run([CLANG, "-fsanitize=address,undefined", str(drv), *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True, capture_output=True, text=True)
    # the HIP runtime's own allocations at exit are not this library's: leak checks off
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr[-3000:]
