"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer:
  * the oracle (oracle/kvarn_oracle.c, gcc) driven through every function on
    small inputs and edge cases by oracle/sanitize_check.c;
  * libkvarn's C-ABI layer (kvarn_api.hip) compiled for the host alone, its
    launchers replaced by recording stubs (tests/native/kvarn_api_host_check.cpp),
    so every validation path and the launch arguments run without a GPU.
The sanitizers abort on their first finding; a zero exit status means none."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
          "-Werror", os.path.join(ROOT, "oracle", "kvarn_oracle.c"),
          os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm", "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert "oracle sanitize check ok" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not found")
def test_abi_layer_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    csrc = os.path.join(ROOT, "kv_cache_bit_kvarn_amd", "csrc")
    # host code only; the sanitizer flags apply to the host compilation
    san = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined".split()
    _run([HIPCC, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g",
          "-fno-omit-frame-pointer", *san, "-fno-sanitize-recover=all", "-Wall",
          "-I", os.path.join(ROOT, "include"), "-I", csrc,
          os.path.join(csrc, "kvarn_api.hip"),
          os.path.join(ROOT, "tests", "native", "kvarn_api_host_check.cpp"), "-o", exe])
    r = _run([exe], env=SAN_ENV)
    assert "kvarn_api host check ok" in r.stdout
