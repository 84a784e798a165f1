"""The CPU oracle and the C ABI's host-side argument checks, built with
AddressSanitizer and UndefinedBehaviorSanitizer and run on the host.

* oracle: tests/sanitize/oracle_driver.c linked with oracle/gdn_oracle.c by gcc
  (-fsanitize=address,undefined, every report fatal).  It calls every oracle entry
  point on small inputs, odd lengths and argument errors.
* ABI: tests/sanitize/abi_driver.cpp linked with gdn_abi.hip, whose host code is
  built with the sanitizers by hipcc (the flags apply to the host compilation only;
  the device code of the library is not instrumented), and with the library's
  other objects as built by gated_deltanet_mixer_amd/build.py.  Every call it makes
  is rejected by a host check before any HIP call, so no GPU is needed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "gdn_oracle.c"),
          "-lm", "-o", exe], timeout=300)
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "all passed" in r.stdout


def test_abi_host_checks_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    build = os.path.join(ROOT, "_build")
    others = [os.path.join(build, f) for f in ("gdn_decode.o", "gdn_prefill.o", "gdn_pass.o")]
    if not all(os.path.exists(o) for o in others):
        import __graft_entry__
        __graft_entry__.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gated_deltanet_mixer_amd", "csrc")]
    abi_o = str(tmp_path / "gdn_abi_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", *san, *inc, "-c", os.path.join(ROOT, "gated_deltanet_mixer_amd", "csrc", "gdn_abi.hip"),
          "-o", abi_o], timeout=600)
    drv_o = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *san, *inc, "-c",
          os.path.join(HERE, "abi_driver.cpp"), "-o", drv_o], timeout=600)
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950", *san, drv_o, abi_o, *others, "-o", exe], timeout=600)
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "all passed" in r.stdout
