"""Address and undefined-behaviour sanitizers on the CPU code.

- The oracle (oracle/ibp_oracle.c) built with gcc -fsanitize=address,undefined
  together with tests/helpers/oracle_sanitize_main.c, which runs every oracle
  function on small inputs in exactly sized heap buffers and checks the round
  trip.
- The C ABI's host code (api.hip: argument checks, error reporting, the
  device and symbol lookups) built with the same sanitizers on its host side
  only, linked with the library's kernel objects and
  tests/helpers/abi_sanitize_main.c, which calls every entry point with
  arguments each check must reject, then valid calls that enqueue nothing
  (IBP_ERR_HIP with no GPU).  Skipped where a GPU is visible: those calls are
  for a machine without one.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr[-4000:]}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-fopenmp",
          os.path.join(ROOT, "oracle", "ibp_oracle.c"),
          os.path.join(ROOT, "tests", "helpers", "oracle_sanitize_main.c"), "-o", exe, "-lm"])
    r = _run([exe], env=dict(ENV, OMP_NUM_THREADS="4"), timeout=300)
    assert "oracle sanitizer run ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr


def test_abi_host_code_under_asan_ubsan(tmp_path):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("the no-device calls need a machine without a GPU")
    build = os.path.join(ROOT, "host_transfer_amd", "_build")
    objs = [os.path.join(build, f + ".hip.o") for f in ("compress", "gather", "gather_cache",
                                                         "meta", "probe")]
    if not all(os.path.exists(o) for o in objs):
        from host_transfer_amd.csrc import build as hb
        hb.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api = str(tmp_path / "api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang",
          "-target-feature", "-Xclang", "-packed-fp32-ops"] + san +
         ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "host_transfer_amd", "csrc"),
          "-c", os.path.join(ROOT, "host_transfer_amd", "csrc", "api.hip"), "-o", api])
    drv = str(tmp_path / "abi_main.o")
    _run([HIPCC, "-x", "c", "-O1", "-g"] + san + ["-I", os.path.join(ROOT, "include"), "-c",
         os.path.join(ROOT, "tests", "helpers", "abi_sanitize_main.c"), "-o", drv])
    exe = str(tmp_path / "abi_san")
    _run([HIPCC, "--offload-arch=gfx950"] + san[:4] + ["-o", exe, drv, api] + objs)
    r = _run([exe, "no-device"], env=ENV, timeout=120)
    assert "abi sanitizer run ok" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
