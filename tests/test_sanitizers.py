"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (oracle/kda_oracle.c) is compiled with the sanitizers into a
  small driver (tests/sanitize/oracle_driver.c) that runs forward and backward
  on packed cases with empty, one-token and ragged sequences, with and without
  states; the same inputs rerun through the normal build must give the same
  outputs.
* The C ABI's host validation (kda_api.cpp, host side sanitized, device side
  as usual) is linked with stub launchers and driven through every entry
  point with valid and invalid arguments (tests/sanitize/abi_driver.cpp).

The sanitizers apply to host code only: the GPU code is built as usual and
never runs here.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "gated_delta_rule_81_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{cmd[0]} failed ({res.returncode}):\n{res.stdout}\n{res.stderr}"
    return res


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-o", exe, os.path.join(SAN, "oracle_driver.c"), "-lm"])
    data = str(tmp_path / "cases.bin")
    _run([exe, data], env=ENV)
    buf = open(data, "rb").read()
    pos = 0

    def take(n, dtype):
        nonlocal pos
        a = np.frombuffer(buf, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    (n_cases,) = take(1, np.int64)
    assert n_cases == 3
    for _ in range(n_cases):
        N, H, dk, dv, T, has_s0, has_ds = (int(x) for x in take(7, np.int64))
        st = take(N + 1, np.int64)
        q, k = take(T * H * dk, np.float64), take(T * H * dk, np.float64)
        v, g = take(T * H * dv, np.float64), take(T * H * dk, np.float64)
        b, dout = take(T * H, np.float64), take(T * H * dv, np.float64)
        s0 = take(N * H * dv * dk, np.float64).reshape(N, H, dv, dk) if has_s0 else None
        ds = take(N * H * dv * dk, np.float64).reshape(N, H, dv, dk) if has_ds else None
        out, sT = take(T * H * dv, np.float64), take(N * H * dv * dk, np.float64)
        grads = [take(n, np.float64) for n in (T * H * dk, T * H * dk, T * H * dv, T * H * dk,
                                               T * H, N * H * dv * dk)]
        q3, k3 = q.reshape(T, H, dk), k.reshape(T, H, dk)
        v3, g3 = v.reshape(T, H, dv), g.reshape(T, H, dk)
        b2 = b.reshape(T, H)
        ref_out, ref_sT = oracle.kda_forward(q3, k3, v3, g3, b2, state0=s0, seq_start=st)
        assert np.array_equal(ref_out.ravel(), out) and np.array_equal(ref_sT.ravel(), sT)
        ref = oracle.kda_backward(q3, k3, v3, g3, b2, dout.reshape(T, H, dv), d_state=ds,
                                  state0=s0, seq_start=st)
        for got, key in zip(grads, ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dstate0")):
            assert np.array_equal(ref[key].ravel(), got), key
    assert pos == len(buf)


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0  # counts without initialising HIP
    except Exception:
        return False


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.skipif(_gpu_visible(), reason="runs on a host without a GPU (every call must stop "
                                           "at the device check; the launchers are stubs)")
def test_abi_validation_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api_o = str(tmp_path / "kda_api.o")
    # kda_api.cpp is HIP source (it holds the fixed scratch array): hipcc builds
    # it with the sanitizers on the host side only
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-x", "hip",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-omit-frame-pointer", *inc,
          "-c", os.path.join(CSRC, "kda_api.cpp"), "-o", api_o])
    exe = str(tmp_path / "abi_driver")
    # host-only sources and the link: plain host compiler
    _run(["/opt/rocm/llvm/bin/clang++", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", *inc,
          os.path.join(SAN, "abi_driver.cpp"), os.path.join(SAN, "launch_stubs.cpp"), api_o,
          "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe])
    res = _run([exe], env=ENV)
    assert "0 failures" in res.stdout
