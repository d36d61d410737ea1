"""The host side of libtlg (plan validation, variant choice, plan geometry and
lifetime, the no-alloc entry point's refusals) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the host pass only, and exercised by a small C++
program that makes no device call.  CPU only."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_host_logic_under_asan(tmp_path):
    exe = tmp_path / "asan_host"
    api = os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", "tlg_api.cpp")
    main = os.path.join(ROOT, "tests", "host", "asan_host.cpp")
    # The kernels' launchers are not needed for host-only calls: a stub unit provides them.
    stub = tmp_path / "stubs.cpp"
    stub.write_text(STUBS)
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-x", "hip", api, str(stub), "-x", "c++", main,
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout[-3000:] + run.stderr[-3000:]
    assert "0 failures" in run.stdout


STUBS = r"""
#include <hip/hip_runtime_api.h>
#include "%s"
namespace tlg {
#define STUB(name) hipError_t name(const GemmParams&, int, int, hipStream_t) { return hipErrorInvalidValue; }
STUB(launch_lds_f16) STUB(launch_lds_bf16) STUB(launch_lds128_f16) STUB(launch_lds128_bf16)
STUB(launch_lds128sk_f16) STUB(launch_lds128sk_bf16) STUB(launch_lds64_f16) STUB(launch_lds64_bf16)
STUB(launch_lds32_f16) STUB(launch_lds32_bf16)
STUB(launch_lds_sk2_f16) STUB(launch_lds_sk2_bf16) STUB(launch_lds128_sk2_f16) STUB(launch_lds128_sk2_bf16)
#define STUB6(name) hipError_t name(const GemmParams&, int, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
STUB6(launch_tile_256_f16) STUB6(launch_tile_256_bf16) STUB6(launch_tile_256w8_f16) STUB6(launch_tile_256w8_bf16)
STUB6(launch_tile_128_f16) STUB6(launch_tile_128_bf16)
hipError_t launch_skinny(const GemmParams&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mx(const MxParams&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_attn(const AttnParams&, int, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_w4(const W4Params&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_sp(const SpParams&, int, hipStream_t) { return hipErrorInvalidValue; }
}
""" % os.path.join(ROOT, "tiled_dense_gemm_02_amd", "csrc", "tlg_internal.h")
