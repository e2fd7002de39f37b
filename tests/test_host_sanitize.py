"""The C ABI's host layer (argument checks, launch plans, segment groups, workspace
arithmetic) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/host_sanitize/driver.cpp on the CPU.  Only the host part of the API source is
instrumented (each sanitizer flag follows -Xarch_host); the kernels' objects are the
regular build's; the executable is linked by g++.  With no GPU present, calls that
reach a launch return CPATTN_ERR_HIP, which the driver accepts."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "context_causal_attention_zigzag_amd")
HIPCC = "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc and g++")
def test_host_layer_under_sanitizers(tmp_path):
    objdir = os.path.join(PKG, "_build")
    kernels = ["fwd.hip.o", "bwd.hip.o", "merge.hip.o", "partition.hip.o"]
    if not all(os.path.exists(os.path.join(objdir, o)) for o in kernels):
        import importlib.util
        spec = importlib.util.spec_from_file_location("cpattn_build", os.path.join(PKG, "_build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    api_o = str(tmp_path / "api_san.o")
    drv_o = str(tmp_path / "driver.o")
    exe = str(tmp_path / "driver")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    base = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    r = subprocess.run(base + san + ["-c", os.path.join(PKG, "csrc", "api.hip"), "-o", api_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"),
                        "-o", drv_o], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run(["g++", "-fsanitize=address,undefined", drv_o, api_o] +
                       [os.path.join(objdir, o) for o in kernels] +
                       ["-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64", "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0 and "host driver: ok" in out, out[-4000:]
