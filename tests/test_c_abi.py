"""The C ABI from C: tests/c_abi/abi_smoke.c is compiled with gcc against
include/gdn_replay.h, linked with the built library and run (host-side
validation only, so no GPU is needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gated_deltanet_state_replayssm_amd")
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_smoke.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_caller_links_and_validates(tmp_path):
    lib = os.path.join(PKG, "libgdnreplay.so")
    assert os.path.exists(lib), "build the library first (gated_deltanet_state_replayssm_amd.build)"
    exe = str(tmp_path / "abi_smoke")
    # the HIP runtime header needs the platform macro when a plain C compiler reads it
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", PKG, "-lgdnreplay", f"-Wl,-rpath,{PKG}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr


STUBS = os.path.join(ROOT, "tests", "c_abi", "launch_stubs.cpp")
API = os.path.join(PKG, "csrc", "api.cpp")


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="gcc / g++ not found")
def test_host_layer_under_address_and_ub_sanitizers(tmp_path):
    """The C-ABI layer (csrc/api.cpp: validation and dispatch) built for the
    host alone with AddressSanitizer and UBSan, the kernel launchers replaced by
    stubs that abort (tests/c_abi/launch_stubs.cpp), driven by the same plain C
    caller: every call must be refused or launch nothing, with no memory or
    undefined-behaviour error in the host code."""
    san = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]
    inc = ["-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include")]
    objs = []
    for src, cc, std in ((API, "g++", "-std=c++17"), (STUBS, "g++", "-std=c++17"),
                         (SRC, "gcc", "-std=c11")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([cc, std, "-g", "-O1", "-Wall", "-Werror", *san, *inc, "-c", src,
                            "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        objs.append(obj)
    exe = str(tmp_path / "abi_asan")
    r = subprocess.run(["g++", *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip() == "OK", r.stdout + r.stderr
