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
