"""The C ABI from plain C: tests/c/abi_host.c is compiled as C99 by gcc against
include/kda.h, linked to the built libkda.so, and run on the host (no GPU: every call it makes
is answered before any device work)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "gated_delta_rule_59_amd")
ROCM_LIB = "/opt/rocm/lib"


def test_c_client_links_and_validates(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libkda.so")):
        pytest.skip("libkda not built")
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    exe = tmp_path / "abi_host"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host.c"),
                    "-L", LIBDIR, "-lkda", f"-Wl,-rpath,{LIBDIR}:{ROCM_LIB}", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")


def test_walk_shape_never_splits_an_in_place_walk(tmp_path):
    """The matrix-core walk's launch shape (kda_plan.h), checked on the host: two workgroups
    per walk only when the walks leave half of the CUs idle, and never when S_T is the S0
    buffer (the second workgroup reads S0 when it starts, possibly after the first stored
    S_T)."""
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = tmp_path / "plan_check"
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                    "-I", os.path.join(ROOT, "gated_delta_rule_59_amd", "csrc"),
                    os.path.join(ROOT, "tests", "c", "plan_check.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"
