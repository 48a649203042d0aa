"""The C header as C: ``tests/c_abi/abi_errors.c`` includes ``include/ddtree.h``, is compiled with
the C compiler (C11, warnings as errors, pedantic), links ``libddtree.so`` and calls every entry
point with invalid arguments, checking the documented DDTREE_ERR_* codes.  Host-side validation
reads no device memory, so this runs without a GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_errors.c")
LIBDIR = os.path.join(ROOT, "tree_verify_mla_absorb_amd")
ROCM_INCLUDE = "/opt/rocm/include"


def test_header_compiles_as_c_and_entry_points_reject_invalid_arguments(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(os.path.join(LIBDIR, "libddtree.so")):
        pytest.fail("libddtree.so is not built")
    exe = str(tmp_path / "abi_errors")
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-isystem", ROCM_INCLUDE, SRC, "-L", LIBDIR, "-lddtree",
           f"-Wl,-rpath,{LIBDIR}", "-o", exe]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
    assert r.returncode == 0, r.stdout
    assert ", 0 failed" in r.stdout
