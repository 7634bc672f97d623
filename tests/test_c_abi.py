"""The boundary used from C and C++ with no Python in between: a program
that includes include/dsa_indexer.h, links libdsa_indexer.so and calls the
host-only entry points and argument checks (tests/c/abi_from_c.c), built as
strict C99 and as C++17 so the header stays valid in both languages; and a
host-side fuzz of every size query, host rule and argument check with
extreme, negative and NaN arguments (tests/c/host_fuzz.c), which must
neither crash nor break the documented results."""

import os
import shutil
import subprocess

import pytest

from dsa_lightning_indexer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_from_c.c")
FUZZ = os.path.join(ROOT, "tests", "c", "host_fuzz.c")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="library not built")


@pytest.mark.parametrize("compiler,flags", [
    ("gcc", ["-std=c99", "-pedantic"]),
    ("g++", ["-x", "c++", "-std=c++17", "-pedantic"]),
])
def test_header_and_library_from_c(tmp_path, compiler, flags):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = [compiler, *flags, "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), SRC,
           "-x", "none", "-L", libdir, "-l:libdsa_indexer.so",
           f"-Wl,-rpath,{libdir}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "c abi ok"


def test_host_fuzz(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    libdir = os.path.dirname(binding.LIB_PATH)
    exe = str(tmp_path / "host_fuzz")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), FUZZ, "-L", libdir,
           "-l:libdsa_indexer.so", "-lm", f"-Wl,-rpath,{libdir}", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "host fuzz ok"
