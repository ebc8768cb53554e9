"""CPU: include/repops.h is a plain C header.

tests/c_abi_consumer.c is compiled as C99 and as C++17, with warnings as
errors, linked against the built librepops.so and run. It checks that a C
program can call the library with no Python or torch in between. Only entry
points that touch no device are called, so no GPU is needed."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi_consumer.c")
INC = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "bit_reproducible_fp32_amd")


def _gpu_initialised():
    import sys
    torch = sys.modules.get("torch")
    return torch is not None and getattr(torch.cuda, "is_initialized", lambda: False)()


@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_c_program_links_and_runs(lang, tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "librepops.so")):
        pytest.skip("librepops.so is not built")
    if _gpu_initialised():
        pytest.skip("no child processes from a process that has initialised the GPU")
    cc = "gcc" if lang == "c99" else "g++"
    if shutil.which(cc) is None:
        pytest.skip("%s not installed" % cc)
    exe = str(tmp_path / ("consumer_" + lang.replace("+", "p")))
    cmd = [cc, "-x", "c" if lang == "c99" else "c++", "-std=" + lang, "-Wall", "-Wextra",
           "-Werror", "-pedantic", "-I", INC, SRC, "-x", "none", "-L", LIBDIR, "-lrepops",
           "-Wl,-rpath," + LIBDIR, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c consumer ok" in r.stdout
