"""kv_quant.h as a C header: a plain C99 program (tests/c_abi_host.c) compiles against it with
-std=c99 -pedantic -Werror, links against libkvq, and runs the host-only calls -- sizes and
handles from the storage format the header defines, geometry validation, the block allocator,
the width controller and the host-side argument checks of the device calls. The same source
also compiles as C++11 through the header's extern "C" guard. No GPU work."""
import os
import shutil
import subprocess

import pytest

import mixed_precision_quantized_kv_amd as kvq

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_host.c")
LIBDIR = os.path.dirname(kvq.LIB_PATH)


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built (run __graft_entry__.build())")


@pytest.mark.parametrize("lang", ["c99", "c++11"])
def test_c_client_compiles_links_and_passes(lang, tmp_path):
    cc = "gcc" if lang == "c99" else "g++"
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} not found")
    exe = str(tmp_path / "client")
    cmd = [cc, f"-std={lang}", "-pedantic", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include")]
    if lang != "c99":
        cmd += ["-x", "c++"]
    cmd += [SRC, "-o", exe, "-L", LIBDIR, "-lkvq", f"-Wl,-rpath,{LIBDIR}", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("0 failures"), r.stdout + r.stderr
