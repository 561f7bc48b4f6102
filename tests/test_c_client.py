"""The C ABI used from plain C, without Python in the process.

tests/abi_client.c allocates device memory with the HIP runtime API, calls the
entry points declared in include/adasum.h and checks closed-form results
(orthogonal gradients are summed, equal gradients are returned unchanged,
integer sums are exact, K = 1 copies, invalid arguments are rejected).  The CPU
tests check that the header is valid C and C++ and that the client compiles
and links against the built library; the GPU test runs it.
"""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT, flush_print

INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "distributed_sgd_gradient_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _need(tool):
    path = shutil.which(tool)
    if path is None:
        pytest.skip(f"{tool} not found")
    return path


def _build_client(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libadasum.so")):
        pytest.skip("libadasum.so not built")
    exe = str(tmp_path / "abi_client")
    cmd = [_need("gcc"), "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", INCLUDE, os.path.join(ROOT, "tests", "abi_client.c"),
           "-L", PKG, "-ladasum", "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("gcc", "-std=c11"), ("g++", "-std=c++17")])
def test_header_is_valid_c_and_cpp(tmp_path, compiler, std):
    src = tmp_path / ("h.cpp" if compiler == "g++" else "h.c")
    src.write_text('#include "adasum.h"\nint main(void) { return adasum_version() > 0 ? 0 : 1; }\n')
    res = subprocess.run([_need(compiler), std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                          "-I", INCLUDE, str(src)], capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr


def test_client_compiles_and_links(tmp_path):
    exe = _build_client(tmp_path)
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
def test_client_runs_on_gpu(gpu, tmp_path):
    exe = _build_client(tmp_path)
    flush_print("running tests/abi_client.c")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    flush_print(res.stdout[-4000:])
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-2000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.startswith(("ok", "FAIL"))]
    assert len(lines) >= 30 and all(ln.startswith("ok") for ln in lines)
