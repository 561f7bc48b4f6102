"""Host-side checks of the C ABI: the library loads, exports every function
include/adasum.h declares, and rejects invalid arguments before any HIP call
(so these run without a GPU; no call here reaches a kernel)."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from distributed_sgd_gradient_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "adasum.h")

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"ADASUM_API\s+[\w\s\*]+?\b(adasum_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(_native.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _native.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _native.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (adasum_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_strerror():
    lib = _native.lib()
    assert lib.adasum_version() >= 100
    for code in (0, -1, -2, -3):
        assert lib.adasum_strerror(code)
    assert lib.adasum_strerror(-99) == b"unknown error code"


def _off(*vals):
    a = np.asarray(vals, dtype=np.int64)
    return a, a.ctypes.data_as(_native._I64P)


def _call_ex(K=2, off=(0, 8, 16), dtype=0, grads=None, out=FAKE + (1 << 30), ws=FAKE + (2 << 30),
             ws_bytes=1 << 20, coeffs=None, stats=None, ortho=None, schedule=0):
    lib = _native.lib()
    arr, p = _off(*off)
    if grads is None:
        grads = [FAKE + (k << 20) for k in range(K)]
    ptrs = (ctypes.c_void_p * max(len(grads), 1))(*grads)
    rc = lib.adasum_combine_ex(ptrs, K, p, arr.size - 1, dtype, schedule, out, ws, ws_bytes, coeffs, stats,
                               ortho, None)
    return rc, lib.adasum_last_error().decode()


@pytest.mark.parametrize("kwargs,needle", [
    (dict(K=0), "K must be >= 1"),
    (dict(dtype=7), "unknown dtype"),
    (dict(off=(1, 8, 16)), "seg_offsets[0] must be 0"),
    (dict(off=(0, 9, 8)), "non-decreasing"),
    (dict(out=None), "out is NULL"),
    (dict(out=FAKE + (1 << 30) + 4), "out must be 16-byte aligned"),
    (dict(grads=[FAKE, FAKE + 8]), "grads[1] must be 16-byte aligned"),
    (dict(grads=[FAKE, 0]), "grads[1] is NULL"),
    (dict(out=FAKE + 16), "overlaps input"),
    (dict(ws=None), "workspace is NULL"),
    (dict(ws_bytes=64), "workspace too small"),
    (dict(ws=FAKE + 32), "overlaps input"),
    (dict(coeffs=FAKE + (1 << 30) + 8), "overlaps"),
    (dict(ortho=FAKE + 32), "overlaps input"),
    (dict(schedule=5), "unknown schedule"),
    (dict(stats=FAKE + (3 << 30) + 4), "8-byte aligned"),
    (dict(ortho=FAKE + (3 << 30) + 2), "8-byte aligned"),
])
def test_invalid_arguments_rejected(kwargs, needle):
    rc, msg = _call_ex(**kwargs)
    assert rc == _native.EINVAL
    assert needle in msg


def test_negative_nseg_and_null_offsets():
    lib = _native.lib()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE + 4096)
    assert lib.adasum_combine(ptrs, 2, None, 1, 0, FAKE + 8192, None) == _native.EINVAL
    arr, p = _off(0)
    assert lib.adasum_combine(ptrs, 2, p, -1, 0, FAKE + 8192, None) == _native.EINVAL
    assert lib.adasum_workspace_bytes(2, p, -1, 0, 0) == _native.EINVAL
    assert lib.adasum_workspace_bytes(2, p, 0, 0, 9) == _native.EINVAL


def test_workspace_size_properties():
    lib = _native.lib()

    def ws(K, off, dtype=0, schedule=0):
        arr, p = _off(*off)
        return lib.adasum_workspace_bytes(K, p, arr.size - 1, dtype, schedule)

    n = 1 << 20
    assert 0 < ws(1, (0, 1000)) < 4096           # K = 1: one single-operand block
    # up to 16 operands form one block: no intermediates, only Gram partials
    # (with room for the low parts of an exact recomputation) and tables
    for K in (2, 3, 9, 16):
        assert 0 < ws(K, (0, n)) < 2 * n
    # 17 = a block of 16 (its result in one fp64 slot) and the carried input,
    # which the second stage reads where it is
    assert n * 8 <= ws(17, (0, n)) < 2 * n * 8
    assert 4 * n * 8 <= ws(64, (0, n)) < 5 * n * 8   # four blocks of 16
    assert ws(16, (0, 64 * n)) > ws(16, (0, n))
    assert ws(16, (0, 0)) >= 0 and ws(2, (0,)) >= 0
    # chain: 16 inputs, then the running result (an fp64 slot) and up to 15
    # more inputs, read where they are, per stage
    assert ws(16, (0, n), 0, 1) < 2 * n
    assert n * 8 <= ws(17, (0, n), 0, 1) < 2 * n * 8
    assert 4 * n * 8 <= ws(64, (0, n), 0, 1) < 5 * n * 8   # four stages below the root


def test_sum_entry_point_validation():
    lib = _native.lib()
    assert lib.adasum_sum_workspace_bytes(64, 1000, 0) == 0
    assert lib.adasum_sum_workspace_bytes(65, 1000, 0) == 8000   # fp64 running sum
    assert lib.adasum_sum_workspace_bytes(0, 1000, 0) == _native.EINVAL
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE + (1 << 20))
    assert lib.adasum_sum(ptrs, 2, 1000, 0, FAKE + 16, None, 0, None) == _native.EINVAL  # out overlaps grads[0]
    assert "overlaps" in lib.adasum_last_error().decode()
    assert lib.adasum_sum(ptrs, 2, 1000, 7, FAKE + (2 << 20), None, 0, None) == _native.EINVAL


def test_adasum_log_reports_the_plan():
    """ADASUM_LOG=1 prints one line per new plan (and per launch on a GPU)."""
    import subprocess
    import sys
    code = ("import ctypes, numpy as np\n"
            "from distributed_sgd_gradient_amd import _native\n"
            "off = np.array([0, 1000, 70000], dtype=np.int64)\n"
            "p = off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))\n"
            "print(_native.lib().adasum_workspace_bytes(70, p, 2, 2, 0))\n")
    env = dict(os.environ, ADASUM_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[adasum] plan K=70 nseg=2 N=70000" in r.stderr
    assert "2 stages" in r.stderr and int(r.stdout.strip()) > 0


def test_last_error_is_per_thread():
    """The message of a failure belongs to the thread that made the call."""
    import threading

    lib = _native.lib()
    arr, p = _off(0, 10, 5)
    assert lib.adasum_workspace_bytes(2, p, 2, 0, 0) == _native.EINVAL
    mine = lib.adasum_last_error().decode()
    assert "non-decreasing" in mine
    seen = {}

    def other():
        seen["fresh"] = lib.adasum_last_error().decode()
        a2, p2 = _off(0, 8)
        seen["rc"] = lib.adasum_workspace_bytes(0, p2, 1, 0, 0)
        seen["own"] = lib.adasum_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["fresh"] == ""
    assert seen["rc"] == _native.EINVAL and "K must be >= 1" in seen["own"]
    assert lib.adasum_last_error().decode() == mine


def test_package_fails_loudly_without_the_library(tmp_path):
    """No fallback: the package's Python files without libadasum.so refuse to import."""
    import shutil
    import sys

    pkg = os.path.join(ROOT, "distributed_sgd_gradient_amd")
    dst = tmp_path / "distributed_sgd_gradient_amd"
    dst.mkdir()
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            shutil.copy(os.path.join(pkg, name), dst / name)
    res = subprocess.run([sys.executable, "-c", "import distributed_sgd_gradient_amd"], cwd=tmp_path,
                         capture_output=True, text=True, env=dict(os.environ, PYTHONPATH=str(tmp_path)))
    assert res.returncode != 0
    assert "libadasum.so is missing" in res.stderr


def test_k_times_nseg_bound():
    """One tree-walk workgroup per (block, segment): K * nseg must fit a launch grid."""
    lib = _native.lib()
    nseg = (1 << 31) // 1000 + 1
    arr = np.zeros(nseg + 1, dtype=np.int64)  # all segments empty
    p = arr.ctypes.data_as(_native._I64P)
    assert lib.adasum_workspace_bytes(1000, p, nseg, 0, 0) == _native.EINVAL
    assert "exceeds 2^31 - 1" in lib.adasum_last_error().decode()
    assert lib.adasum_workspace_bytes(999, p, nseg - 10, 0, 0) > 0


def _call_noalloc(K=2, off=(0, 8, 16), dtype=0, grads=None, out=FAKE + (1 << 30), coeffs=None, schedule=0):
    lib = _native.lib()
    arr, p = _off(*off)
    if grads is None:
        grads = [FAKE + (k << 20) for k in range(K)]
    ptrs = (ctypes.c_void_p * max(len(grads), 1))(*grads)
    rc = lib.adasum_combine_noalloc(ptrs, K, p, arr.size - 1, dtype, schedule, out, coeffs, None, None, None)
    return rc, lib.adasum_last_error().decode()


@pytest.mark.parametrize("kwargs,needle", [
    (dict(K=0), "K must be >= 1"),
    (dict(out=None), "out is NULL"),
    (dict(out=FAKE + 16), "overlaps input"),
    (dict(grads=[FAKE, 0]), "grads[1] is NULL"),
    (dict(coeffs=FAKE + (1 << 30) + 8), "overlaps"),
    # 40 fp32 inputs of 2^24 elements: fp32 slots of the second stage alone
    # need far more than the fixed scratch array holds
    (dict(K=40, off=(0, 1 << 24)), "bytes of scratch"),
])
def test_noalloc_rejects_before_any_launch(kwargs, needle):
    """The no-allocation entry point validates like adasum_combine_ex and
    refuses shapes whose workspace and tables exceed its fixed array."""
    rc, msg = _call_noalloc(**kwargs)
    assert rc == _native.EINVAL and needle in msg, msg
