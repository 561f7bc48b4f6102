"""The no-allocation entry point against adasum_combine_ex (GPU).

adasum_combine_noalloc runs the same kernels with its workspace and tables in
a fixed device array; its output, coefficients, statistics and orthogonality
ratios must equal those of adasum_combine_ex bit for bit, on two calls in a
row, the second with a smaller input of another dtype and schedule (the array
keeps the first call's contents), then on a 64-operand block and on a chain
whose second stage reads an fp64 slot, over a segment long enough for the
walk to read tile groups.
"""

import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from parity import say

pytestmark = pytest.mark.gpu


def _noalloc(grads, off, dtype_code, schedule):
    from distributed_sgd_gradient_amd import _native
    lib = _native.lib()
    g0 = grads[0]
    K, nseg = len(grads), off.size - 1
    out = torch.empty_like(g0)
    coeffs = torch.empty((max(K - 1, 0), nseg, 2), dtype=torch.float64, device=g0.device)
    stats = torch.empty((max(K - 1, 0), nseg, 3), dtype=torch.float64, device=g0.device)
    ortho = torch.empty((nseg,), dtype=torch.float64, device=g0.device)
    ptrs = (ctypes.c_void_p * K)(*[g.data_ptr() for g in grads])
    st = ctypes.c_void_p(torch.cuda.current_stream(g0.device).cuda_stream)
    rc = lib.adasum_combine_noalloc(ptrs, K, off.ctypes.data_as(_native._I64P), nseg, dtype_code, schedule,
                                    out.data_ptr(), coeffs.data_ptr(), stats.data_ptr(), ortho.data_ptr(), st)
    _native.check(rc)
    return out, coeffs, stats, ortho


CASES = [
    # (K, dtype, schedule, lengths): the first call is the larger one
    (16, "f32", "tree", [70000, 3, 0, 12345, 200000, 8191]),
    (5, "bf16", "chain", [1000, 7, 300]),
    (40, "f16", "tree", [20000, 1, 257, 9]),
    (20, "f32", "chain", [300000, 5]),
]


def test_noalloc_matches_combine_ex(gpu):
    import distributed_sgd_gradient_amd as A
    from distributed_sgd_gradient_amd import _native
    codes = {"f32": _native.F32, "f16": _native.F16, "bf16": _native.BF16}
    scheds = {"tree": _native.TREE, "chain": _native.CHAIN}
    for i, (K, dtype, schedule, lengths) in enumerate(CASES):
        say(f"noalloc call {i}: K={K} {dtype} {schedule} lengths={lengths}")
        wl = W.random_case(K, lengths, dtype=dtype, seed=600 + i, kind="shared")
        grads = [g.to(gpu) for g in wl.grads]
        off = np.ascontiguousarray(wl.seg_offsets, dtype=np.int64)
        got = _noalloc(grads, off, codes[dtype], scheds[schedule])
        ref = A.combine(grads, off, schedule=schedule, return_coeffs=True, return_stats=True, return_ortho=True)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), f"call {i}: output differs"
        assert torch.equal(got[1], ref[1]), f"call {i}: coefficients differ"
        assert torch.equal(got[2], ref[2]), f"call {i}: statistics differ"
        assert torch.equal(torch.nan_to_num(got[3], nan=-1.0), torch.nan_to_num(ref[3], nan=-1.0)), f"call {i}"


def test_noalloc_refuses_graph_capture(gpu):
    """Its tables come from host memory on every call, so a call under
    stream capture is refused before anything is enqueued."""
    from distributed_sgd_gradient_amd import _native
    lib = _native.lib()
    wl = W.random_case(3, [500, 9], dtype="f32", seed=640, kind="shared")
    grads = [g.to(gpu) for g in wl.grads]
    off = np.ascontiguousarray(wl.seg_offsets, dtype=np.int64)
    out = torch.empty_like(grads[0])
    ptrs = (ctypes.c_void_p * 3)(*[g.data_ptr() for g in grads])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out.zero_()
        st = ctypes.c_void_p(torch.cuda.current_stream(gpu).cuda_stream)
        rc = lib.adasum_combine_noalloc(ptrs, 3, off.ctypes.data_as(_native._I64P), off.size - 1, _native.F32,
                                        _native.TREE, out.data_ptr(), None, None, None, st)
        msg = lib.adasum_last_error().decode()
    torch.cuda.synchronize()
    assert rc == _native.EINVAL and "cannot be captured" in msg, msg
