"""Python front end of the Adasum combiner: torch tensors in, torch tensor out.

Only argument marshalling happens here: the tensors' device pointers, the
segment offsets and the current HIP stream are handed to the C ABI, and every
step of the combine runs in the library's gfx950 kernels.  torch provides the
device memory (output, workspace, statistics) and the stream.
"""

import ctypes

import numpy as np
import torch

from . import _native

_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_raw_stream(index):
    """Handle of the current stream of device ``index``."""
    if _raw_stream is not None:
        return _raw_stream(index)
    return torch.cuda.current_stream(index).cuda_stream

DTYPE_CODES = {torch.float32: _native.F32, torch.float16: _native.F16, torch.bfloat16: _native.BF16}
SCHEDULES = {"tree": _native.TREE, "chain": _native.CHAIN}


def _offsets(seg_offsets, N=None):
    off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
    if off.ndim != 1 or off.size < 1:
        raise ValueError("seg_offsets must be a 1-D sequence of nseg + 1 offsets")
    if N is not None and int(off[-1]) != N:
        raise ValueError(f"seg_offsets[-1] = {int(off[-1])} but the gradients hold {N} elements")
    return off


def _grad_list(grads):
    if isinstance(grads, torch.Tensor):
        if grads.dim() != 2:
            raise ValueError("a tensor of gradients must be 2-D [K, N]")
        grads = list(grads.unbind(0))
    grads = list(grads)
    if not grads:
        raise ValueError("need at least one gradient")
    g0 = grads[0]
    for g in grads:
        if not isinstance(g, torch.Tensor) or g.device != g0.device or g.dtype != g0.dtype:
            raise ValueError("all gradients must be tensors of one dtype on one device")
        if g.dim() != 1 or g.numel() != g0.numel() or not g.is_contiguous():
            raise ValueError("all gradients must be contiguous 1-D tensors of equal length")
    if g0.device.type != "cuda":
        raise ValueError("gradients must be on a GPU")
    if g0.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {g0.dtype}")
    return grads


def workspace_bytes(K, seg_offsets, dtype, schedule="tree"):
    off = _offsets(seg_offsets)
    code = DTYPE_CODES[dtype]
    L = _native.lib()
    return _native.check(L.adasum_workspace_bytes(
        K, off.ctypes.data_as(_native._I64P), off.size - 1, code, SCHEDULES[schedule]))


def _check_out(out, g0):
    if out is None:
        return torch.empty_like(g0)
    if out.device != g0.device or out.dtype != g0.dtype or out.numel() != g0.numel() or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like the gradients")
    return out


def combine(grads, seg_offsets, *, schedule="tree", out=None, workspace=None, return_coeffs=False,
            return_stats=False, return_ortho=False, stream=None):
    """Adasum of K gradients, each segment on its own.

    grads: list of K contiguous 1-D GPU tensors (fp32 / fp16 / bf16), or one
      [K, N] tensor.  seg_offsets: nseg + 1 CSR offsets (host).  schedule:
      "tree" (pairs level by level) or "chain" (left-to-right recursion).
      Returns the combined gradient (same dtype), followed, when requested,
      by the fp64 coefficient table [K-1, nseg, 2], the statistics table
      [K-1, nseg, 3] and the per-segment orthogonality ratio [nseg].
    """
    grads = _grad_list(grads)
    g0 = grads[0]
    off = _offsets(seg_offsets, g0.numel())
    K, nseg = len(grads), off.size - 1
    dev = g0.device
    out = _check_out(out, g0)
    need = workspace_bytes(K, off, g0.dtype, schedule)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the gradients' device")
    coeffs = torch.empty((max(K - 1, 0), nseg, 2), dtype=torch.float64, device=dev) if return_coeffs else None
    stats = torch.empty((max(K - 1, 0), nseg, 3), dtype=torch.float64, device=dev) if return_stats else None
    ortho = torch.empty((nseg,), dtype=torch.float64, device=dev) if return_ortho else None
    ptrs = (ctypes.c_void_p * K)(*[g.data_ptr() for g in grads])
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    L = _native.lib()
    with torch.cuda.device(dev):
        _native.check(L.adasum_combine_ex(
            ptrs, K, off.ctypes.data_as(_native._I64P), nseg, DTYPE_CODES[g0.dtype], SCHEDULES[schedule],
            out.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            coeffs.data_ptr() if coeffs is not None else None,
            stats.data_ptr() if stats is not None else None,
            ortho.data_ptr() if ortho is not None else None,
            ctypes.c_void_p(stream.cuda_stream)))
    extra = [t for t, want in ((coeffs, return_coeffs), (stats, return_stats), (ortho, return_ortho)) if want]
    return tuple([out] + extra) if extra else out


def plain_sum(grads, *, out=None, workspace=None, stream=None):
    """Synchronous-SGD combination: the element-wise sum of the K gradients,
    accumulated in fp64 in worker order and rounded once."""
    grads = _grad_list(grads)
    g0 = grads[0]
    K, N, dev = len(grads), g0.numel(), g0.device
    out = _check_out(out, g0)
    L = _native.lib()
    need = _native.check(L.adasum_sum_workspace_bytes(K, N, DTYPE_CODES[g0.dtype]))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the gradients' device")
    ptrs = (ctypes.c_void_p * K)(*[g.data_ptr() for g in grads])
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    with torch.cuda.device(dev):
        _native.check(L.adasum_sum(ptrs, K, N, DTYPE_CODES[g0.dtype], out.data_ptr(),
                                   workspace.data_ptr() if workspace is not None else None,
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   ctypes.c_void_p(stream.cuda_stream)))
    return out


def combine_cached(grads, seg_offsets, *, out=None, stream=None):
    """Like :func:`combine` but through ``adasum_combine``, whose workspace the
    library allocates and caches per (device, stream)."""
    grads = _grad_list(grads)
    g0 = grads[0]
    off = _offsets(seg_offsets, g0.numel())
    out = _check_out(out, g0)
    ptrs = (ctypes.c_void_p * len(grads))(*[g.data_ptr() for g in grads])
    if stream is None:
        stream = torch.cuda.current_stream(g0.device)
    L = _native.lib()
    with torch.cuda.device(g0.device):
        _native.check(L.adasum_combine(ptrs, len(grads), off.ctypes.data_as(_native._I64P), off.size - 1,
                                       DTYPE_CODES[g0.dtype], out.data_ptr(),
                                       ctypes.c_void_p(stream.cuda_stream)))
    return out


class Combiner:
    """A combine whose arguments are marshalled once: for calling Adasum on
    the same gradient buffers every step (their contents may change between
    calls, their storage may not).  Each call enqueues one combine on the
    given (else the current) stream and returns ``out``; the coefficient,
    statistic and orthogonality tables, when requested, are the attributes
    ``coeffs``, ``stats`` and ``ortho``, overwritten by every call.
    """

    def __init__(self, grads, seg_offsets, *, schedule="tree", out=None, return_coeffs=False, return_stats=False,
                 return_ortho=False):
        self.grads = _grad_list(grads)  # kept alive for the pointers below
        g0 = self.grads[0]
        self._off = _offsets(seg_offsets, g0.numel())
        K, nseg = len(self.grads), self._off.size - 1
        self.device = dev = g0.device
        self.out = _check_out(out, g0)
        need = workspace_bytes(K, self._off, g0.dtype, schedule)
        self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        self.coeffs = torch.empty((max(K - 1, 0), nseg, 2), dtype=torch.float64, device=dev) if return_coeffs else None
        self.stats = torch.empty((max(K - 1, 0), nseg, 3), dtype=torch.float64, device=dev) if return_stats else None
        self.ortho = torch.empty((nseg,), dtype=torch.float64, device=dev) if return_ortho else None
        self._ptrs = (ctypes.c_void_p * K)(*[g.data_ptr() for g in self.grads])
        self._args = (self._ptrs, K, self._off.ctypes.data_as(_native._I64P), nseg, DTYPE_CODES[g0.dtype],
                      SCHEDULES[schedule], self.out.data_ptr(), self._ws.data_ptr(), self._ws.numel(),
                      self.coeffs.data_ptr() if self.coeffs is not None else None,
                      self.stats.data_ptr() if self.stats is not None else None,
                      self.ortho.data_ptr() if self.ortho is not None else None)
        self._fn = _native.lib().adasum_combine_ex
        self._index = dev.index if dev.index is not None else torch.cuda.current_device()

    def __call__(self, stream=None):
        # the stream as a raw handle: torch's current-stream object costs
        # more host time than a small combine's launches
        st = _current_raw_stream(self._index) if stream is None else stream.cuda_stream
        if torch.cuda.current_device() == self._index:
            _native.check(self._fn(*self._args, st))
        else:
            with torch.cuda.device(self.device):
                _native.check(self._fn(*self._args, st))
        return self.out
