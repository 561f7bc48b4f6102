"""Seeded value generators for the synthetic workloads.

Values are drawn with torch generators on the requested device (the GPU for
full-size workloads, the CPU for small tests), one worker at a time so a
workload never needs more than a few fp32 temporaries of length N beside its
K output buffers.  Each worker buffer is its own allocation, so every base
pointer is at least 256-byte aligned.

Per-segment parameters (scales, cosines, zero flags) are drawn with NumPy from
the workload seed before any subsetting, so a subset of segments keeps the
parameters those segments have in the full workload.
"""

from dataclasses import dataclass, field

import numpy as np
import torch

from .shapes import CONFIGS, config_offsets, offsets_from_lengths

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    K: int
    dtype: str
    seg_offsets: np.ndarray
    grads: list
    config: int = None
    seed: int = None
    notes: dict = field(default_factory=dict)

    @property
    def N(self):
        return int(self.seg_offsets[-1])

    @property
    def nseg(self):
        return int(self.seg_offsets.size - 1)

    def segment_host(self, s):
        """fp64 host copies of segment s of every worker (exact widening)."""
        lo, hi = int(self.seg_offsets[s]), int(self.seg_offsets[s + 1])
        return [g[lo:hi].to(torch.float64).cpu().numpy() for g in self.grads]


def _seed(*key):
    return int(np.random.SeedSequence([int(k) for k in key]).generate_state(1, np.uint64)[0])


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*key))
    return g


def _expand(per_segment, lengths, device):
    vals = torch.as_tensor(per_segment, dtype=torch.float32, device=device)
    reps = torch.as_tensor(lengths, dtype=torch.int64, device=device)
    return torch.repeat_interleave(vals, reps)


def segment_params(config, seed, nseg, K):
    """Per-segment parameters of workload ``config`` drawn from its seed."""
    rng = np.random.default_rng(np.random.SeedSequence([config, seed, 1]))
    params = {}
    if config == 4:
        params["scale"] = np.exp(rng.uniform(np.log(1e-6), 0.0, size=nseg))
    if config == 5:
        params["cosine"] = rng.uniform(-1.0, 1.0, size=nseg)
        flagged = rng.random(nseg) < 0.05
        zero = np.zeros((K, nseg), dtype=bool)
        for s in np.flatnonzero(flagged):
            while True:
                z = rng.random(K) < 0.5
                if z.any():
                    break
            zero[:, s] = z
        params["zero"] = zero
    return params


def make_workload(config, seed=None, device="cpu", segments=None):
    """Build workload ``config`` (1..5) with K worker buffers on ``device``.

    ``segments`` optionally selects a subset of segment ids; the result then
    holds only those segments (concatenated in the given order) with their
    full-workload parameters and freshly drawn values.
    """
    K, dtype, _ = CONFIGS[config]
    seed = config if seed is None else int(seed)
    full_off = config_offsets(config, seed)
    lengths = np.diff(full_off)
    params = segment_params(config, seed, lengths.size, K)
    if segments is not None:
        segments = np.asarray(segments, dtype=np.int64)
        lengths = lengths[segments]
        params = {k: (v[:, segments] if v.ndim == 2 else v[segments]) for k, v in params.items()}
    off = offsets_from_lengths(lengths)
    N = int(off[-1])
    tdt = TORCH_DTYPES[dtype]

    shared = None
    if config in (2, 5):
        shared = torch.randn(N, generator=_gen(device, config, seed, 2, 0),
                             device=device, dtype=torch.float32)
    if config == 5:
        cos = _expand(params["cosine"], lengths, device)
        sin = torch.sqrt(torch.clamp(1.0 - cos * cos, min=0.0))
        shared = shared * cos
    scale = _expand(params["scale"], lengths, device) if config == 4 else None

    grads = []
    for k in range(K):
        x = torch.randn(N, generator=_gen(device, config, seed, 3, k),
                        device=device, dtype=torch.float32)
        if config == 2:
            x.add_(shared)
        elif config == 3:
            x.mul_(1e-3)
        elif config == 4:
            x.mul_(scale)
        elif config == 5:
            x.mul_(sin).add_(shared)
            keep = _expand((~params["zero"][k]).astype(np.float32), lengths, device)
            x.mul_(keep)
        grads.append(x.to(tdt))
        del x
    return Workload(K=K, dtype=dtype, seg_offsets=off, grads=grads, config=config,
                    seed=seed, notes={"params": params})


def random_case(K, lengths, dtype="f32", seed=0, device="cpu", kind="normal",
                zero_workers=()):
    """A small seeded case for edge-case tests.

    kind: "normal"  i.i.d. N(0,1);
          "shared"  shared N(0,1) + independent N(0,1) (pairwise cosine ~0.5);
          "scaled"  N(0,1) times a per-segment scale log-uniform in [1e-6, 1].
    ``zero_workers`` lists workers whose buffers are all zero.
    """
    off = offsets_from_lengths(lengths)
    N = int(off[-1])
    tdt = TORCH_DTYPES[dtype]
    shared = torch.randn(N, generator=_gen("cpu", 99, seed, 2, 0), dtype=torch.float32)
    rng = np.random.default_rng(np.random.SeedSequence([99, seed, 1]))
    scale = torch.repeat_interleave(
        torch.as_tensor(np.exp(rng.uniform(np.log(1e-6), 0.0, size=len(lengths))), dtype=torch.float32),
        torch.as_tensor(np.asarray(lengths, dtype=np.int64)))
    grads = []
    for k in range(K):
        x = torch.randn(N, generator=_gen("cpu", 99, seed, 3, k), dtype=torch.float32)
        if kind == "shared":
            x = x + shared
        elif kind == "scaled":
            x = x * scale
        elif kind != "normal":
            raise ValueError(kind)
        if k in zero_workers:
            x.zero_()
        grads.append(x.to(tdt).to(device))
    return Workload(K=K, dtype=dtype, seg_offsets=off, grads=grads, seed=seed)


def cancelling_pairs(K, lengths, eps, dtype="f32", seed=0):
    """Worker pairs that nearly cancel: g_{2m+1} = -(1 + eps) g_{2m} + eps n.

    Every worker starts as i.i.d. N(0,1) in fp64 (one torch generator seeded
    with ``seed``, workers drawn in order); each odd worker is then replaced
    by the negative of its even neighbour, stretched by 1 + eps, plus eps
    times its own draw, and every worker is rounded to ``dtype``.  A level-1
    node of such a pair is about eps times the size of its operands, so the
    merges above it see a cancellation of about eps^2 in squared norm.  These
    are the near anti-parallel pairs of the operator's properties (parallel
    gradients are averaged; an exactly anti-parallel equal-norm pair gives
    zero).  Host tensors.
    """
    off = offsets_from_lengths(lengths)
    N = int(off[-1])
    g = torch.Generator().manual_seed(int(seed))
    base = [torch.randn(N, generator=g, dtype=torch.float64) for _ in range(K)]
    for k in range(1, K, 2):
        base[k] = -(1.0 + eps) * base[k - 1] + eps * base[k]
    grads = [v.to(TORCH_DTYPES[dtype]) for v in base]
    return Workload(K=K, dtype=dtype, seg_offsets=off, grads=grads, seed=int(seed), notes={"eps": float(eps)})
