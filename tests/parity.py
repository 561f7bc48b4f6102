"""Parity gates shared by the GPU tests: the HIP path against the fp64 oracle.

Gates (the stated tolerances of the combiner):
  * output, per call: relative L2 error ||gpu - oracle|| / ||oracle|| <= 1e-5
    for fp32 inputs and <= 2e-3 for fp16 / bf16 inputs, the oracle rounded once
    to the output dtype;
  * output, per segment (each layer is combined on its own, so each is gated
    against its own norm): the elements that differ from the rounded oracle
    by more than one output ulp, taken together, have an L2 norm of at most
    TOL times the segment's norm.  The one-ulp allowance is there because both
    sides round an fp64 value once: where the exact value sits next to a
    rounding boundary, the two roundings may fall on either side of it (a
    one-element bf16 segment would otherwise fail on representation alone);
  * coefficients: |c_gpu - c_oracle| <= 1e-6 * max(1, |c_oracle|) for every
    (node, segment), except at the operator's discontinuity
    (``oracle.discontinuity_mask`` with ``NEAR_ZERO``, below);
  * statistics (gated loosely, for diagnosis): relative 1e-5.
"""

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
COEFF_TOL = 1e-6
# An operand whose squared norm is at most NEAR_ZERO times the summed squared
# norms of the input gradients under it sits at the zero discontinuity: its
# coefficient jumps to 1 at exactly zero and tends to another value next to
# it, so a node that is zero in exact arithmetic but carries rounding noise
# has no stable coefficient.  Its coefficient and those of the nodes above it
# are not compared; both sides must only agree that the operand is (nearly)
# zero.
NEAR_ZERO = 1e-8


def say(*args):
    print("[parity]", *args, flush=True)


def rel_l2(x, ref):
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    return num / den if den > 0 else num


def ulp(ref, dtype):
    """Spacing of the output format at each value of ``ref`` (fp64 holding
    values of that format): the distance from |x| to the next larger value."""
    ref = np.abs(np.asarray(ref, dtype=np.float64))
    if dtype == "f32":
        return np.abs(np.spacing(ref.astype(np.float32))).astype(np.float64)
    if dtype == "f16":
        return np.abs(np.spacing(ref.astype(np.float16))).astype(np.float64)
    if dtype == "bf16":  # bf16 values are fp32 values with 16 zero low bits
        bits = ref.astype(np.float32).view(np.uint32)
        up = (bits + np.uint32(0x10000)).view(np.float32).astype(np.float64)
        return up - ref
    raise ValueError(dtype)


def segment_gate(got, ref, seg_offsets, dtype, segments=None):
    """Per-segment output gate.  Returns (worst ratio, its segment, worst plain
    relative L2 of any segment); the gate holds when the ratio is <= 1."""
    off = np.asarray(seg_offsets, dtype=np.int64)
    segs = range(off.size - 1) if segments is None else segments
    worst, where, plain = 0.0, -1, 0.0
    for i, s in enumerate(segs):
        if segments is None:
            lo, hi = int(off[s]), int(off[s + 1])
            g, r = got[lo:hi], ref[lo:hi]
        else:  # got and ref are lists of per-segment arrays
            g, r = got[i], ref[i]
        if r.size == 0:
            continue
        d = g - r
        beyond = np.where(np.abs(d) > ulp(r, dtype), d, 0.0)
        num = float(np.linalg.norm(beyond))
        den = float(np.linalg.norm(r))
        ratio = (num / (TOL[dtype] * den)) if den > 0 else (np.inf if num > 0 else 0.0)
        if not np.isfinite(num) and not np.all(np.isfinite(r)):
            ratio = 0.0 if np.array_equal(np.isnan(g), np.isnan(r)) else np.inf  # NaN inputs propagate
        if ratio > worst or where < 0:
            worst, where = ratio, int(s)
        plain = max(plain, rel_l2(g, r) if den > 0 else float(np.linalg.norm(d)))
    return worst, where, plain


def near_zero(s_ref, opnorms):
    """[..., 2] mask: operand a (resp. b) of a node is at the zero
    discontinuity, its oracle |a|^2 at most NEAR_ZERO of the summed squared
    input norms under it (``oracle.operand_input_norms``), which are not all
    zero (an operand over all-zero inputs is exactly zero on both sides and
    its coefficient, exactly 1, stays gated)."""
    return (s_ref[..., 1:3] <= NEAR_ZERO * opnorms) & (opnorms > 0)


def unstable(s_ref, opnorms, schedule="tree"):
    """``oracle.discontinuity_mask`` of every segment: [K-1, nseg, 2] (or
    [K-1, 2] for one segment)."""
    if s_ref.ndim == 2:
        return oracle.discontinuity_mask(s_ref, opnorms, schedule, NEAR_ZERO)
    out = np.zeros(s_ref.shape[:2] + (2,), dtype=bool)
    for s in range(s_ref.shape[1]):
        out[:, s] = oracle.discontinuity_mask(s_ref[:, s], opnorms[:, s], schedule, NEAR_ZERO)
    return out


def coeff_errors(c_gpu, c_ref, exempt=None):
    err = np.abs(c_gpu - c_ref) / np.maximum(1.0, np.abs(c_ref))
    if exempt is not None:
        err = np.where(exempt, 0.0, err)
    return err


def check_coeffs(c_gpu, c_ref, what, exempt=None):
    assert np.all(np.isfinite(c_gpu)), what
    err = coeff_errors(c_gpu, c_ref, exempt)
    worst = float(err.max()) if err.size else 0.0
    assert worst <= COEFF_TOL, f"{what}: coefficient error {worst:.3g}"
    return worst


def check_stats(s_gpu, s_ref, what, opnorms=None, schedule="tree"):
    if s_ref.size == 0:
        return 0
    d, A, B = s_ref[..., 0], s_ref[..., 1], s_ref[..., 2]
    if opnorms is None:
        zero_a = zero_b = np.zeros(A.shape, dtype=bool)
    else:
        direct = near_zero(s_ref, opnorms)
        # at the discontinuity the GPU must also see the operand as (nearly) zero
        assert np.all(s_gpu[..., 1][direct[..., 0]] <= 1e-6 * opnorms[..., 0][direct[..., 0]] + 1e-300), what
        assert np.all(s_gpu[..., 2][direct[..., 1]] <= 1e-6 * opnorms[..., 1][direct[..., 1]] + 1e-300), what
        mask = unstable(s_ref, opnorms, schedule)
        zero_a, zero_b = mask[..., 0], mask[..., 1]
    scale = np.sqrt(np.maximum(A, 0) * np.maximum(B, 0))
    assert np.all((np.abs(s_gpu[..., 1] - A) <= 1e-5 * A + 1e-300) | zero_a), what
    assert np.all((np.abs(s_gpu[..., 2] - B) <= 1e-5 * B + 1e-300) | zero_b), what
    assert np.all((np.abs(s_gpu[..., 0] - d) <= 1e-5 * scale + 1e-300) | zero_a | zero_b), what
    return int(np.count_nonzero(zero_a | zero_b))


def segment_opnorms(wl, schedule="tree"):
    """operand_input_norms of every segment: [K-1, nseg, 2]."""
    rows = [g.double().cpu().numpy() for g in wl.grads]
    out = np.zeros((max(wl.K - 1, 0), wl.nseg, 2))
    for s in range(wl.nseg):
        lo, hi = int(wl.seg_offsets[s]), int(wl.seg_offsets[s + 1])
        out[:, s] = oracle.operand_input_norms([r[lo:hi] for r in rows], schedule)
    return out


def run_gpu(wl, schedule="tree"):
    import distributed_sgd_gradient_amd as A
    out, coeffs, stats = A.combine(wl.grads, wl.seg_offsets, schedule=schedule, return_coeffs=True,
                                   return_stats=True)
    torch.cuda.synchronize()
    return out, coeffs, stats


def evaluate(wl, schedule="tree"):
    """Run the GPU combine and the oracle on a workload; return every figure
    the gates use, without asserting: {rel_l2, seg_ratio, seg_worst, seg_plain,
    coeff_err, exempt, got, ref, ...}."""
    out, coeffs, stats = run_gpu(wl, schedule)
    combine = oracle.combine_chain if schedule == "chain" else oracle.combine
    ref = combine([g.double().cpu().numpy() for g in wl.grads], wl.seg_offsets, out_format=wl.dtype)
    got = out.double().cpu().numpy()
    opn = segment_opnorms(wl, schedule)
    mask = unstable(ref["stats"], opn, schedule)
    c = coeffs.cpu().numpy()
    cerr = coeff_errors(c, ref["coeffs"], mask)
    ratio, seg, plain = segment_gate(got, ref["out_rounded"], wl.seg_offsets, wl.dtype)
    return {"rel_l2": rel_l2(got, ref["out_rounded"]), "seg_ratio": ratio, "seg_worst": seg, "seg_plain": plain,
            "coeff_err": float(cerr.max()) if cerr.size else 0.0, "coeffs_finite": bool(np.all(np.isfinite(c))),
            "exempt": int(np.count_nonzero(mask)), "got": got, "ref": ref, "coeffs": c,
            "stats": stats.cpu().numpy(), "opnorms": opn, "mask": mask}


def passes(ev, dtype):
    return (ev["rel_l2"] <= TOL[dtype] and ev["seg_ratio"] <= 1.0 and ev["coeff_err"] <= COEFF_TOL
            and ev["coeffs_finite"])


def full_check(wl, label, schedule="tree"):
    """Compare every element and every (node, segment) with the oracle."""
    say(label, f"K={wl.K} dtype={wl.dtype} N={wl.N} nseg={wl.nseg} schedule={schedule}")
    ev = evaluate(wl, schedule)
    err = ev["rel_l2"]
    assert err <= TOL[wl.dtype], f"{label}: relative L2 {err:.3g}"
    assert ev["seg_ratio"] <= 1.0, (f"{label}: segment {ev['seg_worst']} misses the per-segment gate "
                                    f"({ev['seg_ratio']:.3g} of its budget)")
    check_coeffs(ev["coeffs"], ev["ref"]["coeffs"], label, ev["mask"])
    nz = check_stats(ev["stats"], ev["ref"]["stats"], label, ev["opnorms"], schedule)
    say(label, f"relative L2 {err:.3g}; worst segment {ev['seg_worst']}: {ev['seg_ratio']:.3g} of its budget "
        f"(plain relative L2 up to {ev['seg_plain']:.3g}); coefficient error {ev['coeff_err']:.3g}"
        + (f"; {nz} node(s) at or above the zero discontinuity not compared" if nz else ""))
    return ev["got"], ev["ref"], err


def sampled_check(wl, segments, label, schedule="tree"):
    """Full-size run; compare the chosen segments one by one with the oracle."""
    say(label, f"K={wl.K} dtype={wl.dtype} N={wl.N} nseg={wl.nseg} sampled={len(segments)} schedule={schedule}")
    out, coeffs, stats = run_gpu(wl, schedule)
    walk = oracle.adasum_chain if schedule == "chain" else oracle.adasum_tree
    c_all = coeffs.cpu().numpy()
    s_all = stats.cpu().numpy()
    worst = 0.0
    num = den = 0.0
    gots, refs = [], []
    for s in segments:
        lo, hi = int(wl.seg_offsets[s]), int(wl.seg_offsets[s + 1])
        rows = wl.segment_host(s)
        res, cf, st = walk(rows)
        ref = oracle.round_to_format(res, wl.dtype)
        got = out[lo:hi].double().cpu().numpy()
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
        gots.append(got)
        refs.append(ref)
        st = np.asarray(st).reshape(-1, 3)
        opn = oracle.operand_input_norms(rows, schedule)
        worst = max(worst, check_coeffs(c_all[:, s], np.asarray(cf).reshape(-1, 2), f"{label} seg {s}",
                                        unstable(st, opn, schedule)))
        check_stats(s_all[:, s], st, f"{label} seg {s}", opn, schedule)
    err = np.sqrt(num / den) if den > 0 else np.sqrt(num)
    ratio, seg, plain = segment_gate(gots, refs, wl.seg_offsets, wl.dtype, segments=list(segments))
    say(label, f"sampled relative L2 {err:.3g}; worst segment {seg}: {ratio:.3g} of its budget (plain relative L2 "
        f"up to {plain:.3g}); worst coefficient error {worst:.3g}")
    assert err <= TOL[wl.dtype]
    assert ratio <= 1.0, f"{label}: segment {seg} misses the per-segment gate ({ratio:.3g} of its budget)"
    return out
