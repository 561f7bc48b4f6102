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
    (node, segment);
  * statistics (gated loosely, for diagnosis): relative 1e-5.
Exempt, and reported: what the oracle itself does not determine.  At a zero
operand the operator's coefficient jumps to 1, and under deep cancellation
fp64 arithmetic no longer fixes the coefficients above it or, in a long
chain, the results built on them.  ``oracle.stability`` reruns the oracle
with every nonzero input moved by one fp64 ulp; a coefficient that moves by
more than a tenth of its tolerance, or a segment whose output does, is not
compared (``UNSTABLE``).
"""

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "f16": 2e-3, "bf16": 2e-3}
COEFF_TOL = 1e-6
# A tenth of each tolerance: the motion under one-ulp noise above which the
# oracle is no reference for a coefficient or a segment's output.
UNSTABLE = {"coeff": COEFF_TOL / 10, "f32": TOL["f32"] / 10, "f16": TOL["f16"] / 10, "bf16": TOL["bf16"] / 10}


def say(*args):
    print("[parity]", *args, flush=True)


def finite_part(x, ref):
    """Where the rounded oracle is not finite (an output that overflows its
    format, or NaN inputs), the GPU must hold the same value (the same
    infinity, or NaN); returns (x, ref) restricted to the finite entries of
    ref, or None when the non-finite entries differ."""
    fin = np.isfinite(ref)
    if fin.all():
        return x, ref
    a, b = x[~fin], ref[~fin]
    same = (np.isnan(a) & np.isnan(b)) | (a == b)
    return (x[fin], ref[fin]) if same.all() else None


def rel_l2(x, ref):
    part = finite_part(x, ref)
    if part is None:
        return float("inf")
    x, ref = part
    den = float(np.linalg.norm(ref))
    num = float(np.linalg.norm(x - ref))
    if not np.isfinite(num):  # a non-finite GPU value where the oracle is finite
        return float("inf")
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


def segment_gate(got, ref, seg_offsets, dtype, segments=None, exempt=()):
    """Per-segment output gate over the segments not in ``exempt``.  Returns
    (worst ratio, its segment, worst plain relative L2 of any gated segment);
    the gate holds when the ratio is <= 1."""
    off = np.asarray(seg_offsets, dtype=np.int64)
    segs = range(off.size - 1) if segments is None else segments
    worst, where, plain = 0.0, -1, 0.0
    for i, s in enumerate(segs):
        if s in exempt:
            continue
        if segments is None:
            lo, hi = int(off[s]), int(off[s + 1])
            g, r = got[lo:hi], ref[lo:hi]
        else:  # got and ref are lists of per-segment arrays
            g, r = got[i], ref[i]
        if r.size == 0:
            continue
        part = finite_part(g, r)
        if part is None:
            ratio = plain_s = np.inf
        else:
            g, r = part
            d = g - r
            beyond = np.where(np.abs(d) > ulp(r, dtype), d, 0.0)
            num = float(np.linalg.norm(beyond))
            den = float(np.linalg.norm(r))
            ratio = (num / (TOL[dtype] * den)) if den > 0 else (np.inf if num > 0 else 0.0)
            if not np.isfinite(num):
                ratio = np.inf
            plain_s = rel_l2(g, r)
        if ratio > worst or where < 0:
            worst, where = ratio, int(s)
        plain = max(plain, plain_s)
    return worst, where, plain


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


def check_stats(s_gpu, s_ref, what, exempt=None):
    """(a.b, |a|^2, |b|^2) of every node: |a|^2 where its coefficient ca is
    gated, |b|^2 where cb is, a.b where both are."""
    if s_ref.size == 0:
        return
    d, A, B = s_ref[..., 0], s_ref[..., 1], s_ref[..., 2]
    if exempt is None:
        ea = eb = np.zeros(A.shape, dtype=bool)
    else:
        ea, eb = exempt[..., 0], exempt[..., 1]
    scale = np.sqrt(np.maximum(A, 0) * np.maximum(B, 0))
    assert np.all((np.abs(s_gpu[..., 1] - A) <= 1e-5 * A + 1e-300) | ea), what
    assert np.all((np.abs(s_gpu[..., 2] - B) <= 1e-5 * B + 1e-300) | eb), what
    assert np.all((np.abs(s_gpu[..., 0] - d) <= 1e-5 * scale + 1e-300) | ea | eb), what


def oracle_with_stability(rows, seg_offsets, schedule, dtype):
    """The oracle's result on host rows (rounded to dtype as out_rounded),
    with the coefficients ([K-1, nseg, 2]) and segments it does not determine."""
    st = oracle.stability(rows, seg_offsets, schedule)
    ref = st["base"]
    ref["out_rounded"] = oracle.round_to_format(ref["out"], dtype)
    coeff_exempt = st["coeff_motion"] > UNSTABLE["coeff"]
    seg_exempt = set(np.flatnonzero(st["output_motion"] > UNSTABLE[dtype]).tolist())
    return ref, coeff_exempt, seg_exempt


def gated_elements(seg_offsets, seg_exempt, n):
    keep = np.ones(n, dtype=bool)
    for s in seg_exempt:
        keep[int(seg_offsets[s]):int(seg_offsets[s + 1])] = False
    return keep


def run_gpu(wl, schedule="tree"):
    import distributed_sgd_gradient_amd as A
    out, coeffs, stats = A.combine(wl.grads, wl.seg_offsets, schedule=schedule, return_coeffs=True,
                                   return_stats=True)
    torch.cuda.synchronize()
    return out, coeffs, stats


def evaluate(wl, schedule="tree"):
    """Run the GPU combine and the oracle on a workload; return every figure
    the gates use, without asserting: {rel_l2, seg_ratio, seg_worst, seg_plain,
    coeff_err, exempt, exempt_segments, got, ref, ...}."""
    out, coeffs, stats = run_gpu(wl, schedule)
    rows = [g.double().cpu().numpy() for g in wl.grads]
    ref, cex, sex = oracle_with_stability(rows, wl.seg_offsets, schedule, wl.dtype)
    got = out.double().cpu().numpy()
    keep = gated_elements(wl.seg_offsets, sex, got.size)
    c = coeffs.cpu().numpy()
    cerr = coeff_errors(c, ref["coeffs"], cex)
    ratio, seg, plain = segment_gate(got, ref["out_rounded"], wl.seg_offsets, wl.dtype, exempt=sex)
    return {"rel_l2": rel_l2(got[keep], ref["out_rounded"][keep]), "seg_ratio": ratio, "seg_worst": seg,
            "seg_plain": plain, "coeff_err": float(cerr.max()) if cerr.size else 0.0,
            "coeffs_finite": bool(np.all(np.isfinite(c))), "exempt": int(np.count_nonzero(cex)),
            "exempt_segments": sorted(sex), "got": got, "ref": ref, "coeffs": c, "stats": stats.cpu().numpy(),
            "mask": cex}


def passes(ev, dtype):
    return (ev["rel_l2"] <= TOL[dtype] and ev["seg_ratio"] <= 1.0 and ev["coeff_err"] <= COEFF_TOL
            and ev["coeffs_finite"])


def _exempt_note(ev):
    notes = []
    if ev["exempt"]:
        notes.append(f"{ev['exempt']} coefficient(s) the oracle does not determine, not compared")
    if ev["exempt_segments"]:
        notes.append(f"segment(s) {ev['exempt_segments']} whose oracle output is not determined, not compared")
    return ("; " + "; ".join(notes)) if notes else ""


def full_check(wl, label, schedule="tree"):
    """Compare every element and every (node, segment) with the oracle."""
    say(label, f"K={wl.K} dtype={wl.dtype} N={wl.N} nseg={wl.nseg} schedule={schedule}")
    ev = evaluate(wl, schedule)
    err = ev["rel_l2"]
    assert err <= TOL[wl.dtype], f"{label}: relative L2 {err:.3g}"
    assert ev["seg_ratio"] <= 1.0, (f"{label}: segment {ev['seg_worst']} misses the per-segment gate "
                                    f"({ev['seg_ratio']:.3g} of its budget)")
    check_coeffs(ev["coeffs"], ev["ref"]["coeffs"], label, ev["mask"])
    check_stats(ev["stats"], ev["ref"]["stats"], label, ev["mask"])
    say(label, f"relative L2 {err:.3g}; worst segment {ev['seg_worst']}: {ev['seg_ratio']:.3g} of its budget "
        f"(plain relative L2 up to {ev['seg_plain']:.3g}); coefficient error {ev['coeff_err']:.3g}" + _exempt_note(ev))
    return ev["got"], ev["ref"], err


def sampled_check(wl, segments, label, schedule="tree"):
    """Full-size run; compare the chosen segments one by one with the oracle."""
    say(label, f"K={wl.K} dtype={wl.dtype} N={wl.N} nseg={wl.nseg} sampled={len(segments)} schedule={schedule}")
    out, coeffs, stats = run_gpu(wl, schedule)
    c_all = coeffs.cpu().numpy()
    s_all = stats.cpu().numpy()
    worst = 0.0
    num = den = 0.0
    gots, refs, skipped, ncx = [], [], set(), 0
    for s in segments:
        lo, hi = int(wl.seg_offsets[s]), int(wl.seg_offsets[s + 1])
        rows = wl.segment_host(s)
        ref, cex, sex = oracle_with_stability(rows, [0, hi - lo], schedule, wl.dtype)
        got = out[lo:hi].double().cpu().numpy()
        if sex:
            skipped.add(int(s))
        else:
            num += float(np.sum((got - ref["out_rounded"]) ** 2))
            den += float(np.sum(ref["out_rounded"] ** 2))
        gots.append(got)
        refs.append(ref["out_rounded"])
        ncx += int(np.count_nonzero(cex))
        worst = max(worst, check_coeffs(c_all[:, s:s + 1], ref["coeffs"], f"{label} seg {s}", cex))
        check_stats(s_all[:, s:s + 1], ref["stats"], f"{label} seg {s}", cex)
    err = np.sqrt(num / den) if den > 0 else np.sqrt(num)
    ratio, seg, plain = segment_gate(gots, refs, wl.seg_offsets, wl.dtype, segments=list(segments), exempt=skipped)
    ev = {"exempt": ncx, "exempt_segments": sorted(skipped)}
    say(label, f"sampled relative L2 {err:.3g}; worst segment {seg}: {ratio:.3g} of its budget (plain relative L2 "
        f"up to {plain:.3g}); worst coefficient error {worst:.3g}" + _exempt_note(ev))
    assert err <= TOL[wl.dtype]
    assert ratio <= 1.0, f"{label}: segment {seg} misses the per-segment gate ({ratio:.3g} of its budget)"
    return out
