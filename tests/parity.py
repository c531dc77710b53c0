"""Float comparison of GPU results with the float64 oracle.

Three checks per output, so that an error confined to a few rows, a tile or a
ragged tail is not diluted by the size of the whole tensor:

* spec: relative Frobenius error against the float64 oracle <= 2e-3 (the
  stated tolerance);
* one rounding: relative Frobenius error against the oracle rounded once to
  the output format (bf16 outputs are specified as fp32 accumulation with one
  rounding), which a correct kernel meets with a much smaller error than the
  spec bound (only fp32 summation order differs);
* local: the same one-rounding error taken per row and per 128 x 128 tile,
  the largest of which must stay below a bound that a single wrong row or
  tile exceeds (rows shorter than 256 elements are taken a few at a time);
  an element whose float64 value is within 1/32 of a bf16 step of a rounding
  midpoint may take either neighbour.
"""

from __future__ import annotations

import numpy as np

SPEC = 2e-3          # stated tolerance, float64 reference
ONE_BF16 = 6e-4      # against the bf16-rounded reference, whole tensor
LOCAL_BF16 = 1.5e-3  # against the bf16-rounded reference, per row / tile
ONE_F32 = 2e-5       # fp32 outputs (u): whole tensor
LOCAL_F32 = 1e-4     # fp32 outputs: per row / tile
TILE = 128


def _rel(a, b):
    den = float(np.linalg.norm(b))
    num = float(np.linalg.norm(a - b))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def bf16_round(ref):
    """float64 values rounded to bf16 (through fp32; a double rounding can
    differ only on exact fp32 ties, which do not matter to these norms)."""
    u = np.ascontiguousarray(np.asarray(ref, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


MIN_GROUP = 256      # elements: below this one rounding step can dominate a group


def _ulp_bf16(x):
    """Spacing of bf16 numbers at |x| (the normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def worst_group(got, ref, bound):
    """Where local_max finds its worst group: (kind, rows, cols, size, worst
    element difference in bf16 steps of the reference, elements differing,
    share of the group's norm held by its largest element)."""
    g = np.atleast_2d(np.asarray(got, np.float64))
    r = np.atleast_2d(np.asarray(ref, np.float64))
    best = (-1.0, None)
    rows_per = max(1, -(-MIN_GROUP // r.shape[1]))
    groups = [("rows", slice(i, i + rows_per), slice(None)) for i in range(0, r.shape[0], rows_per)]
    groups += [("tile", slice(i, i + TILE), slice(j, j + TILE))
               for i in range(0, r.shape[0], TILE) for j in range(0, r.shape[1], TILE)]
    for kind, si, sj in groups:
        a, b = g[si, sj], r[si, sj]
        lim = bound if a.size >= MIN_GROUP else bound + 2.0 ** -8
        e = _rel(a, b) * bound / lim
        if e > best[0]:
            best = (e, (kind, si, sj, a, b))
    e, (kind, si, sj, a, b) = best
    steps = np.abs(a - b) / _ulp_bf16(b)
    nb = float(np.linalg.norm(b))
    share = float(np.max(np.abs(b))) / nb if nb > 0 else 0.0
    return {"kind": kind, "rows": (si.start, si.stop), "cols": (sj.start, sj.stop), "size": int(a.size),
            "max_steps": float(steps.max()), "n_diff": int(np.count_nonzero(a != b)),
            "top_share": round(share, 3)}


def local_max(got, ref, bound):
    """Largest relative error over groups of rows (consecutive rows holding
    at least MIN_GROUP elements; one row when rows are that long) and over
    128 x 128 tiles, each normalised to `bound`: a group smaller than
    MIN_GROUP (a ragged tail tile) is allowed one bf16 rounding step (2^-8)
    more, since a single output element that rounds the other way can carry
    most of its norm.  Groups whose reference is all zero must match exactly.
    Returns the worst error scaled so that a value <= `bound` passes."""
    g = np.atleast_2d(np.asarray(got, np.float64))
    r = np.atleast_2d(np.asarray(ref, np.float64))
    worst = 0.0

    def take(a, b):
        nonlocal worst
        lim = bound if a.size >= MIN_GROUP else bound + 2.0 ** -8
        worst = max(worst, _rel(a, b) * bound / lim)

    rows_per = max(1, -(-MIN_GROUP // r.shape[1]))
    for i in range(0, r.shape[0], rows_per):
        take(g[i:i + rows_per], r[i:i + rows_per])
    for i in range(0, r.shape[0], TILE):
        for j in range(0, r.shape[1], TILE):
            take(g[i:i + TILE, j:j + TILE], r[i:i + TILE, j:j + TILE])
    return worst


NEAR_TIE = 2.0 ** -5  # of a bf16 step: either rounding of such a value is correct


def near_tie_ref(got, ref):
    """The bf16-rounded reference, except where the float64 value lies within
    NEAR_TIE of a bf16 step from a rounding midpoint and the result is the
    other neighbour: fp32 accumulation in any order may round such a value
    either way.  Used only by the per-group check, where one element that
    carries much of a small group's norm would otherwise turn a correct
    rounding into a large group error."""
    ref = np.asarray(ref, np.float64)
    got = np.asarray(got, np.float64)
    one = bf16_round(ref)
    step = _ulp_bf16(one)
    lo = np.where(one <= ref, one, one - step)
    mid = lo + step / 2
    near = np.abs(ref - mid) <= NEAR_TIE * step
    other = np.where(one == lo, lo + step, lo)
    return np.where(near & (got == other), got, one)


def report(got, ref, fmt="bf16"):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    one_ref = bf16_round(ref) if fmt == "bf16" else ref
    local_ref = near_tie_ref(got, ref) if fmt == "bf16" else ref
    local = LOCAL_BF16 if fmt == "bf16" else LOCAL_F32
    return {"spec": _rel(got, ref), "one": _rel(got, one_ref),
            "local": local_max(got, local_ref, local)}


def check(outputs, fmts=None):
    """outputs: {name: (got, ref)}; fmts: {name: 'bf16' | 'f32'} (default bf16).
    Raises AssertionError naming every output and bound that fails."""
    fmts = fmts or {}
    errs, bad = {}, []
    for name, (got, ref) in outputs.items():
        fmt = fmts.get(name, "bf16")
        e = report(got, ref, fmt)
        errs[name] = e
        one, loc = (ONE_BF16, LOCAL_BF16) if fmt == "bf16" else (ONE_F32, LOCAL_F32)
        if not e["spec"] <= SPEC:
            bad.append(f"{name}: spec {e['spec']:.3e} > {SPEC}")
        if not e["one"] <= one:
            bad.append(f"{name}: one-rounding {e['one']:.3e} > {one}")
        if not e["local"] <= loc:
            local_ref = near_tie_ref(got, ref) if fmt == "bf16" else np.asarray(ref, np.float64)
            where = worst_group(got, local_ref, loc)
            bad.append(f"{name}: local {e['local']:.3e} > {loc} at {where}")
    summary = {k: {kk: f"{vv:.2e}" for kk, vv in v.items()} for k, v in errs.items()}
    assert not bad, f"{bad}; all: {summary}"
    return errs
