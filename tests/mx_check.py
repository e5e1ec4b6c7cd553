"""Comparison of MXFP8 FFN outputs that allows for the E4M3 rounding of h.

Both sides compute h = silu(a) * u from identical 8-bit operands but sum the
dot products in different orders and precisions (the GPU's MFMA in fp32, the
oracle in fp64), then round h to E4M3.  Where h lies within that summation
difference of a rounding boundary the two sides may keep the neighbouring
codes, and both are correct roundings of the exact h.  Such a flip moves the
decoded h_i by one E4M3 step s_i, which shifts every output y_j of the row by
s_i * Wd[j, i] -- a known direction per flip.

`check_flips` accepts a GPU result when its difference from the oracle is
explained by flips at near-ties only: it fits the difference with the
columns of the down weights that belong to near-tie elements (least
squares), rounds every coefficient to 0 or one step up or down (a block
whose maximum sits near a power of two may also change scale, so its
elements may move by up to two steps), and requires the remainder -- the
summation-order difference of everything else -- to be below 1e-3 of the
output RMS.  Elements far from a boundary are not fitted, so any other
deviation (a wrong scale, a wrong element, a transposed block) lands in the
remainder and fails.
"""

from __future__ import annotations

import numpy as np

import oracle

# a GPU h is taken to lie within ETA * |h| + FLOOR * RMS(h of the row) of
# the oracle's: the summation difference of a dot product scales with the
# sum of its absolute terms, not with its value (measured on the GPU: below
# 6e-4 * |h| and below 1e-4 * RMS(h))
ETA = 2.0 ** -9
FLOOR = 2.0 ** -11
RESID_TOL = 1e-3

_VALS = None


def _vals():
    global _VALS
    if _VALS is None:
        _VALS = oracle.e4m3_value(np.arange(0x7F))  # positive finite E4M3 values, ascending
    return _VALS


def near_ties(h32: np.ndarray):
    """For one fp32 h row: indices of the elements whose E4M3 code may differ
    between the two sides, their step sizes, and whether the flip is a block
    scale change (bound 2 steps) rather than an element rounding (1 step)."""
    vals = _vals()
    mids = (vals[:-1] + vals[1:]) / 2
    _, sc = oracle.mxfp8_quantize(np.ascontiguousarray(h32[None], np.float32))
    s = np.repeat(sc[0].astype(np.int64) - 127, 32)
    p = np.exp2(s.astype(np.float64))
    q = np.abs(h32.astype(np.float64)) / p
    j = np.clip(np.searchsorted(mids, q) - 1, 0, len(mids) - 1)
    j2 = np.clip(j + 1, 0, len(mids) - 1)
    jn = np.where(np.abs(q - mids[j]) <= np.abs(q - mids[j2]), j, j2)   # nearest boundary
    dist = np.abs(q - mids[jn])
    step = (vals[jn + 1] - vals[jn]) * p
    floor = FLOOR * float(np.sqrt(np.mean(h32.astype(np.float64) ** 2))) / p
    cand = dist <= ETA * q + floor
    qb = q.reshape(-1, 32)
    amax = qb.max(1)
    nb = (amax >= 512.0 * (1 - ETA)) | ((amax <= 256.0 * (1 + ETA)) & (amax > 0))
    block = np.repeat(nb, 32)
    idx = np.nonzero(cand | block)[0]
    # a scale change moves every element of the block by at most one step of
    # the larger scale (twice this scale's step)
    bound = np.where(block[idx], 2.0 * np.maximum(step[idx], (vals[1] - vals[0]) * p[idx]), step[idx])
    return idx, bound, block[idx]


def down_columns(wd, idx):
    """Decoded columns idx of an MXFP8 down weight given as (codes [H, I],
    scales [H, I/32]), float64 [H, len(idx)]."""
    codes, scales = wd
    return oracle.e4m3_value(codes[:, idx]) * np.exp2(scales[:, idx // 32].astype(np.float64) - 127)


def check_flips(err: np.ndarray, parts, rms_ref: float, what: str):
    """err: [H] GPU minus oracle for one output row.  parts: list of
    (gain, down weight (codes, scales) of the expert, h32 [I]) -- the rows
    whose down projections add into it.  Returns (flips found, remainder).

    The near-tie columns are fitted by least squares and each coefficient is
    rounded to a whole number of E4M3 steps (-1..1, or -2..2 for a block
    that may change scale); the remainder after those flips must stay below
    RESID_TOL * rms_ref.  A near-tie whose flip could move no output by more
    than 5% of that bound is left out of the fit (its coefficient would be
    noise); if it did flip, its effect stays inside the remainder."""
    cols, bounds, blocks = [], [], []
    for gain, wd, h in parts:
        idx, bnd, blk = near_ties(h)
        if len(idx):
            c = gain * down_columns(wd, idx)
            keep = np.abs(c).max(0) * bnd > 0.05 * RESID_TOL * rms_ref
            cols.append(c[:, keep])
            bounds.append(np.where(blk[keep], bnd[keep] / 2, bnd[keep]))   # one step
            blocks.append(blk[keep])
    resid = err
    flips = 0
    if cols and sum(c.shape[1] for c in cols):
        A = np.concatenate(cols, axis=1)
        step = np.concatenate(bounds)
        lim = np.where(np.concatenate(blocks), 2, 1)
        def rounded_fit(d):
            n = np.clip(np.rint(d / step), -lim, lim)
            return n, err - A @ (n * step)
        # normal equations first (several times faster at these sizes); the
        # SVD least-squares solution when their rounded fit leaves too much
        try:
            n, resid = rounded_fit(np.linalg.solve(A.T @ A, A.T @ err))
        except np.linalg.LinAlgError:
            n, resid = None, None
        if resid is None or np.abs(resid).max() > RESID_TOL * rms_ref:
            n, resid = rounded_fit(np.linalg.lstsq(A, err, rcond=None)[0])
        flips = int(np.count_nonzero(n))
    rmax = float(np.abs(resid).max()) if resid.size else 0.0
    assert rmax <= RESID_TOL * rms_ref, \
        f"{what}: difference not explained by rounding flips: remainder {rmax:.3e} > {RESID_TOL} * {rms_ref:.3e}"
    return flips, rmax
