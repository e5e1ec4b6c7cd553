"""The flip-tolerant MXFP8 comparison (tests/mx_check.py) on the CPU: it must
accept outputs whose h differs from the oracle's only by rounding flips at
near-ties, and reject planted mistakes (a wrong block scale, a wrong code away
from a tie, two swapped elements, a dropped element)."""

import numpy as np
import pytest

import oracle

from mx_check import check_flips


def setup(seed=0, E=2, H=256, I=384, R=40):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, H)).astype(np.float32)
    ws = [(rng.standard_normal((E, I, H)) / np.sqrt(H)).astype(np.float32),
          (rng.standard_normal((E, I, H)) / np.sqrt(H)).astype(np.float32),
          (rng.standard_normal((E, H, I)) / np.sqrt(I)).astype(np.float32)]
    q = [oracle.mxfp8_quantize(w) for w in ws]
    xq, xs = oracle.mxfp8_quantize(x)
    off = np.linspace(0, R, E + 1).astype(np.int32)
    y, h = oracle.grouped_ffn_mxfp8(xq, xs, off, *q, return_h=True)
    return q, off, y, h


def simulate(q, off, h, noise, seed=1, edit=None):
    """y from a perturbed h (as a different summation would give), quantised
    with the oracle's own rounding; `edit` plants a mistake in (codes, scales)."""
    rng = np.random.default_rng(seed)
    hp = (h.astype(np.float64) * (1 + noise * rng.standard_normal(h.shape))).astype(np.float32)
    hq, hs = oracle.mxfp8_quantize(hp)
    if edit:
        edit(hq, hs)
    hd = oracle.mxfp8_decode(hq, hs)
    wd = oracle.mxfp8_decode(*q[2])
    e_of = np.searchsorted(off, np.arange(h.shape[0]), side="right") - 1
    return np.stack([wd[e_of[r]] @ hd[r] for r in range(h.shape[0])]).astype(np.float32)


def run_check(q, off, y, h, ys):
    rms = float(np.sqrt((y.astype(np.float64) ** 2).mean()))
    e_of = np.searchsorted(off, np.arange(h.shape[0]), side="right") - 1
    n = 0
    for r in range(h.shape[0]):
        wd = (q[2][0][e_of[r]], q[2][1][e_of[r]])
        f, _ = check_flips(ys[r].astype(np.float64) - y[r], [(1.0, wd, h[r])], rms, f"row {r}")
        n += f
    return n


def test_accepts_rounding_flips():
    q, off, y, h = setup()
    ys = simulate(q, off, h, noise=2e-4)
    assert np.abs(ys - y).max() > 1e-3          # flips happened
    assert run_check(q, off, y, h, ys) > 0


def test_accepts_identical():
    q, off, y, h = setup()
    assert run_check(q, off, y, h, simulate(q, off, h, noise=0.0)) == 0


def far_from_tie(h, row):
    """An element of h[row] whose code no perturbation of 1e-3 would change."""
    hq, hs = oracle.mxfp8_quantize(h[row:row + 1])
    v = oracle.mxfp8_decode(hq, hs)[0]
    i = int(np.argmin(np.abs(np.abs(h[row]) - np.abs(v)) / np.maximum(np.abs(v), 1e-30)
                      + (np.abs(v) < 1e-2 * np.abs(v).max())))
    return i


@pytest.mark.parametrize("mistake", ["scale", "code", "swap", "drop"])
def test_rejects_planted_mistakes(mistake):
    q, off, y, h = setup()
    r = 7
    i = far_from_tie(h, r)

    def edit(hq, hs):
        if mistake == "scale":
            hs[r, i // 32] += 1
        elif mistake == "code":
            hq[r, i] = hq[r, i] + 1 if (hq[r, i] & 0x7F) < 0x7E else hq[r, i] - 1
        elif mistake == "swap":
            j = (i + 5) % h.shape[1]
            hq[r, i], hq[r, j] = hq[r, j], hq[r, i]
        else:
            hq[r, i] = 0
    ys = simulate(q, off, h, noise=0.0, edit=edit)
    with pytest.raises(AssertionError):
        run_check(q, off, y, h, ys)
