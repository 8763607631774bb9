"""The W4A4 accuracy study (oracle/w4a4_study.py, reading R19): its quantisers pinned
by brute force, and the study's errors on seeded prefill inputs (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import w4a4_study as S
from bit_moe_expert_amd import workloads as wl

GRID = np.unique(np.abs(oracle.e2m1_value(np.arange(16))))   # 0, .5, 1, 1.5, 2, 3, 4, 6


def brute_e2m1(v):
    """Nearest of the eight E2M1 magnitudes (ties: the one whose index is even in the
    grid of one spacing, i.e. whose last mantissa bit is 0), saturating at 6."""
    a = min(abs(v), 6.0)
    d = np.abs(GRID - a)
    best = np.flatnonzero(d == d.min())
    if best.size > 1:  # a tie: the even code (mantissa bit 0) of the two
        codes = [int(np.flatnonzero(np.abs(oracle.e2m1_value(np.arange(8))) == GRID[b])[0]) for b in best]
        pick = best[[c % 2 == 0 for c in codes].index(True)]
    else:
        pick = best[0]
    return np.copysign(GRID[pick], v)


def test_e2m1_round_brute_force():
    vals = np.concatenate([GRID, -GRID, (GRID[1:] + GRID[:-1]) / 2, np.linspace(-8, 8, 641),
                           np.random.default_rng(0).uniform(-7, 7, 500)])
    got = S.e2m1_round(vals)
    want = np.array([brute_e2m1(v) for v in vals])
    assert np.array_equal(got, want)
    assert np.array_equal(S.e2m1_round(GRID), GRID)           # representable values stay
    assert S.e2m1_round(np.array([5.0]))[0] == 4.0            # tie between 4 and 6 -> 4
    assert S.e2m1_round(np.array([1e9]))[0] == 6.0            # saturation


def test_mxfp4_quantize_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 128)) * np.exp2(rng.uniform(-20, 20, (40, 1)))
    x[3, 32:64] = 0.0
    q, e = S.mxfp4_quantize(x)
    xb = x.reshape(40, 4, 32)
    amax = np.abs(xb).max(-1)
    nz = amax > 0
    # the smallest e with amax * 2^-e <= 6
    assert np.all(np.ldexp(amax[nz], -e[nz]) <= 6.0)
    assert np.all(np.ldexp(amax[nz], -(e[nz] - 1)) > 6.0)
    assert np.all(e[~nz] == 0)
    # each value rounded to the nearest E2M1 value at its block's scale
    scaled = np.ldexp(xb, -e[..., None]).reshape(-1)
    want = np.array([brute_e2m1(v) for v in scaled]).reshape(q.shape)
    assert np.array_equal(q, want)


@pytest.mark.parametrize("name", ["prefill", "long_prefill"])
def test_w4a4_study(name):
    """The study's numbers (quoted where the design discusses W4A4): rms and max error of
    the expert outputs, relative to their rms, on 32 seeded tokens' first 6 experts."""
    w = wl.workload(name)
    inp = wl.make_inputs(w, seed=0, T=32)
    res = S.study(inp, np.arange(32), experts=6)
    print(f"\n  {name}: " + ", ".join(f"{k} rms {a:.4f} max {b:.4f}" for k, (a, b) in res.items()))
    (r8, m8), (r4, m4) = res["w4a8"], res["w4a4"]
    assert 0.01 < r8 < 0.1 and r8 < r4           # FP8 activations: a few percent
    assert r4 > 2 * r8                          # FP4 activations and rescaled weights: several times that
