"""Pins for the oracle's NVFP4 fake quantization (CPU only).

Each test checks the oracle against something other than itself: hand-worked
cases, exact rational brute force, an integer formulation of the E2M1 step
over every bf16 value and every E4M3 scale, torch's float8_e4m3fn cast for
the scale step, and the idempotence property with its documented exceptions.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.nvfp4 import E4M3_GRID, e2m1_code, e4m3_scale_code, fake_nvfp4
from workloads import make_inputs, random_bf16

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_worked_cases():
    cases = []
    with open(os.path.join(HERE, "golden", "nvfp4_worked_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, xs, sb, ys = [p.strip() for p in line.split("|")]
            x = np.array([float(t) for t in xs.split()])
            y = np.array([float(t) for t in ys.split()])
            neg_zero = np.array([t == "-0" for t in ys.split()])
            cases.append((name, x, int(sb, 16), y, neg_zero))
    return cases


WORKED = _load_worked_cases()


@pytest.mark.parametrize("case", WORKED, ids=[c[0] for c in WORKED])
def test_worked_cases(case):
    name, x, sbyte, y, neg_zero = case
    assert x.shape == (16,) and y.shape == (16,)
    xh, s, scode, _ = fake_nvfp4(x)
    assert int(scode[0]) == sbyte
    assert np.array_equal(xh, y)
    # signed zeros: compare sign bits where the expectation is a zero
    zero = y == 0
    assert np.array_equal(np.signbit(xh[zero]), neg_zero[zero])


# ---------------------------------------------------------------------------
# Exact rational brute force: nearest grid point by exhaustive search.

def _e4m3_values_fraction():
    vals = []
    for code in range(127):  # 0x7F is NaN
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(Fraction(m, 512))
        else:
            vals.append(Fraction(8 + m, 8) * Fraction(2) ** (e - 7))
    return vals


_E4M3_F = _e4m3_values_fraction()
_E2M1_F = [Fraction(n, 2) for n in (0, 1, 2, 3, 4, 6, 8, 12)]


def _rne_fraction(t: Fraction, grid):
    """Nearest grid value by exhaustive search; a tie picks the even code."""
    best = None
    for code, g in enumerate(grid):
        d = abs(g - t)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def _fq_fraction(block):
    xs = [Fraction(float(v)) for v in block]
    amax = max(abs(v) for v in xs)
    scode = _rne_fraction(amax / 6, _E4M3_F)  # saturation: 448 is the nearest beyond
    s = _E4M3_F[scode]
    out = []
    for v in xs:
        if s == 0:
            c = Fraction(0)
        else:
            c = _E2M1_F[_rne_fraction(abs(v) / s, _E2M1_F)]
        out.append(-(c * s) if v < 0 else c * s)
    return scode, out


@pytest.mark.parametrize("dist,seed,scale", [("normal", 11, 1.0), ("loguniform", 12, 1.0),
                                             ("normal", 13, 1e-3), ("normal", 14, 300.0)])
def test_fraction_brute_force(dist, seed, scale):
    x = random_bf16((96, 16), seed, scale=scale, dist=dist).double().numpy()
    xh, _, scode, _ = fake_nvfp4(x)
    for g in range(x.shape[0]):
        sc, out = _fq_fraction(x[g])
        assert int(scode[g, 0]) == sc, (g, x[g])
        assert [Fraction(float(v)) for v in xh[g]] == out, (g, x[g])


def test_fraction_brute_force_ties():
    """Groups built so that many elements sit exactly on E2M1 midpoints."""
    rng = np.random.default_rng(5)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for trial in range(200):
        s = E4M3_GRID[rng.integers(1, 127)]
        vals = rng.choice(mids, size=15) * s * rng.choice([-1.0, 1.0], size=15)
        block = np.concatenate([[6.0 * s], vals])  # amax/6 == s exactly
        f32 = block.astype(np.float32)
        if not np.array_equal(f32.astype(np.float64), block):
            continue
        sc, out = _fq_fraction(block)
        xh, _, scode, _ = fake_nvfp4(block)
        assert int(scode[0]) == sc
        assert [Fraction(float(v)) for v in xh] == out


# ---------------------------------------------------------------------------
# Exhaustive E2M1 step: every positive finite bf16 x against every positive
# E4M3 scale, decided with integer arithmetic.

def _all_positive_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)  # +0 excluded, below +inf
    return (bits << 16).view(np.float32).astype(np.float64)


def _integer_e2m1_code(x, s):
    """RNE_E2M1(x/s) decided with integers: x = mx*2^ex, s = ms*2^es."""
    mx, ex = np.frexp(x)  # x = mx * 2^ex, 0.5 <= mx < 1
    mxi = np.round(mx * 2 ** 24).astype(np.int64)  # exact integer significand
    exi = ex.astype(np.int64) - 24
    ms, es = np.frexp(s)
    msi = np.round(ms * 2 ** 24).astype(np.int64)
    esi = es.astype(np.int64) - 24
    # strip trailing zeros so the integers stay small
    for arr, e in ((mxi, exi), (msi, esi)):
        while True:
            even = (arr % 2 == 0) & (arr != 0)
            if not even.any():
                break
            arr[even] //= 2
            e[even] += 1
    # 4 * midpoints between consecutive E2M1 codes k and k+1
    mid4 = [1, 3, 5, 7, 10, 14, 20]
    code = np.zeros(np.broadcast(x, s).shape, dtype=np.int64)
    d = exi - esi + 2  # compare mx*2^d with mid4*ms
    d = np.clip(d, -60, 60)
    for k, m4 in enumerate(mid4):
        lhs = np.where(d >= 0, mxi * np.left_shift(1, np.clip(d, 0, 40)), mxi)
        rhs = np.where(d >= 0, m4 * msi, m4 * msi * np.left_shift(1, np.clip(-d, 0, 40)))
        big_l = d > 40
        big_r = d < -40
        gt = np.where(big_l, True, np.where(big_r, False, lhs > rhs))
        eq = np.where(big_l | big_r, False, lhs == rhs)
        up = gt | (eq & ((k + 1) % 2 == 0))
        code += up
    return code


@pytest.mark.slow
def test_e2m1_exhaustive_integer():
    xs = _all_positive_bf16()
    for scode in range(1, 127):
        s = E4M3_GRID[scode]
        want = _integer_e2m1_code(xs, np.full_like(xs, s))
        got = e2m1_code(xs, np.full_like(xs, s))
        bad = np.nonzero(want != got)[0]
        assert bad.size == 0, (scode, xs[bad[:5]], want[bad[:5]], got[bad[:5]])


# ---------------------------------------------------------------------------
# The scale step against a library cast (torch float32 -> float8_e4m3fn, RNE).

def test_e4m3_step_vs_torch_cast():
    amax = _all_positive_bf16()
    v32 = (torch.from_numpy(amax.astype(np.float32)) / 6.0)
    ok = v32 <= 448.0
    lib = v32[ok].to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
    ours = e4m3_scale_code(amax[ok.numpy()])
    assert ok.sum() > 17000
    assert np.array_equal(ours, lib)
    # beyond 448 the scale saturates
    assert np.all(e4m3_scale_code(amax[~ok.numpy()]) == 126)


def test_e4m3_grid_vs_torch():
    codes = torch.arange(127, dtype=torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(vals, E4M3_GRID)


# ---------------------------------------------------------------------------
# Properties.

def test_idempotent_on_qkv_like_data():
    q, k, v, _ = make_inputs("ref_shape", seqlen=256, heads=2)
    for t in (q, k, v):
        x = t.double().numpy()
        xh, s, _, _ = fake_nvfp4(x)
        assert s.min() >= 2.0 ** -7
        xhh, _, _, _ = fake_nvfp4(xh)
        assert np.array_equal(xh, xhh)


def test_idempotence_documented_exceptions():
    # Below scale 2^-7 a second pass can move values: amax 0.005889892578125
    # -> 0.005859375 (scale 2^-9) -> 0 (its /6 is exactly 2^-10, a tie to 0).
    x = np.array([0.005889892578125] + [0.0] * 15)
    x1 = fake_nvfp4(x)[0]
    x2 = fake_nvfp4(x1)[0]
    assert x1[0] == 0.005859375 and x2[0] == 0.0
    # amax 0.0185546875 -> 0.015625 -> 0.01171875
    y = np.array([0.0185546875] + [0.0] * 15)
    y1 = fake_nvfp4(y)[0]
    y2 = fake_nvfp4(y1)[0]
    assert y1[0] == 0.015625 and y2[0] == 0.01171875


def test_outputs_exact_in_bf16():
    x = random_bf16((512, 64), 21, dist="loguniform").double().numpy()
    xh = fake_nvfp4(x)[0]
    f32 = xh.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), xh)
    assert np.all((f32.view(np.uint32) & 0xFFFF) == 0)


def test_short_last_group_is_zero_padded():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 40)).astype(np.float32).astype(np.float64)
    padded = np.concatenate([x, np.zeros((5, 8))], axis=1)
    a = fake_nvfp4(x)[0]
    b = fake_nvfp4(padded)[0][:, :40]
    assert np.array_equal(a, b)


def test_axis_argument():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 48)).astype(np.float32).astype(np.float64)
    assert np.array_equal(fake_nvfp4(x, axis=0)[0], fake_nvfp4(x.T, axis=-1)[0].T)


def test_scale_invariance_by_powers_of_two():
    # Multiplying a group by 2^k (staying within normal scale range) multiplies
    # the result by 2^k: the E4M3 and E2M1 grids are binade-periodic there.
    x = random_bf16((64, 16), 31).double().numpy()
    for k in (-3, 1, 4):
        a = fake_nvfp4(x * 2.0 ** k)[0]
        b = fake_nvfp4(x)[0] * 2.0 ** k
        assert np.array_equal(a, b)


def test_fp32_inputs_brute_force():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((64, 16)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    x = x.astype(np.float64)
    xh, _, scode, _ = fake_nvfp4(x)
    for g in range(x.shape[0]):
        sc, out = _fq_fraction(x[g])
        assert int(scode[g, 0]) == sc
        assert [Fraction(float(v)) for v in xh[g]] == out
