"""NVFP4 fake quantization, written out exactly in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY.  This is the oracle that the GPU path is checked
against.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import it; the product path never does.

What it follows
---------------
"NVFP4 Attention QAT Backward" (cuDNN frontend docs), §Overview: Q, K and V
are fake-quantized to E2M1 with one E4M3 scale per 16 values and dequantized
at once; the local-scale conversion is a *precise* division, so that exact
E2M1 midpoints keep round-to-nearest-even.  The scale is one E4M3 value per
16 contiguous elements (the FastVideo ``attn_qat_infer`` API page likewise
speaks of per-16 E4M3 scale factors).

For one group ``x[0..15]`` (a short last group is padded with zeros):

1. ``amax = max |x_i|``.
2. ``s = RNE_E4M3(amax / 6)``: the E4M3FN value nearest to ``amax/6``, an
   exact tie going to the even code, saturating at 448 (E4M3FN has no
   infinity).  6 is the largest E2M1 magnitude.
3. ``c_i = RNE_E2M1(|x_i| / s)``: the E2M1 magnitude nearest to ``|x_i|/s``
   (grid 0, 0.5, 1, 1.5, 2, 3, 4, 6), ties to the even code, saturating at 6.
   When ``s == 0`` every code is 0.
4. ``x_hat_i = sign(x_i) * c_i * s`` (the sign of a value that rounds to zero
   is kept: -0.0).

Readings taken where the pages are silent (all listed in the design notes):
single-level scaling (no per-tensor fp32 scale); the scale uses division by
6 and round-to-nearest-even (not a ceiling); saturation at 448 and at 6;
``s == 0`` gives zeros; -0.0 is kept.

How it is computed
------------------
Rounding ``t / f`` to nearest on a grid ``G`` is the same as finding the point
of the scaled grid ``f * G`` nearest to ``t``.  Every point of ``6 * G_E4M3``
and of ``s * G_E2M1`` has at most 7 significant bits, so in fp64 these scaled
grids, the midpoints between neighbours and all comparisons against bf16 or
fp32 data are exact: the result is the exact-rational rounding, with no
division performed at all.
"""
from __future__ import annotations

import numpy as np

GROUP = 16

# E2M1 magnitudes in code order (code = 2-bit exponent, 1-bit mantissa; bias 1).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0


def _e4m3_grid() -> np.ndarray:
    """All finite non-negative E4M3FN values, indexed by their byte code 0..126.

    Byte = (e << 3) | m with a 4-bit exponent (bias 7) and a 3-bit mantissa;
    e == 0 is subnormal (m * 2^-9); 0x7F is NaN and is not a value.
    """
    vals = []
    for code in range(127):
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_GRID = _e4m3_grid()
E4M3_MAX = 448.0


def _nearest_code(t: np.ndarray, factor, grid: np.ndarray) -> np.ndarray:
    """Index k of the point ``factor * grid[k]`` nearest to ``t``; ties go to the even index.

    ``grid`` is a sorted 1-D grid starting at 0; ``factor > 0`` is a scalar or
    an array shaped like ``t``; ``t >= 0``.  Values beyond the last point
    saturate to it.  Code parity equals the mantissa's last bit for both
    formats, so "even index" is "even mantissa".  All products
    ``factor * grid[k]`` are exact in fp64 for the factors used here.
    """
    t = np.asarray(t, dtype=np.float64)
    factor = np.broadcast_to(np.asarray(factor, dtype=np.float64), t.shape)
    n = grid.shape[0]
    # i = (number of points <= t) - 1, i.e. point[i] <= t < point[i+1]
    count = np.zeros(t.shape, dtype=np.int64)
    for g in grid:
        count += (factor * g <= t)
    i = np.clip(count - 1, 0, n - 1)
    j = np.minimum(i + 1, n - 1)
    lo = factor * grid[i]
    hi = factor * grid[j]
    twice_t = 2.0 * t
    twice_mid = lo + hi
    up = (twice_t > twice_mid) | ((twice_t == twice_mid) & (j % 2 == 0))
    return np.where(i >= n - 1, n - 1, i + up.astype(np.int64))


def e4m3_scale_code(amax: np.ndarray) -> np.ndarray:
    """Byte code of RNE_E4M3(amax / 6), saturating at 448."""
    return _nearest_code(np.asarray(amax, np.float64), 6.0, E4M3_GRID)


def e2m1_code(abs_x: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """E2M1 magnitude code (0..7) of RNE_E2M1(|x| / s) for a scale s > 0."""
    return _nearest_code(abs_x, scale, E2M1_GRID)


def fake_nvfp4(x, axis: int = -1):
    """Fake-quantize ``x`` in groups of 16 along ``axis``.

    Returns ``(x_hat, scale, scale_code, code)``:
      * ``x_hat``: fp64 array shaped like ``x``, the dequantized values (exact);
      * ``scale``: fp64 block scales, shape of ``x`` with ``axis`` -> ceil(L/16);
      * ``scale_code``: the same scales as E4M3FN bytes (uint8);
      * ``code``: the 4-bit E2M1 code per element (bit 3 = sign), uint8.
    A last group shorter than 16 is padded with zeros, which do not change
    the group's amax.
    """
    x = np.asarray(x, dtype=np.float64)
    x = np.moveaxis(x, axis, -1)
    L = x.shape[-1]
    G = -(-L // GROUP)
    pad = G * GROUP - L
    xp = np.concatenate([x, np.zeros(x.shape[:-1] + (pad,))], axis=-1) if pad else x
    xg = xp.reshape(x.shape[:-1] + (G, GROUP))
    a = np.abs(xg)
    amax = a.max(axis=-1)
    scode = e4m3_scale_code(amax)
    s = E4M3_GRID[scode]
    s_el = np.broadcast_to(s[..., None], a.shape)
    mag = np.where(s_el > 0, e2m1_code(a, np.where(s_el > 0, s_el, 1.0)), 0)
    xhat_mag = E2M1_GRID[mag] * s_el
    neg = np.signbit(xg)
    xhat = np.where(neg, -xhat_mag, xhat_mag)  # keeps -0.0 for negatives rounded to 0
    code = (mag | (neg.astype(np.int64) << 3)).astype(np.uint8)
    xhat = xhat.reshape(x.shape[:-1] + (G * GROUP,))[..., :L]
    code = code.reshape(x.shape[:-1] + (G * GROUP,))[..., :L]
    return (np.moveaxis(xhat, -1, axis), np.moveaxis(s, -1, axis),
            np.moveaxis(scode.astype(np.uint8), -1, axis), np.moveaxis(code, -1, axis))


def fake_nvfp4_values(x, axis: int = -1) -> np.ndarray:
    """Only the dequantized values of :func:`fake_nvfp4`."""
    return fake_nvfp4(x, axis)[0]
