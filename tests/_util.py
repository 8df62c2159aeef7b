"""Shared comparison helpers for the tests (no method arithmetic here)."""
from __future__ import annotations

import numpy as np

# Tolerances for floating-point results of the attention path: relative
# Frobenius error and elementwise error relative to the reference's max.
REL_FRO_TOL = 5e-3
ELEM_TOL = 2e-2


# Every check_close call appends (name, relative Frobenius error, max abs
# error, max|ref|) here; tests/conftest.py can write them out as a table.
MARGINS: list = []


def as_np64(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def rel_fro(got, ref) -> float:
    got, ref = as_np64(got), as_np64(ref)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    return float(num / den) if den > 0 else float(num)


def check_close(got, ref, name: str = "", rel_tol: float = REL_FRO_TOL,
                elem_tol: float = ELEM_TOL):
    """Relative Frobenius error <= rel_tol and max|err| <= elem_tol * max|ref|."""
    got, ref = as_np64(got), as_np64(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    rf = rel_fro(got, ref)
    amax = float(np.max(np.abs(ref))) if ref.size else 0.0
    emax = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    MARGINS.append((name, rf, emax, amax, rel_tol, elem_tol))
    assert rf <= rel_tol, f"{name}: rel Frobenius error {rf:.3e} > {rel_tol}"
    assert emax <= elem_tol * amax + 1e-30, (
        f"{name}: max abs error {emax:.3e} > {elem_tol} * max|ref| ({amax:.3e})")
    return rf, emax


def bf16_bits(x) -> np.ndarray:
    """Raw 16-bit patterns of a bf16 torch tensor."""
    import torch
    return x.detach().to("cpu").contiguous().view(torch.int16).numpy().astype(np.uint16)


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of fp64 values that are exactly representable in bf16."""
    x = np.asarray(x, dtype=np.float64)
    f32 = x.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), x, equal_nan=True), "not fp32-exact"
    bits = f32.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def fwd_plan(b: int, h: int, nq: int, nkv: int, causal: bool):
    """The library's documented key coverage of a forward: (key runs, whether
    the 32-query-tile path runs).  Non-causal with at most 32 queries per
    head: 32-query tiles, the key tiles dealt out to
    min(ceil(512 / bh), max(1, key tiles / 8)) workgroups per head.
    Otherwise (causal too) the keys are split when fewer than 256 query
    tiles of 128 exist, with at least 4 key tiles of 32 per split, for about
    512 workgroups."""
    bh, ktiles = b * h, (nkv + 31) // 32
    if not causal and nq <= 32:
        return min((512 + bh - 1) // bh, max(1, ktiles // 8)), True
    wgs = bh * ((nq + 127) // 128)
    if wgs >= 256:
        return 1, False
    s = min((512 + wgs - 1) // wgs, ktiles // 4)
    return (s if s >= 2 else 1), False


def bwd_plan(b: int, h: int, nq: int, nkv: int):
    """The library's documented split of the backward loops for small
    problems: (dQ key-loop splits, dK/dV query-loop splits).  dK/dV splits
    when the key blocks of 128 over all heads number fewer than 256, into
    min(ceil(256 / key blocks), query sub-tiles of 32 / 4); dQ when the query
    blocks of 128 number fewer than 256, into min(ceil(512 / query blocks),
    key tiles of 32 / 4); a split below 2 is none."""
    bh = b * h
    kblocks, qblocks = bh * ((nkv + 127) // 128), bh * ((nq + 127) // 128)
    dq = dkdv = 1
    if kblocks < 256:
        s = min((256 + kblocks - 1) // kblocks, ((nq + 31) // 32) // 4)
        dkdv = s if s >= 2 else 1
    if qblocks < 256:
        s = min((512 + qblocks - 1) // qblocks, ((nkv + 31) // 32) // 4)
        dq = s if s >= 2 else 1
    return dq, dkdv
