"""GPU parity of attnqat_fake_nvfp4 against the oracle: bit-exact.

Covers every E4M3 block scale with every bf16 value that can sit in a group
of that scale (the whole E2M1 step, both signs), the zero-scale underflow,
random bf16 and fp32 tensors of several row lengths, in-place use, and the
empty input.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.nvfp4 import fake_nvfp4
from tests._util import bf16_bits, f64_to_bf16_bits
from workloads import random_bf16, random_f32

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _all_positive_bf16() -> np.ndarray:
    bits = np.arange(1, 0x7F80, dtype=np.uint32)
    return (bits << 16).view(np.float32).astype(np.float64)


def _e4m3_values() -> np.ndarray:
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _crafted_groups() -> np.ndarray:
    """Groups [6*s, x_1..x_15] for every E4M3 scale s: the first element fixes
    the scale at exactly s, the other 15 sweep every bf16 value of magnitude
    <= 6*s with both signs.  Plus groups whose amax makes the scale 0."""
    pos = _all_positive_bf16()
    rows = []
    for s in _e4m3_values()[1:]:
        xs = pos[pos <= 6 * s]
        vals = np.concatenate([xs, -xs])
        pad = (-len(vals)) % 15
        vals = np.concatenate([vals, np.zeros(pad)]).reshape(-1, 15)
        rows.append(np.concatenate([np.full((len(vals), 1), 6 * s), vals], axis=1))
    tiny = pos[pos <= 6 * 2.0 ** -10]
    tiny = np.concatenate([tiny, np.zeros((-len(tiny)) % 16)]).reshape(-1, 16)
    rows.append(tiny)
    rows.append(-tiny)
    return np.concatenate(rows, axis=0)


def _run_bf16(x64: np.ndarray):
    x = torch.from_numpy(x64.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.double().numpy(), x64)
    xd = x.to(DEV)
    xh, sc = B.attnqat_fake_nvfp4(xd)
    torch.cuda.synchronize()
    return xh.cpu(), sc.cpu()


def _compare_bf16(x64, xh_gpu, sc_gpu):
    ref, _, scode, _ = fake_nvfp4(x64)
    got_bits = bf16_bits(xh_gpu)
    want_bits = f64_to_bf16_bits(ref)
    bad = np.nonzero(got_bits != want_bits)
    assert bad[0].size == 0, (
        f"{bad[0].size} mismatches, first at {tuple(i[0] for i in bad)}: "
        f"x={x64[tuple(i[0] for i in bad)]} got={got_bits[tuple(i[0] for i in bad)]:#06x} "
        f"want={want_bits[tuple(i[0] for i in bad)]:#06x}")
    assert np.array_equal(sc_gpu.numpy(), scode)


def test_every_scale_and_every_bf16_value():
    x64 = _crafted_groups()
    print(f"[fake_nvfp4 exhaustive] groups={x64.shape[0]}", flush=True)
    xh, sc = _run_bf16(x64)
    _compare_bf16(x64, xh, sc)


@pytest.mark.parametrize("shape,dist,seed,scale", [
    ((4096, 128), "normal", 1, 1.0),
    ((1000, 64), "loguniform", 2, 1.0),
    ((333, 16), "normal", 3, 1e-3),
    ((257, 48), "normal", 4, 500.0),
    ((2, 3, 77, 128), "loguniform", 5, 1.0),
])
def test_random_bf16(shape, dist, seed, scale):
    x = random_bf16(shape, seed, scale=scale, dist=dist)
    x64 = x.double().numpy()
    xh, sc = B.attnqat_fake_nvfp4(x.to(DEV))
    torch.cuda.synchronize()
    _compare_bf16(x64, xh.cpu(), sc.cpu())


@pytest.mark.parametrize("shape,seed,scale", [((2048, 128), 7, 1.0), ((300, 32), 8, 1e-4),
                                              ((64, 16), 9, 1e4)])
def test_random_f32(shape, seed, scale):
    x = random_f32(shape, seed, scale)
    # widen the dynamic range per row
    x = x * torch.exp2(torch.arange(shape[0]).float().remainder(24) - 12)[:, None]
    x64 = x.double().numpy()
    xh, sc = B.attnqat_fake_nvfp4(x.to(DEV))
    torch.cuda.synchronize()
    ref, _, scode, _ = fake_nvfp4(x64)
    got = xh.cpu().double().numpy()
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.array_equal(sc.cpu().numpy(), scode)


def test_f32_values_at_and_beside_every_midpoint():
    """fp32 inputs at every E2M1 midpoint times every E4M3 scale, and 1-3 fp32
    ulps to either side: the fp32 path shares its rounding code with the
    probability quantization of the dK/dV kernel."""
    scales = _e4m3_values()[1:]
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 1.0, 2.0, 4.0])
    groups = []
    for s in scales:
        base = (mids * s).astype(np.float32)
        vals = [base]
        for k in (1, 2, 3):
            vals.append(np.nextafter(base, np.float32(np.inf)))
            vals.append(np.nextafter(base, np.float32(0)))
            base_up, base_dn = vals[-2], vals[-1]
            for _ in range(k - 1):
                base_up = np.nextafter(base_up, np.float32(np.inf))
                base_dn = np.nextafter(base_dn, np.float32(0))
            vals[-2], vals[-1] = base_up, base_dn
        v = np.concatenate(vals).astype(np.float64)
        v = np.concatenate([v, -v])
        pad = (-len(v)) % 15
        v = np.concatenate([v, np.zeros(pad)]).reshape(-1, 15)
        groups.append(np.concatenate([np.full((len(v), 1), 6 * s), v], axis=1))
    x64 = np.concatenate(groups)
    x = torch.from_numpy(x64.astype(np.float32))
    assert np.array_equal(x.double().numpy(), x64)
    xh, sc = B.attnqat_fake_nvfp4(x.to(DEV))
    torch.cuda.synchronize()
    ref, _, scode, _ = fake_nvfp4(x64)
    got = xh.cpu().double().numpy()
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, (x64[bad][:5], got[bad][:5], ref[bad][:5])
    assert np.array_equal(np.signbit(got), np.signbit(ref))
    assert np.array_equal(sc.cpu().numpy(), scode)


def test_in_place_and_without_scales():
    x = random_bf16((512, 128), 10)
    x64 = x.double().numpy()
    xd = x.to(DEV)
    sc = torch.empty((512, 8), dtype=torch.uint8, device=DEV)
    B.attnqat_fake_nvfp4(xd, x_hat=xd, scales=sc)
    torch.cuda.synchronize()
    _compare_bf16(x64, xd.cpu(), sc.cpu())
    # NULL scales pointer: only values are written
    y = random_bf16((64, 64), 11).to(DEV)
    out = torch.empty_like(y)
    st = B._lib.attnqat_fake_nvfp4(B._ptr(y), B.DTYPE_BF16, B._ptr(out), None, 64, 64,
                                   B._stream(None))
    assert st == B.OK
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out.cpu()), f64_to_bf16_bits(fake_nvfp4(y.cpu().double().numpy())[0]))


def test_empty_and_misaligned():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    xh, sc = B.attnqat_fake_nvfp4(x)
    assert xh.numel() == 0
    base = torch.zeros(16 * 64 + 8, dtype=torch.bfloat16, device=DEV)
    bad = base[1:1 + 16 * 64].view(16, 64)  # 2-byte offset
    with pytest.raises(B.AttnQatError) as e:
        B.attnqat_fake_nvfp4(bad, x_hat=torch.empty_like(bad),
                             scales=torch.empty(16, 4, dtype=torch.uint8, device=DEV))
    assert e.value.status == B.ERR_MISALIGNED


def test_scale_at_every_e4m3_rounding_boundary():
    """The block scale is the E4M3 rounding (ties to even, saturating at 448)
    of amax/6.  Groups whose amax is 6 times every E4M3 midpoint, nudged by
    0..4 fp32 ulps either way, plus every positive bf16 amax up to 6 * 480:
    the scale bytes and the dequantized values are bit-exact to the oracle
    (fp32 path, which shares the device scale arithmetic of every kernel)."""
    g = _e4m3_values()
    mids = np.concatenate([[2.0 ** -10], (g[:-1] + g[1:]) / 2, [464.0, 470.0, 480.0, 1e4]])
    amax = []
    for m in (6.0 * mids).astype(np.float32):
        up = dn = m
        amax.append(m)
        for _ in range(4):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
            amax += [up, dn]
    bf = _all_positive_bf16()
    amax = np.concatenate([np.array(amax, dtype=np.float64), bf[bf <= 6 * 480.0]])
    x64 = np.zeros((amax.size, 16))
    x64[:, 0] = amax
    x64[:, 1] = amax / 3.0  # a second value rounded with the same scale
    x64 = x64.astype(np.float32).astype(np.float64)
    x = torch.from_numpy(x64.astype(np.float32))
    xh, sc = B.attnqat_fake_nvfp4(x.to(DEV))
    torch.cuda.synchronize()
    ref, _, scode, _ = fake_nvfp4(x64)
    assert np.array_equal(sc.cpu().numpy(), scode)
    assert np.array_equal(xh.cpu().double().numpy(), ref)
