"""Packed NVFP4 storage (attnqat_nvfp4_pack) and the forward that reads K^/V^
from it (attnqat_fwd_packed).

The packed codes and scale bytes are bit-exact to the oracle's E2M1 codes
and E4M3FN bytes ("NVFP4 Attention QAT Backward", §Overview rounding; the
nibble order is the one documented in the header).  The packed forward's
O_hp and lse are checked against the oracle forward at the stated bar
(relative Frobenius error 5e-3, elementwise 2e-2 * max|ref|); since its
dequantization is exact it also agrees with attnqat_fwd to within fp32
rounding order (a much tighter check of the same kernel pipeline).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.attention import qat_forward_head
from oracle.nvfp4 import fake_nvfp4
from tests._util import REL_FRO_TOL, check_close, rel_fro
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _oracle_packed(x):
    """Oracle codes packed two to a byte (element 2i low nibble) and scale bytes."""
    _, _, scode, code = fake_nvfp4(x.double().numpy())
    code = code.astype(np.uint8)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.astype(np.uint8), scode


def _tie_heavy(rows, L, seed):
    """bf16 values that sit exactly on E2M1 midpoints and grid points of
    E4M3 scales, plus zeros, negative zeros, tiny and saturating values."""
    g = torch.Generator().manual_seed(seed)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0,
                         6.0, 0.0, 7.0])
    s = 2.0 ** torch.randint(-8, 6, (rows, L // 16, 1), generator=g).float()
    v = mids[torch.randint(0, 16, (rows, L // 16, 16), generator=g)] * s
    # one element per group sets the group's amax to 6 s exactly
    v[..., 0] = 6.0 * s[..., 0]
    sign = torch.where(torch.rand(rows, L // 16, 16, generator=g) < 0.5, -1.0, 1.0)
    v = (v * sign).reshape(rows, L)
    v[0, :16] = -0.0
    v[1 % rows, 16:32] = 1e-30
    return v.to(torch.bfloat16)


@pytest.mark.parametrize("rows,L,kind", [(1, 16, "randn"), (37, 64, "randn"), (512, 128, "randn"),
                                         (300, 128, "ties"), (64, 256, "ties"),
                                         (1000, 64, "loguniform")])
def test_pack_is_bit_exact(rows, L, kind):
    g = torch.Generator().manual_seed(rows + L)
    if kind == "randn":
        x = torch.randn(rows, L, generator=g).to(torch.bfloat16)
    elif kind == "ties":
        x = _tie_heavy(rows, L, seed=rows)
    else:
        x = (torch.exp(torch.empty(rows, L).uniform_(-60, 60, generator=g)) *
             torch.where(torch.rand(rows, L, generator=g) < 0.5, -1.0, 1.0)).to(torch.bfloat16)
    codes, scales = B.attnqat_nvfp4_pack(x.to(DEV))
    torch.cuda.synchronize()
    ref_codes, ref_scales = _oracle_packed(x)
    assert np.array_equal(codes.cpu().numpy(), ref_codes)
    assert np.array_equal(scales.cpu().numpy(), ref_scales)
    # the packed form decodes to fake_nvfp4's values
    xh, sc = B.attnqat_fake_nvfp4(x.to(DEV))
    assert torch.equal(sc, scales)


def _fwd(q, k, v, causal, scale, packed):
    p = B.problem_for(q, k, causal, scale)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    if packed:
        kc, ks = B.attnqat_nvfp4_pack(k)
        vc, vs = B.attnqat_nvfp4_pack(v)
        B.attnqat_fwd_packed(p, q, kc, ks, vc, vs, o, lse, ws)
    else:
        B.attnqat_fwd(p, q, k, v, o, lse, ws)
    torch.cuda.synchronize()
    return o, lse


def _synthetic(n, d, seed, nk=None, heads=2):
    g = torch.Generator().manual_seed(seed)
    nk = n if nk is None else nk
    mk = lambda m: torch.randn(1, heads, m, d, generator=g).to(torch.bfloat16).to(DEV)
    return mk(n), mk(nk), mk(nk)


def _check_packed_forward(q, k, v, causal, scale, heads, label):
    """Packed forward against the oracle forward on the given heads, and
    against attnqat_fwd: lse to within the fp32 rounding order; O_hp to
    within one bf16 rounding of O_hp and the fp32 rounding order, except
    with at most 32 non-causal queries per head, where the packed kernel
    rounds P to fp16 instead of bf16 before P V^ (then both are held to the
    stated bar against each other, as each is against the oracle)."""
    o1, l1 = _fwd(q, k, v, causal, scale, packed=False)
    o2, l2 = _fwd(q, k, v, causal, scale, packed=True)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    for b_, h in heads:
        o64, l64 = qat_forward_head(qc[b_, h], kc[b_, h], vc[b_, h], scale, causal)
        check_close(o2[b_, h].cpu(), o64, f"{label} packed O_hp[{b_},{h}]")
        check_close(l2[b_, h].cpu(), l64, f"{label} packed lse[{b_},{h}]")
    # one bf16 rounding of O_hp, fp32 rounding order of the softmax sums
    # (bf16 against fp16 probabilities on the 32-query-tile path)
    fp16_p = not causal and q.shape[2] <= 32
    assert rel_fro(o2, o1) <= (REL_FRO_TOL if fp16_p else 1e-3), (label, rel_fro(o2, o1))
    assert rel_fro(l2, l1) <= 1e-6, (label, rel_fro(l2, l1))


@pytest.mark.parametrize("n,d,causal,nk", [
    (128, 64, False, None), (200, 64, True, None), (333, 128, False, None), (77, 64, True, None),
    (100, 128, False, 260), (300, 64, False, 40), (1, 128, True, None), (17, 64, False, None),
])
def test_packed_forward_matches_oracle(n, d, causal, nk):
    q, k, v = _synthetic(n, d, seed=n + 3 * d, nk=nk)
    _check_packed_forward(q, k, v, causal, 1.0 / math.sqrt(d), [(0, 0), (0, 1)],
                          f"n={n} d={d} causal={causal} nk={nk}")


@pytest.mark.parametrize("name,heads", [("ref_shape", [(0, 0), (0, 8), (0, 15)]),
                                        ("small_causal", [(0, 0), (0, 1), (0, 2), (0, 3)])])
def test_packed_forward_on_workloads(name, heads):
    w = WORKLOADS[name]
    q, k, v, _ = (t.to(DEV) for t in make_inputs(w))
    _check_packed_forward(q, k, v, w.causal, w.softmax_scale, heads, name)


def test_pack_and_packed_forward_reject_bad_arguments():
    x = torch.zeros(4, 32, dtype=torch.bfloat16, device=DEV)
    codes = torch.full((4, 16), 7, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(4, 2, dtype=torch.uint8, device=DEV)
    lib = B._lib
    assert lib.attnqat_nvfp4_pack(x.data_ptr(), None, scales.data_ptr(), 4, 32, None) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_nvfp4_pack(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), 4, 24,
                                  None) == B.ERR_INVALID_ARGUMENT
    base = torch.zeros(80, dtype=torch.uint8, device=DEV)
    assert lib.attnqat_nvfp4_pack(x.data_ptr(), base[4:].data_ptr(), scales.data_ptr(), 4, 32,
                                  None) == B.ERR_MISALIGNED
    torch.cuda.synchronize()
    assert torch.all(codes == 7)
    q, k, v = _synthetic(64, 128, seed=1, heads=1)
    p = B.problem_for(q, k, False, 0.1)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    kc, ks = B.attnqat_nvfp4_pack(k)
    rc = lib.attnqat_fwd_packed(B.ctypes.byref(p), q.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                None, ks.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                ws.data_ptr(), ws.numel(), None)
    assert rc == B.ERR_INVALID_ARGUMENT
    rc = lib.attnqat_fwd_packed(B.ctypes.byref(p), q.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                kc.data_ptr(), ks.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                ws.data_ptr(), 100, None)
    assert rc == B.ERR_WORKSPACE_TOO_SMALL
