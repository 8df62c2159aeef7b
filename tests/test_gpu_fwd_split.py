"""The forward over few queries or a short problem: split over keys, or in
32-query tiles.

When the 128-query tiles of all heads cannot fill the chip, attnqat_fwd and
attnqat_fwd_packed split the keys over workgroups (causal problems too: a
split whose keys all lie above a query tile's diagonal contributes nothing);
non-causal problems with at most 32 queries per head run 32-query tiles
whose four waves take separate key runs.  Either way the runs' partial results
(unnormalized O, row max and row sum) are merged into O_hp and lse.  The
result is the same QAT forward ("NVFP4 Attention QAT Backward", §Overview
formula block; lse natural log, §Tensor contract), so it is checked against
the oracle forward at the stated bar (relative Frobenius error 5e-3,
elementwise 2e-2 * max|ref|), from bf16 K/V and from packed NVFP4 K/V (the
storage of the Attn-QAT summary's "FP4 only where it's free").  The cases
include a single query, a single key, ragged key counts (tails inside the
last run), runs and waves without keys, and both head sizes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.attention import qat_forward_head
from oracle.nvfp4 import fake_nvfp4
from tests._util import check_close, f64_to_bf16_bits, fwd_plan

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(b, h, nq, nkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, h, nq, d, generator=g)
    k = torch.randn(b, h, nkv, d, generator=g)
    v = torch.randn(b, h, nkv, d, generator=g)
    # a few large channels, as in the outlier workload, so the scales differ
    k[..., : d // 16] *= 4.0
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


CASES = [  # b, h, nq, nkv, d
    # split over keys (more than 32 queries)
    (1, 4, 64, 3001, 64),
    (2, 3, 100, 8192, 128),
    (1, 2, 130, 2500, 128),   # two query tiles, ragged keys
    (1, 1, 40, 300, 64),      # two splits of 5 tiles, the last tile 12 keys
    # 32-query tiles (at most 32 queries)
    (1, 2, 16, 4100, 128),    # 64 waves per head over 129 tiles: wave 0 takes three, the tail among them
    (1, 1, 1, 20000, 128),    # a single query
    (1, 3, 32, 1000, 64),     # a full query tile
    (2, 2, 5, 77, 128),       # one workgroup per head: three waves of one tile (the last 13 keys), one idle
    (1, 1, 17, 1, 64),        # a single key (three idle waves)
    (3, 5, 9, 2049, 128),     # the last tile holds one key
    (1, 1, 24, 65536, 64),    # long keys
    (8, 32, 4, 2000, 128),    # 256 heads: two key runs per head
    (4, 8, 30, 3000, 64),     # 32 heads, D = 64
]


CAUSAL_CASES = [  # b, h, n, d: short causal problems, split over keys
    (1, 4, 1024, 64),   # 8 splits: the first query tiles' later splits get no keys
    (1, 2, 300, 128),   # 2 splits, ragged tail
]


@pytest.mark.parametrize("b,h,n,d", CAUSAL_CASES)
def test_short_causal_forward_matches_oracle(b, h, n, d):
    _run(b, h, n, n, d, causal=True)


@pytest.mark.parametrize("b,h,nq,nkv,d", CASES)
def test_few_query_forward_matches_oracle(b, h, nq, nkv, d):
    _run(b, h, nq, nkv, d, causal=False)


def _run(b, h, nq, nkv, d, causal):
    scale = d ** -0.5
    q, k, v = _inputs(b, h, nq, nkv, d, seed=nq * 7 + nkv)
    S, dec = fwd_plan(b, h, nq, nkv, causal)
    assert dec or S > 1, "the case must split the keys or take the 32-query tiles"
    kind = "32-query tiles" if dec else "split"
    print(f"[few-query fwd] B{b} H{h} Nq{nq} Nkv{nkv} D{d} causal={causal}: {kind}, "
          f"{S} key runs", flush=True)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    p = B.problem_for(qd, kd, causal, scale)
    # 0xFF-filled: the call must write Q^, K^, V^ and their scales itself
    ws = torch.full((B.attnqat_fwd_workspace_bytes(p),), 0xFF, dtype=torch.uint8, device=DEV)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, qd, kd, vd, o, lse, ws)
    torch.cuda.synchronize()
    L = B.attnqat_workspace_layout(p, B.WS_FWD)
    parts = {}
    for name, t in (("q", q), ("k", k), ("v", v)):
        n = t.numel()
        parts[name] = (ws[L[f"{name}_hat"]:L[f"{name}_hat"] + 2 * n].view(torch.int16)
                       .view(t.shape).cpu(),
                       ws[L[f"{name}_scale"]:L[f"{name}_scale"] + n // 16]
                       .view(*t.shape[:3], d // 16).cpu())
    # the same forward from packed NVFP4 K/V
    kc, ks = B.attnqat_nvfp4_pack(kd)
    vc, vs = B.attnqat_nvfp4_pack(vd)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    ws2 = torch.full_like(ws, 0xFF)  # the packed call must write Q^ and its scales itself
    B.attnqat_fwd_packed(p, qd, kc, ks, vc, vs, o2, lse2, ws2)
    torch.cuda.synchronize()
    nqh = b * h * nq * d
    qhat = ws2[L["q_hat"]:L["q_hat"] + 2 * nqh].view(torch.int16).view(b, h, nq, d).cpu()
    qsc = ws2[L["q_scale"]:L["q_scale"] + nqh // 16].view(b, h, nq, d // 16).cpu()
    for bi in range(b):
        for hi in range(h):
            # Q^, K^, V^ and their scale bytes (the oracle's fake_nvfp4)
            fq = {name: fake_nvfp4(t[bi, hi].double().numpy())
                  for name, t in (("q", q), ("k", k), ("v", v))}
            qh, kh, vh = fq["q"][0], fq["k"][0], fq["v"][0]
            assert np.array_equal(qhat[bi, hi].numpy().view(np.uint16), f64_to_bf16_bits(qh))
            assert np.array_equal(qsc[bi, hi].numpy(), fq["q"][2])
            # the bf16 call's workspace (written by the quantization pass, or
            # by the 32-query-tile kernel itself)
            for name in ("q", "k", "v"):
                xh, xs = parts[name]
                assert np.array_equal(xh[bi, hi].numpy().view(np.uint16),
                                      f64_to_bf16_bits(fq[name][0])), (name, bi, hi)
                assert np.array_equal(xs[bi, hi].numpy(), fq[name][2]), (name, bi, hi)
            o64, l64 = qat_forward_head(qh, kh, vh, scale, causal, quantize=False)
            tag = f"{kind} Nq{nq} Nkv{nkv} D{d} causal={causal}"
            check_close(o[bi, hi].cpu(), o64, f"{tag} O_hp[{bi},{hi}]")
            check_close(lse[bi, hi].cpu(), l64, f"{tag} lse[{bi},{hi}]")
            check_close(o2[bi, hi].cpu(), o64, f"{tag} packed O_hp[{bi},{hi}]")
            check_close(lse2[bi, hi].cpu(), l64, f"{tag} packed lse[{bi},{hi}]")
    # packed and bf16 K/V give the same values up to the fp32 rounding order
    assert torch.allclose(o.float(), o2.float(), rtol=1e-2, atol=1e-3)
    assert torch.allclose(lse, lse2, rtol=1e-5, atol=1e-5)

