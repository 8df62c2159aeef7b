"""The forward split over keys: few queries against long K/V.

When the 128-query tiles of all heads cannot fill the chip and the problem is
non-causal, attnqat_fwd and attnqat_fwd_packed split the keys over
workgroups and merge the splits' partial results (unnormalized O, row max
and row sum) into O_hp and lse.  The result is the same QAT forward
("NVFP4 Attention QAT Backward", §Overview formula block; lse natural log,
§Tensor contract), so it is checked against the oracle forward at the
stated bar (relative Frobenius error 5e-3, elementwise 2e-2 * max|ref|),
from bf16 K/V and from packed NVFP4 K/V (the storage of the Attn-QAT
summary's "FP4 only where it's free").  The cases include a single query,
ragged key counts (tails inside the last split), splits without keys and
both head sizes.
"""
from __future__ import annotations

import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.attention import qat_forward_head, quantize_qkv
from tests._util import check_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _splits(b, h, nq, nkv):
    """The library's documented split policy (non-causal): enough splits for
    about 512 workgroups when fewer than 256 query tiles exist, at least 4
    key tiles of 32 keys per split."""
    wgs = b * h * ((nq + 127) // 128)
    if wgs >= 256:
        return 1
    s = min((512 + wgs - 1) // wgs, ((nkv + 31) // 32) // 4)
    return s if s >= 2 else 1


def _inputs(b, h, nq, nkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, h, nq, d, generator=g)
    k = torch.randn(b, h, nkv, d, generator=g)
    v = torch.randn(b, h, nkv, d, generator=g)
    # a few large channels, as in the outlier workload, so the scales differ
    k[..., : d // 16] *= 4.0
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


CASES = [  # b, h, nq, nkv, d
    (1, 2, 16, 4100, 128),    # 129 key tiles in 32 splits of 5: the last 6 splits are empty
    (1, 4, 64, 3001, 64),
    (2, 3, 100, 8192, 128),
    (1, 1, 1, 20000, 128),    # a single query
    (1, 2, 130, 2500, 128),   # two query tiles, ragged keys
    (1, 1, 40, 300, 64),      # two splits of 5 tiles, the last tile 12 keys
]


@pytest.mark.parametrize("b,h,nq,nkv,d", CASES)
def test_split_forward_matches_oracle(b, h, nq, nkv, d):
    scale = d ** -0.5
    q, k, v = _inputs(b, h, nq, nkv, d, seed=nq * 7 + nkv)
    S = _splits(b, h, nq, nkv)
    assert S > 1, "the case must take the split path"
    print(f"[split fwd] B{b} H{h} Nq{nq} Nkv{nkv} D{d}: {S} key splits", flush=True)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    p = B.problem_for(qd, kd, False, scale)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, qd, kd, vd, o, lse, ws)
    # the same forward from packed NVFP4 K/V
    kc, ks = B.attnqat_nvfp4_pack(kd)
    vc, vs = B.attnqat_nvfp4_pack(vd)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    B.attnqat_fwd_packed(p, qd, kc, ks, vc, vs, o2, lse2, ws)
    torch.cuda.synchronize()
    for bi in range(b):
        for hi in range(h):
            qh, kh, vh = quantize_qkv(q[bi, hi].double().numpy(), k[bi, hi].double().numpy(),
                                      v[bi, hi].double().numpy())
            o64, l64 = qat_forward_head(qh, kh, vh, scale, False, quantize=False)
            tag = f"split Nq{nq} Nkv{nkv} D{d}"
            check_close(o[bi, hi].cpu(), o64, f"{tag} O_hp[{bi},{hi}]")
            check_close(lse[bi, hi].cpu(), l64, f"{tag} lse[{bi},{hi}]")
            check_close(o2[bi, hi].cpu(), o64, f"{tag} packed O_hp[{bi},{hi}]")
            check_close(lse2[bi, hi].cpu(), l64, f"{tag} packed lse[{bi},{hi}]")
    # packed and bf16 K/V give the same values up to the fp32 rounding order
    assert torch.allclose(o.float(), o2.float(), rtol=1e-2, atol=1e-3)
    assert torch.allclose(lse, lse2, rtol=1e-5, atol=1e-5)

