"""The forward's lazy rescale against the oracle.

The forward keeps a row's exponent base until some row of the wave sees a
tile max more than 8 (log2 units) above it; until then P = 2^(x - base) may
reach 2^8, and a larger rise rescales the accumulator mid-loop.  These
inputs make both happen late in the key loop: channel 0 of Q carries a
per-row weight in [0, 4] and channel 0 of K a few spikes at chosen keys, so
that each row's max jumps at those keys by its weight times the spike (in
log2 units up to about 3, 10, 6 and 23 for the heaviest rows, under 1 for
the lightest).  Rows of one wave then cross the threshold at different keys
or never, so per-row factors of 1 and of less than 1 occur in one rescale.
O_hp and lse are checked against the oracle forward ("NVFP4 Attention QAT
Backward", §Overview formula block; lse natural log) at the stated bar, on
the unsplit, split-over-keys and 32-query-tile paths, from bf16 and from
packed K/V, causal and not.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.attention import qat_forward_head, quantize_qkv
from tests._util import check_close, fwd_plan

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(b, h, nq, nkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, h, nq, d, generator=g)
    k = torch.randn(b, h, nkv, d, generator=g)
    v = torch.randn(b, h, nkv, d, generator=g)
    q[..., 0] = torch.linspace(0.0, 4.0, nq)
    for frac, amp in ((0.3, 6.0), (0.55, 20.0), (0.8, 12.0), (0.97, 45.0)):
        k[..., int(frac * (nkv - 1)), 0] = amp
    return q.bfloat16(), k.bfloat16(), v.bfloat16()


CASES = [  # b, h, nq, nkv, d, causal, rows checked per head (None: all)
    (1, 8, 4096, 4096, 128, False, 96),   # 256 query tiles: unsplit
    (1, 8, 4096, 4096, 64, True, 96),     # causal, unsplit
    (1, 2, 256, 4096, 128, False, None),  # split over keys
    (1, 2, 512, 512, 128, True, None),    # short causal, split over keys
    (1, 2, 16, 4096, 128, False, None),   # 32-query tiles
    (2, 2, 30, 3000, 64, False, None),    # 32-query tiles, D = 64, ragged keys
]


@pytest.mark.parametrize("b,h,nq,nkv,d,causal,nrows", CASES)
def test_forward_with_late_max_jumps_matches_oracle(b, h, nq, nkv, d, causal, nrows):
    S, dec = fwd_plan(b, h, nq, nkv, causal)
    kind = "32-query tiles" if dec else ("split" if S > 1 else "unsplit")
    print(f"[late max jumps] B{b} H{h} Nq{nq} Nkv{nkv} D{d} causal={causal}: {kind}, "
          f"{S} key runs", flush=True)
    scale = d ** -0.5
    q, k, v = _inputs(b, h, nq, nkv, d, seed=nq + nkv + d)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    p = B.problem_for(qd, kd, causal, scale)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    outs = []
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, qd, kd, vd, o, lse, ws)
    outs.append(("", o, lse))
    if not causal:
        kc, ks = B.attnqat_nvfp4_pack(kd)
        vc, vs = B.attnqat_nvfp4_pack(vd)
        o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
        B.attnqat_fwd_packed(p, qd, kc, ks, vc, vs, o2, lse2, ws)
        outs.append((" packed", o2, lse2))
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for bi in range(b):
        for hi in range(h):
            rows = (np.arange(nq) if nrows is None else
                    np.unique(np.concatenate([[0, nq - 1], rng.choice(nq, nrows, replace=False)])))
            qh, kh, vh = quantize_qkv(q[bi, hi].double().numpy(), k[bi, hi].double().numpy(),
                                      v[bi, hi].double().numpy())
            o64, l64 = qat_forward_head(qh, kh, vh, scale, causal, rows=rows, quantize=False)
            for tag, og, lg in outs:
                name = f"late max jumps {kind} Nq{nq} Nkv{nkv} D{d} causal={causal}{tag}"
                check_close(og[bi, hi, rows].cpu(), o64, f"{name} O_hp[{bi},{hi}]")
                check_close(lg[bi, hi, rows].cpu(), l64, f"{name} lse[{bi},{hi}]")
