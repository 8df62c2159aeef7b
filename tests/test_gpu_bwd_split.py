"""The backward on small problems, with its loops split over workgroups.

When a problem's key blocks (128 keys) cannot fill the chip, attnqat_bwd
splits the dK/dV kernel's loop over query sub-tiles; when its query blocks
(128 queries) cannot fill it, the dQ kernel's loop over key tiles.  Each
split writes fp32 partial sums that a reduction adds in a fixed order.  The
result is the same QAT backward ("NVFP4 Attention QAT Backward", §Overview
formula block), so it is checked against the oracle at the stated bar
(relative Frobenius error 5e-3, elementwise 2e-2 * max|ref|) through the
same full-case protocol as the unsplit shapes (forward, quantized
workspace, backward on the oracle forward's rounded outputs, and the GPU
forward -> GPU backward chain).  The cases cover both splits, the dQ split
alone, causal key blocks whose later splits get no queries (and query
blocks whose later splits get no keys), ragged tails and both head sizes;
results must also be bitwise repeatable.
"""
from __future__ import annotations

import math

import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from tests._util import bwd_plan
from tests.test_gpu_attention import DEV, run_full_case

pytestmark = pytest.mark.gpu


def _synthetic(b, h, nq, nkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda m: torch.randn(b, h, m, d, generator=g).to(torch.bfloat16)  # noqa: E731
    return mk(nq), mk(nkv), mk(nkv), mk(nq)


CASES = [  # b, h, nq, nkv, d, causal, heads checked (None: all)
    (1, 16, 1024, 1024, 128, False, [(0, 0), (0, 7), (0, 15)]),  # dQ 4 splits, dK/dV 2
    (1, 2, 1024, 1024, 64, True, None),   # 8 and 8: the causal ends get empty splits
    (1, 2, 333, 333, 128, True, None),    # 2 and 2, ragged tails
    (2, 3, 640, 1000, 64, False, [(0, 0), (1, 2)]),  # dQ 8, dK/dV 5, cross-attention
    (1, 2, 100, 260, 128, False, None),   # dQ split only
]


@pytest.mark.parametrize("b,h,nq,nkv,d,causal,heads", CASES)
def test_split_backward_matches_oracle(b, h, nq, nkv, d, causal, heads):
    sq, skv = bwd_plan(b, h, nq, nkv)
    assert sq > 1 or skv > 1, "the case must split a backward loop"
    q, k, v, do = _synthetic(b, h, nq, nkv, d, seed=7 * nq + nkv + d)
    run_full_case(q, k, v, do, causal, 1.0 / math.sqrt(d), heads=heads,
                  label=f"split loops q{sq} kv{skv}")


def test_split_backward_is_bitwise_repeatable():
    b, h, n, d = 1, 4, 1024, 64
    q, k, v, do = (t.to(DEV) for t in _synthetic(b, h, n, n, d, seed=5))
    p = B.problem_for(q, k, True, 0.125)
    assert bwd_plan(b, h, n, n) == (8, 8)
    wsf = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, q, k, v, o, lse, wsf)
    outs = []
    for fill in (0, 255):
        ws = torch.full((B.attnqat_bwd_workspace_bytes(p),), fill, dtype=torch.uint8, device=DEV)
        g = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        B.attnqat_bwd(p, q, k, v, o, do, lse, *g, ws)
        torch.cuda.synchronize()
        outs.append(g)
    for a_, b_ in zip(*outs):
        assert torch.equal(a_.view(torch.int16), b_.view(torch.int16))
