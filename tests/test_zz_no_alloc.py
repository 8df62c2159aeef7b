"""attnqat_bwd_noalloc (the backward with the library's static device
workspace, for callers that cannot allocate) against attnqat_bwd: the same
kernels, so the outputs must be bit-identical.  Calls in a row on one GPU,
each smaller than the one before (the static array keeps the previous call's
contents), and a problem whose workspace exceeds the array is rejected.  A
small problem whose split-loop partial sums would not fit beside the rest
runs its loops unsplit instead: its outputs then equal attnqat_bwd's up to
the fp32 rounding order of the partial sums and one bf16 rounding."""
from __future__ import annotations

import math

import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from tests._util import rel_fro

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(b, h, n, d, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda: torch.randn(b, h, n, d, generator=g).to(torch.bfloat16).to(DEV)
    return mk(), mk(), mk(), mk()


def _both(b, h, n, d, causal, seed, exact=True):
    q, k, v, do = _inputs(b, h, n, d, seed)
    p = B.problem_for(q, k, causal, 1.0 / math.sqrt(d))
    wsf = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, q, k, v, o, lse, wsf)
    ref = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    wsb = torch.empty(B.attnqat_bwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    B.attnqat_bwd(p, q, k, v, o, do, lse, *ref, wsb)
    got = [torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
           torch.full_like(v, float("nan"))]
    B.attnqat_bwd_noalloc(p, q, k, v, o, do, lse, *got)
    torch.cuda.synchronize()
    print(f"[noalloc] B{b} H{h} N{n} D{d} causal={causal} workspace "
          f"{B.attnqat_bwd_workspace_bytes(p)} bytes", flush=True)
    for r, g_ in zip(ref, got):
        if exact:
            assert torch.equal(r.view(torch.int16), g_.view(torch.int16))
        else:
            assert rel_fro(g_, r) <= 2e-3, rel_fro(g_, r)


def test_noalloc_backward_matches_backward_on_consecutive_calls():
    # the reference shape (workspace 52.2 MB of the 64 MiB array), then two
    # smaller problems, each reusing the array the previous call left
    _both(1, 16, 4096, 128, False, seed=1)
    _both(1, 4, 1000, 128, True, seed=2)
    _both(2, 3, 333, 64, False, seed=3)


def test_noalloc_runs_small_problems_unsplit_when_the_partials_do_not_fit():
    # B1 H16 N1024 D128: 80.5 MB with the split loops' partial sums, 13.5 MB
    # without; the previous test left the array holding other contents
    p = B.make_problem(1, 16, 1024, 1024, 128, False, 1.0 / math.sqrt(128))
    assert B.attnqat_bwd_workspace_bytes(p) > B.NOALLOC_MAX_WORKSPACE_BYTES
    _both(1, 16, 1024, 128, False, seed=5, exact=False)
    _both(1, 2, 512, 64, True, seed=6)  # then a smaller one that splits again


def test_noalloc_rejects_a_workspace_beyond_the_array():
    q, k, v, do = _inputs(1, 1, 64, 128, seed=4)
    p = B.make_problem(2, 40, 8192, 8192, 128, True, 1.0 / math.sqrt(128))
    assert B.attnqat_bwd_workspace_bytes(p) > B.NOALLOC_MAX_WORKSPACE_BYTES
    lse = torch.zeros(1, 1, 64, device=DEV)
    rc = B._lib.attnqat_bwd_noalloc(B.ctypes.byref(p), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    q.data_ptr(), do.data_ptr(), lse.data_ptr(), q.data_ptr(),
                                    k.data_ptr(), v.data_ptr(), None)
    assert rc == B.ERR_UNSUPPORTED
