"""GPU parity of the quantized forward output (attnqat_fwd_quantized).

O = fake_nvfp4(P) V^ with P the normalized softmax and the P groups of 16
consecutive keys from key 0 (Attn-QAT summary, §Method; the reading is the
oracle's, ``qat_forward_quantized_head``).  Bar: relative Frobenius error
5e-3 and elementwise error 2e-2 * max|ref| against the fp64 oracle; O_hp and
lse from the same call equal attnqat_fwd's bit for bit.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from oracle.attention import qat_forward_quantized_head
from tests._util import check_close
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def gpu_fwd_quantized(q, k, v, causal, scale, p_scale=1.0):
    p = B.problem_for(q, k, causal, scale, p_scale)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o_hp = torch.empty_like(q)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd_quantized(p, q, k, v, o_hp, lse, o, ws)
    # the first pass alone, for comparison
    o_hp2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)
    B.attnqat_fwd(p, q, k, v, o_hp2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(o_hp, o_hp2) and torch.equal(lse, lse2)
    return o


def run_case(q, k, v, causal, scale, p_scale=1.0, heads=None, rows=None, label=""):
    Bb, H = q.shape[:2]
    heads = [(b, h) for b in range(Bb) for h in range(H)] if heads is None else heads
    print(f"[fwd output parity] {label} shape={tuple(q.shape)} nkv={k.shape[2]} "
          f"causal={causal} p_scale={p_scale} heads={heads}", flush=True)
    o = gpu_fwd_quantized(q.to(DEV), k.to(DEV), v.to(DEV), causal, scale, p_scale).cpu()
    for b, h in heads:
        r = np.arange(q.shape[2]) if rows is None else rows
        ref = qat_forward_quantized_head(q[b, h], k[b, h], v[b, h], scale, causal, p_scale,
                                         rows=r)
        err = check_close(o[b, h, r], ref, f"{label} O[{b},{h}]")
        print(f"  [{b},{h}] rel err O {err[0]:.2e}", flush=True)


def _synthetic(n, d, seed, nk=None, heads=1):
    g = torch.Generator().manual_seed(seed)
    nk = n if nk is None else nk
    mk = lambda m: torch.randn(1, heads, m, d, generator=g).to(torch.bfloat16)
    return mk(n), mk(nk), mk(nk)


@pytest.mark.parametrize("p_scale", [1.0, 2688.0])
def test_tiny_workload(p_scale):
    w = WORKLOADS["tiny"]
    q, k, v, _ = make_inputs(w)
    run_case(q, k, v, w.causal, w.softmax_scale, p_scale, label="tiny")


@pytest.mark.parametrize("p_scale", [1.0, 2688.0])
def test_small_causal_workload(p_scale):
    w = WORKLOADS["small_causal"]
    q, k, v, _ = make_inputs(w)
    run_case(q, k, v, w.causal, w.softmax_scale, p_scale, label="small_causal")


@pytest.mark.timeout(600)
def test_ref_shape_workload():
    w = WORKLOADS["ref_shape"]
    q, k, v, _ = make_inputs(w)
    rows = np.sort(np.random.default_rng(5).choice(w.seqlen, 256, replace=False))
    for p_scale in (1.0, 2688.0):
        run_case(q, k, v, w.causal, w.softmax_scale, p_scale, heads=[(0, 0), (0, 15)],
                 rows=rows, label="ref_shape")


@pytest.mark.timeout(900)
def test_video_dit_workload_sampled():
    """N = 32760: the last 8-key group of every row is a partial group."""
    w = WORKLOADS["video_dit"]
    q, k, v, _ = make_inputs(w, heads=2)
    N = w.seqlen
    rows = np.unique(np.concatenate([[0, 1, N - 57, N - 1],
                                     np.random.default_rng(4).choice(N, 40, replace=False)]))
    run_case(q, k, v, w.causal, w.softmax_scale, 2688.0, rows=rows, label="video_dit")


@pytest.mark.parametrize("n,d,causal,nk", [
    (200, 64, True, None), (333, 128, False, None), (77, 64, True, None), (130, 128, True, None),
    (100, 128, False, 260), (300, 64, False, 40), (17, 64, False, None), (16, 128, True, None),
    (1, 64, True, None), (1, 128, False, 5),
    # few queries against long keys: the first pass takes the 32-query tiles
    (16, 128, False, 5000), (24, 64, False, 3000),
])
def test_ragged_and_degenerate_shapes(n, d, causal, nk):
    q, k, v = _synthetic(n, d, seed=n * 5 + d, nk=nk, heads=2)
    for p_scale in (1.0, 2688.0):
        run_case(q, k, v, causal, 1.0 / math.sqrt(d), p_scale, label=f"ragged n={n} nk={nk}")


def test_causal_row_zero_closed_form():
    """Query 0 sees key 0 alone: P = 1 -> P^F = 1.03125, so O[0] = 1.03125 v^_0."""
    q, k, v = _synthetic(40, 128, seed=21)
    p = B.problem_for(q.to(DEV), k.to(DEV), True, 0.1)
    o = gpu_fwd_quantized(q.to(DEV), k.to(DEV), v.to(DEV), True, 0.1).cpu()
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o_hp = torch.empty_like(q, device=DEV)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd(p, q.to(DEV), k.to(DEV), v.to(DEV), o_hp, lse, ws)
    torch.cuda.synchronize()
    vh0 = o_hp[0, 0, 0].cpu().double()  # O_hp[0] = v^_0 exactly
    assert torch.equal(o[0, 0, 0], (1.03125 * vh0).to(torch.bfloat16))


def test_output_stays_in_bounds_and_rejects_null():
    n, d, H = 200, 64, 2
    q, k, v = (t.to(DEV) for t in _synthetic(n, d, seed=9, heads=H))
    p = B.problem_for(q, k, True, 0.125)
    numel = H * n * d
    guard = 4096
    buf = torch.full((numel + guard,), -12345.0, dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(B.attnqat_fwd_workspace_bytes(p), dtype=torch.uint8, device=DEV)
    o_hp = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    B.attnqat_fwd_quantized(p, q, k, v, o_hp, lse, buf[:numel].view(1, H, n, d), ws)
    torch.cuda.synchronize()
    assert torch.all(buf[numel:] == -12345.0)
    assert torch.all(torch.isfinite(buf[:numel].float()))
    rc = B._lib.attnqat_fwd_quantized(B.ctypes.byref(p), q.data_ptr(), k.data_ptr(),
                                      v.data_ptr(), o_hp.data_ptr(), lse.data_ptr(), None,
                                      ws.data_ptr(), ws.numel(), None)
    assert rc == B.ERR_INVALID_ARGUMENT
