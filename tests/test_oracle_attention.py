"""Pins for the oracle's QAT attention forward and backward (CPU only).

The oracle is checked against: torch's fp64 scaled-dot-product attention and
autograd (a library routine) on the fake-quantized inputs, central finite
differences, the FlashAttention row-sum identity that the high-precision
auxiliary output keeps exact, and closed forms (causal row 0, uniform P).
The quantized forward output O = P^F V^ is pinned by the same closed forms,
by the adjoint identity <O, dO> = <V^, dV> with the backward's dV, and by
reducing to O_hp without P quantization.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle.attention import (qat_backward, qat_backward_full_head, qat_backward_head,
                              qat_ds_head, qat_forward, qat_forward_head,
                              qat_forward_quantized_head, quantize_qkv)
from oracle.nvfp4 import fake_nvfp4_values
from workloads import make_inputs


def _heads_np(n=64, d=64, seed=0, nk=None):
    g = torch.Generator().manual_seed(seed)
    nk = n if nk is None else nk
    q = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    k = torch.randn(nk, d, generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn(nk, d, generator=g).to(torch.bfloat16).double().numpy()
    do = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    return q, k, v, do


def _sdpa(qh, kh, vh, scale, causal):
    t = lambda a: torch.from_numpy(a)[None, None]
    return torch.nn.functional.scaled_dot_product_attention(
        t(qh), t(kh), t(vh), is_causal=causal, scale=scale)[0, 0].numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(64, 64), (80, 128), (37, 64)])
def test_forward_matches_sdpa_on_quantized_inputs(causal, n, d):
    q, k, v, _ = _heads_np(n, d, seed=n + d)
    s = 1.0 / math.sqrt(d)
    o, lse = qat_forward_head(q, k, v, s, causal)
    qh, kh, vh = quantize_qkv(q, k, v)
    ref = _sdpa(qh, kh, vh, s, causal)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    S = s * (torch.from_numpy(qh) @ torch.from_numpy(kh).T)
    if causal:
        S = S.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), rtol=1e-13, atol=1e-13)


def test_forward_unquantized_is_plain_attention():
    q, k, v, _ = _heads_np(48, 64, seed=3)
    o, _ = qat_forward_head(q, k, v, 0.125, False, quantize=False)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 0.125, False), rtol=1e-12, atol=1e-12)


def test_cross_attention_forward():
    q, k, v, _ = _heads_np(40, 64, seed=4, nk=72)
    o, _ = qat_forward_head(q, k, v, 0.125, False)
    qh, kh, vh = quantize_qkv(q, k, v)
    np.testing.assert_allclose(o, _sdpa(qh, kh, vh, 0.125, False), rtol=1e-12, atol=1e-12)


def _autograd_grads(qh, kh, vh, do, scale, causal):
    tq, tk, tv = (torch.from_numpy(a).clone().requires_grad_(True) for a in (qh, kh, vh))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None], is_causal=causal, scale=scale)[0, 0]
    (o * torch.from_numpy(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(64, 64), (50, 128)])
def test_backward_ste_matches_autograd(causal, n, d):
    """dQ, dK (straight-through) and dV with P-quantization off equal fp64
    autograd of <SDPA(Q^, K^, V^), dO> when O_hp is the exact forward output."""
    q, k, v, do = _heads_np(n, d, seed=7 * n + d)
    s = 1.0 / math.sqrt(d)
    o, lse = qat_forward_head(q, k, v, s, causal)
    qh, kh, vh = quantize_qkv(q, k, v)
    gq, gk, gv = _autograd_grads(qh, kh, vh, do, s, causal)
    dq, dk, dv = qat_backward_head(q, k, v, o, do, lse, s, causal, quantize_p=False)
    np.testing.assert_allclose(dq, gq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, gk, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, gv, rtol=1e-10, atol=1e-11)
    # with P quantization on, dQ and dK do not change (STE), dV does
    dq2, dk2, dv2 = qat_backward_head(q, k, v, o, do, lse, s, causal)
    assert np.array_equal(dq, dq2) and np.array_equal(dk, dk2)
    assert not np.allclose(dv, dv2)


def test_backward_finite_differences():
    """Central differences of <attn(Q^,K^,V^), dO> in Q^ and K^ on a tiny head."""
    n, d = 12, 32
    q, k, v, do = _heads_np(n, d, seed=99)
    s = 0.3
    qh, kh, vh = quantize_qkv(q, k, v)
    o, lse = qat_forward_head(q, k, v, s, False)
    dq, dk, _ = qat_backward_head(q, k, v, o, do, lse, s, False)

    def f(qq, kk):
        out, _ = qat_forward_head(qq, kk, vh, s, False, quantize=False)
        return float((out * do).sum())

    h = 1e-6
    rng = np.random.default_rng(0)
    for _ in range(40):
        i, j = rng.integers(n), rng.integers(d)
        e = np.zeros_like(qh)
        e[i, j] = h
        fd_q = (f(qh + e, kh) - f(qh - e, kh)) / (2 * h)
        fd_k = (f(qh, kh + e) - f(qh, kh - e)) / (2 * h)
        assert abs(fd_q - dq[i, j]) <= 1e-6 * max(1.0, abs(dq[i, j]))
        assert abs(fd_k - dk[i, j]) <= 1e-6 * max(1.0, abs(dk[i, j]))


def test_rowsum_identity_holds_with_o_hp_and_breaks_with_quantized_o():
    """rowsum(P * (dO V^T)) = rowsum(O_hp * dO) exactly for O_hp = P V^; it
    fails when the output is formed with the quantized P^F instead."""
    q, k, v, do = _heads_np(128, 64, seed=5)
    s = 0.125
    qh, kh, vh = quantize_qkv(q, k, v)
    o, lse = qat_forward_head(q, k, v, s, False)
    P = np.exp(s * qh @ kh.T - lse[:, None])
    lhs = (P * (do @ vh.T)).sum(1)
    rhs = (o * do).sum(1)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    PF = fake_nvfp4_values(P, axis=1)
    o_q = PF @ vh
    bad = (o_q * do).sum(1)
    assert np.max(np.abs(lhs - bad)) > 1e-3 * np.max(np.abs(rhs))


def test_ds_rows_and_dk_sum_to_zero():
    q, k, v, do = _heads_np(48, 64, seed=6)  # 48 keys <= 64 dims: K^ has full column rank
    s = 0.125
    o, lse = qat_forward_head(q, k, v, s, True)
    qh, kh, vh = quantize_qkv(q, k, v)
    dq, dk, dv = qat_backward_head(q, k, v, o, do, lse, s, True)
    assert np.max(np.abs(dk.sum(0))) <= 1e-11 * np.abs(dk).max()
    # recover dS from dQ = s dS K^ and check its rows sum to zero
    dS = np.linalg.lstsq(kh.T, (dq / s).T, rcond=None)[0].T
    assert np.max(np.abs(dS.sum(1))) <= 1e-9


@pytest.mark.parametrize("causal,n,nk", [(False, 40, 72), (True, 56, 56)])
def test_ds_intermediate(causal, n, nk):
    """dS reproduces dQ = s dS K^ and dK = s dS^T Q^ (both pinned against
    autograd above), its rows sum to zero (softmax Jacobian, O_hp exact) and
    causal entries above the diagonal are exactly zero."""
    q, k, v, do = _heads_np(n, 64, seed=n + nk, nk=nk)
    s = 0.11
    o, lse = qat_forward_head(q, k, v, s, causal)
    qh, kh, _ = quantize_qkv(q, k, v)
    dS = qat_ds_head(q, k, v, o, do, lse, s, causal)
    dq, dk, _ = qat_backward_head(q, k, v, o, do, lse, s, causal)
    assert dS.shape == (n, nk)
    assert np.max(np.abs(s * dS @ kh - dq)) <= 1e-12 * np.abs(dq).max()
    assert np.max(np.abs(s * dS.T @ qh - dk)) <= 1e-12 * np.abs(dk).max()
    assert np.max(np.abs(dS.sum(1))) <= 1e-12 * np.abs(dS).max() * nk
    if causal:
        assert np.all(dS[np.triu_indices(n, 1)] == 0.0)


def test_causal_row_zero_closed_form():
    q, k, v, do = _heads_np(32, 64, seed=8)
    s = 0.125
    qh, kh, vh = quantize_qkv(q, k, v)
    o, lse = qat_forward_head(q, k, v, s, True)
    assert np.array_equal(o[0], vh[0])
    assert lse[0] == pytest.approx(s * float(qh[0] @ kh[0]), rel=0, abs=1e-14)
    dq, dk, dv = qat_backward_head(q, k, v, o, do, lse, s, True)
    assert np.max(np.abs(dq[0])) <= 1e-14
    # a single-token causal head: P = [[1]]; fq(1) has scale 0.171875 (0x23)
    # and code 6, so P^F = 1.03125 and dV = 1.03125 dO; with p_scale = 2688
    # (= 448 * 6) the lone 1.0 quantizes to exactly 1.
    q1, k1, v1, do1 = q[:1], k[:1], v[:1], do[:1]
    o1, lse1 = qat_forward_head(q1, k1, v1, s, True)
    _, _, dv1 = qat_backward_head(q1, k1, v1, o1, do1, lse1, s, True)
    assert np.array_equal(dv1[0], 1.03125 * do1[0])
    _, _, dv2 = qat_backward_head(q1, k1, v1, o1, do1, lse1, s, True, p_scale=2688.0)
    assert np.array_equal(dv2[0], do1[0])


@pytest.mark.parametrize("n,expect_pf,p_scale", [(128, 2.0 ** -7, 1.0),
                                                 (4096, 0.0, 1.0),
                                                 (4096, 2.0 ** -12, 2688.0)])
def test_uniform_p_closed_form(n, expect_pf, p_scale):
    """Q = 0 gives P = 1/N.  N=128: amax/6 rounds to the subnormal scale 2^-9
    and P^F = 4*2^-9 = 2^-7 exactly; N=4096: the scale underflows to 0 and
    dV = 0; with p_scale = 2688, 2688/4096 = 0.65625 -> scale 0.109375,
    code 6 -> P^F = 2^-12 exactly."""
    d = 64
    g = torch.Generator().manual_seed(n)
    q = np.zeros((n, d))
    k = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    do = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    o, lse = qat_forward_head(q, k, v, 0.125, False)
    _, kh, vh = quantize_qkv(q, k, v)
    np.testing.assert_allclose(o, np.broadcast_to(vh.mean(0), o.shape), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, math.log(n))
    _, _, dv = qat_backward_head(q, k, v, o, do, lse, 0.125, False, p_scale=p_scale,
                                 key_groups=[0, 3])
    np.testing.assert_allclose(dv, np.broadcast_to(expect_pf * do.sum(0), dv.shape),
                               rtol=1e-12, atol=1e-12)


def test_subset_and_full_paths_agree():
    q, k, v, do = _heads_np(72, 64, seed=9)  # 72 keys: last group has 8
    for causal in (False, True):
        o, lse = qat_forward_head(q, k, v, 0.125, causal)
        a = qat_backward_full_head(q, k, v, o, do, lse, 0.125, causal)
        b = qat_backward_head(q, k, v, o, do, lse, 0.125, causal)
        for x, y in zip(a, b):
            np.testing.assert_allclose(x, y, rtol=1e-12, atol=1e-13)
        rows = [0, 5, 71]
        c = qat_backward_head(q, k, v, o, do, lse, 0.125, causal, rows=rows, key_groups=[4, 1])
        np.testing.assert_allclose(c[0], a[0][rows], rtol=1e-12, atol=1e-13)
        keys = list(range(64, 72)) + list(range(16, 32))
        np.testing.assert_allclose(c[1], a[1][keys], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(c[2], a[2][keys], rtol=1e-12, atol=1e-13)
        o2, lse2 = qat_forward_head(q, k, v, 0.125, causal, rows=rows)
        np.testing.assert_allclose(o2, o[rows], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse2, lse[rows], rtol=1e-13, atol=1e-14)


def test_p_quant_groups_along_keys_with_zero_padded_tail():
    """dV uses fq(P) grouped along keys from key 0; the 8-key tail group is
    zero-padded, i.e. it quantizes exactly as if 8 zero-probability keys
    followed."""
    q, k, v, do = _heads_np(40, 64, seed=10, nk=40)
    o, lse = qat_forward_head(q, k, v, 0.125, False)
    _, _, dv = qat_backward_head(q, k, v, o, do, lse, 0.125, False)
    qh, kh, vh = quantize_qkv(q, k, v)
    P = np.exp(0.125 * qh @ kh.T - lse[:, None])
    Ppad = np.concatenate([P, np.zeros((40, 8))], axis=1)
    PF = np.concatenate([fake_nvfp4_values(Ppad[:, 16 * g:16 * g + 16], axis=1)
                         for g in range(3)], axis=1)[:, :40]
    np.testing.assert_allclose(dv, PF.T @ do, rtol=1e-13, atol=1e-13)


def test_batched_wrappers_on_tiny_workload():
    q, k, v, do = make_inputs("tiny")
    fw = qat_forward(q, k, v, 0.125, False)
    o = np.stack([fw[(0, 0)][0]])[None]
    lse = np.stack([fw[(0, 0)][1]])[None]
    bw = qat_backward(q, k, v, o, do, lse, 0.125, False)
    dq, dk, dv = bw[(0, 0)]
    assert dq.shape == (128, 64) and dk.shape == (128, 64) and dv.shape == (128, 64)
    assert np.all(np.isfinite(dq)) and np.abs(dv).max() > 0


# --- the quantized forward output O = P^F V^ --------------------------------

def test_quantized_output_without_p_quant_is_o_hp():
    q, k, v, _ = _heads_np(56, 64, seed=11)
    for causal in (False, True):
        o_hp, _ = qat_forward_head(q, k, v, 0.125, causal)
        o = qat_forward_quantized_head(q, k, v, 0.125, causal, quantize_p=False)
        np.testing.assert_allclose(o, o_hp, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("p_scale", [1.0, 2688.0])
@pytest.mark.parametrize("causal", [False, True])
def test_quantized_output_is_adjoint_of_backward_dv(causal, p_scale):
    """<O, dO> = <V^, dV>: the forward's P^F is the one whose transpose the
    backward multiplies into dO (dV is the straight-through gradient of O)."""
    q, k, v, do = _heads_np(72, 64, seed=12)  # 72 keys: a short last group
    o_hp, lse = qat_forward_head(q, k, v, 0.125, causal)
    o = qat_forward_quantized_head(q, k, v, 0.125, causal, p_scale=p_scale)
    _, _, dv = qat_backward_full_head(q, k, v, o_hp, do, lse, 0.125, causal, p_scale=p_scale)
    _, _, vh = quantize_qkv(q, k, v)
    lhs, rhs = float((o * do).sum()), float((vh * dv).sum())
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs))
    # and it differs from O_hp (the quantization is not a no-op here)
    assert np.max(np.abs(o - o_hp)) > 1e-3 * np.max(np.abs(o_hp))


@pytest.mark.parametrize("n,p_scale,expect", [(128, 1.0, "mean"), (4096, 1.0, "zero"),
                                              (4096, 2688.0, "mean")])
def test_quantized_output_uniform_p_closed_form(n, p_scale, expect):
    """Q = 0 gives P = 1/N.  N=128: P^F = 2^-7 = P, so O = mean(V^); N=4096:
    the scale underflows and O = 0; with p_scale = 2688, P^F = 2^-12 = P
    again and O = mean(V^)."""
    d = 64
    g = torch.Generator().manual_seed(n + 1)
    q = np.zeros((n, d))
    k = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    v = torch.randn(n, d, generator=g).to(torch.bfloat16).double().numpy()
    rows = [0, 7, n - 1]
    o = qat_forward_quantized_head(q, k, v, 0.125, False, p_scale=p_scale, rows=rows)
    _, _, vh = quantize_qkv(q, k, v)
    want = np.zeros((3, d)) if expect == "zero" else np.broadcast_to(vh.mean(0), (3, d))
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-14)


def test_quantized_output_causal_row_zero_closed_form():
    """Causal query 0 sees only key 0 with P = 1: fq(1) = 1.03125 (scale
    0.171875, code 6), so O[0] = 1.03125 v^_0; with p_scale = 2688 it is v^_0."""
    q, k, v, _ = _heads_np(32, 64, seed=13)
    _, _, vh = quantize_qkv(q, k, v)
    o = qat_forward_quantized_head(q, k, v, 0.125, True, rows=[0])
    assert np.array_equal(o[0], 1.03125 * vh[0])
    o2 = qat_forward_quantized_head(q, k, v, 0.125, True, p_scale=2688.0, rows=[0])
    assert np.array_equal(o2[0], vh[0])


def test_quantized_output_groups_along_keys_with_zero_padded_tail():
    q, k, v, _ = _heads_np(40, 64, seed=14, nk=40)
    o_hp, lse = qat_forward_head(q, k, v, 0.125, False)
    o = qat_forward_quantized_head(q, k, v, 0.125, False)
    qh, kh, vh = quantize_qkv(q, k, v)
    P = np.exp(0.125 * qh @ kh.T - lse[:, None])
    Ppad = np.concatenate([P, np.zeros((40, 8))], axis=1)
    PF = np.concatenate([fake_nvfp4_values(Ppad[:, 16 * g:16 * g + 16], axis=1)
                         for g in range(3)], axis=1)[:, :40]
    np.testing.assert_allclose(o, PF @ vh, rtol=1e-13, atol=1e-13)
    # rows subset = full rows
    o_rows = qat_forward_quantized_head(q, k, v, 0.125, False, rows=[3, 39])
    np.testing.assert_allclose(o_rows, o[[3, 39]], rtol=1e-13, atol=1e-14)
