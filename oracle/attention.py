"""Naive fp64 NVFP4 fake-quantized attention: the QAT forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What it follows
---------------
"NVFP4 Attention QAT Backward" (cuDNN frontend docs), §Overview (the formula
block) and §High-level wrapper:

* ``Q^, K^, V^ = fake_nvfp4(Q), fake_nvfp4(K), fake_nvfp4(V)``, groups of 16
  along the head dimension;
* ``P = softmax(s * Q^ K^T)`` (unquantized), ``O_hp = P V^`` (the
  high-precision auxiliary saved before any probability quantization) and
  ``lse`` = the natural-log log-sum-exp of each row of ``s * Q^ K^T``;
* the quantized user-visible output ``O = fake_nvfp4(P)  V^`` (Attn-QAT
  summary, §Method; see :func:`qat_forward_quantized_head` for the reading);
* backward: ``dS = P * (dO V^T - rowsum(O_hp * dO))``, ``dQ = s dS K^``,
  ``dK = s dS^T Q^`` (straight-through: the unquantized P), and
  ``dV = fake_nvfp4(P)^T dO`` with P grouped in 16s along the key index.

The Attn-QAT summary page (§Key claims, fixes 1 and 2; §Method) gives the
reason for ``O_hp`` (it keeps the FlashAttention identity
``rowsum(P * dP) = rowsum(O_hp * dO)`` exact) and for re-quantizing the
recomputed P in the backward.

Readings (listed in the design notes): causal masking is ``key j <= query i``
(self-attention only, ``Nq == Nkv``); masked and out-of-range keys have
``P = 0``; P groups start at key 0 and a short last group is zero-padded;
``delta`` uses the supplied ``O_hp``; ``p_scale`` (default 1, the literal
formula) is an optional pre-scale so that ``P^F = fake_nvfp4(p_scale P) /
p_scale``.

All arithmetic is fp64 on the exact bf16 input values; the only library
primitives are NumPy matmul, exp, log and max.
"""
from __future__ import annotations

import numpy as np

from .nvfp4 import GROUP, fake_nvfp4_values


def _as64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch tensor
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _causal_mask(rows: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """True where key j is masked for query i (j > i)."""
    return keys[None, :] > rows[:, None]


def quantize_qkv(q, k, v):
    """The fake-quantized Q^, K^, V^ of one head (groups along the head dim)."""
    return fake_nvfp4_values(q, -1), fake_nvfp4_values(k, -1), fake_nvfp4_values(v, -1)


def qat_forward_head(q, k, v, softmax_scale: float, causal: bool, rows=None,
                     quantize: bool = True):
    """QAT forward of one head.  ``q``: (Nq, D); ``k``, ``v``: (Nk, D).

    Returns ``(o_hp, lse)`` for the query rows ``rows`` (all rows if None):
    ``o_hp`` (len(rows), D) and ``lse`` (len(rows),), both fp64.
    ``quantize=False`` skips the fake quantization (a plain attention, used
    to pin this function to a library routine).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    if causal and q.shape[0] != k.shape[0]:
        raise ValueError("causal attention is self-attention only (Nq == Nk)")
    qh, kh, vh = quantize_qkv(q, k, v) if quantize else (q, k, v)
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(k.shape[0])
    S = softmax_scale * (qh[r] @ kh.T)
    if causal:
        S = np.where(_causal_mask(r, keys), -np.inf, S)
    m = S.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(S - m).sum(axis=1))
    P = np.exp(S - lse[:, None])
    return P @ vh, lse


def qat_forward_quantized_head(q, k, v, softmax_scale: float, causal: bool,
                               p_scale: float = 1.0, rows=None, quantize_p: bool = True):
    """The quantized, user-visible QAT forward output of one head.

    The Attn-QAT summary (§Method) forms the low-precision output from the
    FP32 softmax probabilities fake-quantized to ``P^F`` and ``V^F``:
    ``O = P^F V^``.  Reading taken here: ``P`` is the *normalized* softmax,
    ``P = exp(s Q^ K^T - lse)`` with the row's natural-log lse, and ``P^F =
    fake_nvfp4(p_scale P) / p_scale`` grouped in 16s along the key index from
    key 0 -- exactly the ``P^F`` whose transpose the backward multiplies into
    dO for dV, so dV is the straight-through gradient of this O.  (A one-pass
    forward would instead quantize the unnormalized running-max ``p`` tile by
    tile; that is not what is computed here.)

    Returns ``O`` (len(rows), D) in fp64 for the query rows ``rows`` (all if
    None).  ``quantize_p=False`` skips the quantization of P (then ``O`` is
    ``O_hp``).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    if causal and q.shape[0] != k.shape[0]:
        raise ValueError("causal attention is self-attention only (Nq == Nk)")
    r = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    _, lse = qat_forward_head(q, k, v, softmax_scale, causal, rows=r)
    qh, kh, vh = quantize_qkv(q, k, v)
    keys = np.arange(k.shape[0])
    S = softmax_scale * (qh[r] @ kh.T)
    P = np.exp(S - lse[:, None])
    if causal:
        P = np.where(_causal_mask(r, keys), 0.0, P)
    PF = fake_nvfp4_values(p_scale * P, axis=1) / p_scale if quantize_p else P
    return PF @ vh


def _probabilities(qh, kh, lse, softmax_scale, causal, rows, keys):
    """P[rows, keys] recomputed from lse; masked entries are 0."""
    S = softmax_scale * (qh[rows] @ kh[keys].T)
    P = np.exp(S - lse[rows][:, None])
    if causal:
        P = np.where(_causal_mask(rows, keys), 0.0, P)
    return P


def qat_backward_head(q, k, v, o_hp, do, lse, softmax_scale: float, causal: bool,
                      p_scale: float = 1.0, rows=None, key_groups=None,
                      quantize: bool = True, quantize_p: bool = True):
    """QAT backward of one head.

    Inputs: ``q`` (Nq, D), ``k``/``v`` (Nk, D), ``o_hp``/``do`` (Nq, D),
    ``lse`` (Nq,).  Returns ``(dq, dk, dv)`` in fp64, where ``dq`` covers the
    query rows ``rows`` (all if None) and ``dk``/``dv`` cover the keys of the
    16-key groups ``key_groups`` (all keys if None), in that order.
    ``quantize``/``quantize_p`` switch the fake quantization of Q/K/V and of
    P off (used only to pin this function against autograd).
    """
    q, k, v, o_hp, do, lse = map(_as64, (q, k, v, o_hp, do, lse))
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is self-attention only (Nq == Nk)")
    qh, kh, vh = quantize_qkv(q, k, v) if quantize else (q, k, v)
    delta = (o_hp * do).sum(axis=1)  # rowsum(O_hp * dO), from the supplied O_hp
    all_rows = np.arange(Nq)
    all_keys = np.arange(Nk)

    def dS_of(rows_, keys_):
        P = _probabilities(qh, kh, lse, softmax_scale, causal, rows_, keys_)
        dP = do[rows_] @ vh[keys_].T
        return P, P * (dP - delta[rows_][:, None])

    # dQ over the requested rows, all keys.
    r = all_rows if rows is None else np.asarray(rows, dtype=np.int64)
    _, dS_r = dS_of(r, all_keys)
    dq = softmax_scale * (dS_r @ kh)

    # dK and dV over the requested key groups, all rows.
    groups = range(-(-Nk // GROUP)) if key_groups is None else key_groups
    dk_parts, dv_parts = [], []
    for g in groups:
        keys_g = np.arange(GROUP * g, min(GROUP * (g + 1), Nk))
        P, dS = dS_of(all_rows, keys_g)
        dk_parts.append(softmax_scale * (dS.T @ qh))
        if quantize_p:
            PF = fake_nvfp4_values(p_scale * P, axis=1) / p_scale  # one group of keys
        else:
            PF = P
        dv_parts.append(PF.T @ do)
    D = q.shape[1]
    dk = np.concatenate(dk_parts, axis=0) if dk_parts else np.zeros((0, D))
    dv = np.concatenate(dv_parts, axis=0) if dv_parts else np.zeros((0, D))
    return dq, dk, dv


def qat_backward_full_head(q, k, v, o_hp, do, lse, softmax_scale: float, causal: bool,
                           p_scale: float = 1.0):
    """Same result as :func:`qat_backward_head` over every row and key, computed
    with whole-matrix products (faster for full-size checks)."""
    q, k, v, o_hp, do, lse = map(_as64, (q, k, v, o_hp, do, lse))
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is self-attention only (Nq == Nk)")
    qh, kh, vh = quantize_qkv(q, k, v)
    delta = (o_hp * do).sum(axis=1)
    P = _probabilities(qh, kh, lse, softmax_scale, causal, np.arange(Nq), np.arange(Nk))
    dS = P * (do @ vh.T - delta[:, None])
    dq = softmax_scale * (dS @ kh)
    dk = softmax_scale * (dS.T @ qh)
    PF = fake_nvfp4_values(p_scale * P, axis=1) / p_scale
    dv = PF.T @ do
    return dq, dk, dv


def qat_ds_head(q, k, v, o_hp, do, lse, softmax_scale: float, causal: bool):
    """The backward's dS = P * (dO V^T - rowsum(O_hp * dO)) of one head,
    (Nq, Nk) in fp64 (page "NVFP4 Attention QAT Backward", §Overview formula
    block), with P recomputed from lse from the fake-quantized Q^ and K^ and
    masked entries 0.  dQ = s dS K^ and dK = s dS^T Q^ of
    :func:`qat_backward_head` are products with it."""
    q, k, v, o_hp, do, lse = map(_as64, (q, k, v, o_hp, do, lse))
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is self-attention only (Nq == Nk)")
    qh, kh, vh = quantize_qkv(q, k, v)
    delta = (o_hp * do).sum(axis=1)
    P = _probabilities(qh, kh, lse, softmax_scale, causal, np.arange(Nq), np.arange(Nk))
    return P * (do @ vh.T - delta[:, None])


def _heads(B, H, heads):
    return [(b, h) for b in range(B) for h in range(H)] if heads is None else list(heads)


def qat_forward(q, k, v, softmax_scale: float, causal: bool, heads=None, rows=None):
    """Batched QAT forward over (B, H, N, D) inputs.

    Returns ``{(b, h): (o_hp, lse)}`` for the heads ``heads`` (all if None).
    """
    B, H = q.shape[0], q.shape[1]
    out = {}
    for b, h in _heads(B, H, heads):
        out[(b, h)] = qat_forward_head(q[b, h], k[b, h], v[b, h], softmax_scale, causal, rows)
    return out


def qat_forward_quantized(q, k, v, softmax_scale: float, causal: bool, p_scale: float = 1.0,
                          heads=None, rows=None):
    """Batched quantized forward output; returns ``{(b, h): O}``."""
    B, H = q.shape[0], q.shape[1]
    return {(b, h): qat_forward_quantized_head(q[b, h], k[b, h], v[b, h], softmax_scale,
                                               causal, p_scale, rows)
            for b, h in _heads(B, H, heads)}


def qat_backward(q, k, v, o_hp, do, lse, softmax_scale: float, causal: bool,
                 p_scale: float = 1.0, heads=None, rows=None, key_groups=None):
    """Batched QAT backward; returns ``{(b, h): (dq, dk, dv)}``."""
    B, H = q.shape[0], q.shape[1]
    out = {}
    for b, h in _heads(B, H, heads):
        if rows is None and key_groups is None:
            out[(b, h)] = qat_backward_full_head(q[b, h], k[b, h], v[b, h], o_hp[b, h],
                                                 do[b, h], lse[b, h], softmax_scale,
                                                 causal, p_scale)
        else:
            out[(b, h)] = qat_backward_head(q[b, h], k[b, h], v[b, h], o_hp[b, h], do[b, h],
                                            lse[b, h], softmax_scale, causal, p_scale,
                                            rows, key_groups)
    return out
