"""Thin ctypes binding of libattnqat.so (include/attnqat.h and the
measurement entry points of include/attnqat_instrument.h).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory (``data_ptr()``) and streams.  The functions
keep the C names; ``nvfp4_attention_qat_backward`` additionally mirrors the
high-level wrapper of "NVFP4 Attention QAT Backward" (§High-level wrapper:
it returns ``dq_tensor``/``dk_tensor``/``dv_tensor``, accepts preallocated
outputs and an explicit stream).

The C ABI takes plain pointers and cannot check buffer sizes, so every
function here checks each tensor's dtype, shape, contiguity and device
against the problem before the call and raises ValueError on a mismatch.

If the library is missing this module raises on import: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnqat.so")

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_MISALIGNED = -3
ERR_WORKSPACE_TOO_SMALL = -4
ERR_HIP = -5
DTYPE_BF16 = 0
DTYPE_F32 = 1
WS_FWD = 0
WS_BWD = 1


class attnqat_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("seqlen_q", ctypes.c_int32), ("seqlen_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("p_scale", ctypes.c_float)]


class attnqat_ws_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("total_bytes", "q_hat", "k_hat", "v_hat", "q_scale", "k_scale", "v_scale",
                 "delta")]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python nvfp4_fake_quantized_amd/csrc/build.py` (no fallback exists)")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.POINTER(attnqat_problem)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_SIGS = {
    "attnqat_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attnqat_version": (ctypes.c_int, []),
    "attnqat_check_support": (ctypes.c_int, [_P]),
    "attnqat_check_device": (ctypes.c_int, [ctypes.c_int]),
    "attnqat_fwd_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(_sz)]),
    "attnqat_bwd_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(_sz)]),
    "attnqat_workspace_layout": (ctypes.c_int, [_P, ctypes.c_int,
                                                ctypes.POINTER(attnqat_ws_layout)]),
    "attnqat_fake_nvfp4": (ctypes.c_int, [_vp, ctypes.c_int, _vp, _vp, ctypes.c_int64,
                                          ctypes.c_int64, _vp]),
    "attnqat_fwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "attnqat_bwd": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                   _vp]),
    "attnqat_fwd_quantized": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "attnqat_nvfp4_pack": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp]),
    "attnqat_fwd_packed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp]),
    "attnqat_fwd_timed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp, _vp]),
    "attnqat_fwd_quantized_timed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                                   _vp, _vp]),
    "attnqat_bwd_timed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                         _sz, _vp, _vp]),
    "attnqat_probe_mfma_peak": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, ctypes.c_int, _vp]),
    "attnqat_probe_issue_mix": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp]),
    "attnqat_probe_lds_write": (ctypes.c_int, [ctypes.c_int, _vp, ctypes.c_int, ctypes.c_int,
                                               _vp]),
    "attnqat_bwd_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


class AttnQatError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def status_string(status: int) -> str:
    return _lib.attnqat_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise AttnQatError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


# The page's default softmax scale (§Tensor contract: it must match the
# forward's), used only by the high-level wrappers when none is given.
PAGE_DEFAULT_SOFTMAX_SCALE = 1.0 / math.sqrt(128.0)


def make_problem(batch, heads, seqlen_q, seqlen_kv, head_dim, causal, softmax_scale,
                 p_scale=1.0) -> attnqat_problem:
    """The C problem struct; ``softmax_scale`` is required (the library has
    no default)."""
    if softmax_scale is None:
        raise ValueError("softmax_scale is required (it must match the forward's)")
    return attnqat_problem(batch, heads, seqlen_q, seqlen_kv, head_dim, int(bool(causal)),
                           float(softmax_scale), float(p_scale))


def problem_for(q, k, causal, softmax_scale, p_scale=1.0) -> attnqat_problem:
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be (B, H, S, D) tensors")
    B, H, Nq, D = q.shape
    return make_problem(B, H, Nq, k.shape[2], D, causal, softmax_scale, p_scale)


# ---- argument checks (the C ABI takes raw pointers) --------------------------

def _expect(t, name, dtype, shape=None, numel=None, device=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _device_of(t):
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU (HIP) device")
    return t.device


def _check_attention(p: attnqat_problem, q, k=None, v=None, o_hp=None, d_o=None, lse=None,
                     dq=None, dk=None, dv=None, o=None, workspace=None):
    """Every tensor of an attention call against the problem."""
    qs = (p.batch, p.heads, p.seqlen_q, p.head_dim)
    ks = (p.batch, p.heads, p.seqlen_kv, p.head_dim)
    bf = torch.bfloat16
    _expect(q, "q", bf, qs)
    dev = _device_of(q)
    for t, n, shp in ((k, "k", ks), (v, "v", ks), (o_hp, "o_hp", qs), (d_o, "d_o", qs),
                      (dq, "dq", qs), (dk, "dk", ks), (dv, "dv", ks), (o, "o", qs)):
        if t is not None:
            _expect(t, n, bf, shp, device=dev)
    if lse is not None:
        _expect(lse, "lse", torch.float32, qs[:3], device=dev)
    if workspace is not None:
        _expect(workspace, "workspace", torch.uint8, device=dev)


# ---- C-ABI functions (same names) --------------------------------------------

def attnqat_version() -> int:
    return _lib.attnqat_version()


def attnqat_check_support(p: attnqat_problem) -> int:
    return _lib.attnqat_check_support(ctypes.byref(p))


def attnqat_check_device(device: int = 0) -> int:
    return _lib.attnqat_check_device(device)


def attnqat_fwd_workspace_bytes(p: attnqat_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.attnqat_fwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)),
           "attnqat_fwd_workspace_bytes")
    return n.value


def attnqat_bwd_workspace_bytes(p: attnqat_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.attnqat_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)),
           "attnqat_bwd_workspace_bytes")
    return n.value


def attnqat_workspace_layout(p: attnqat_problem, which: int) -> dict:
    out = attnqat_ws_layout()
    _check(_lib.attnqat_workspace_layout(ctypes.byref(p), which, ctypes.byref(out)),
           "attnqat_workspace_layout")
    return {name: getattr(out, name) for name, _ in attnqat_ws_layout._fields_}


def attnqat_fake_nvfp4(x, x_hat=None, scales=None, stream=None):
    """fake_nvfp4 of a contiguous bf16/fp32 CUDA tensor in groups of 16 along
    its last dim.  Returns ``(x_hat, scales)`` (scales: uint8 E4M3FN bytes)."""
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("x must be bf16 or fp32")
    dtype = DTYPE_BF16 if x.dtype == torch.bfloat16 else DTYPE_F32
    L = x.shape[-1] if x.dim() > 0 else 1
    rows = x.numel() // L if L else 0
    if x_hat is None:
        x_hat = torch.empty_like(x)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (max(L // 16, 0),), dtype=torch.uint8,
                             device=x.device)
    _expect(x, "x", x.dtype)
    _expect(x_hat, "x_hat", x.dtype, numel=x.numel(), device=x.device)
    _expect(scales, "scales", torch.uint8, numel=rows * (L // 16), device=x.device)
    _device_of(x)
    _check(_lib.attnqat_fake_nvfp4(_ptr(x), dtype, _ptr(x_hat), _ptr(scales), rows, L,
                                   _stream(stream)), "attnqat_fake_nvfp4")
    return x_hat, scales


def attnqat_fwd(p: attnqat_problem, q, k, v, o_hp, lse, workspace, stream=None):
    _check_attention(p, q, k, v, o_hp=o_hp, lse=lse, workspace=workspace)
    _check(_lib.attnqat_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp), _ptr(lse),
                            _ptr(workspace), workspace.numel(), _stream(stream)), "attnqat_fwd")


def attnqat_nvfp4_pack(x, codes=None, scales=None, stream=None):
    """Packed NVFP4 storage of a bf16 tensor along its last dim: returns
    ``(codes, scales)`` (uint8, last dim L/2 and L/16)."""
    if x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("expected a contiguous bf16 tensor")
    L = x.shape[-1]
    rows = x.numel() // L if L else 0
    if codes is None:
        codes = torch.empty(x.shape[:-1] + (L // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(x.shape[:-1] + (L // 16,), dtype=torch.uint8, device=x.device)
    _expect(codes, "codes", torch.uint8, numel=rows * (L // 2), device=x.device)
    _expect(scales, "scales", torch.uint8, numel=rows * (L // 16), device=x.device)
    _device_of(x)
    _check(_lib.attnqat_nvfp4_pack(_ptr(x), _ptr(codes), _ptr(scales), rows, L,
                                   _stream(stream)), "attnqat_nvfp4_pack")
    return codes, scales


def attnqat_fwd_packed(p: attnqat_problem, q, k_codes, k_scales, v_codes, v_scales, o_hp, lse,
                       workspace, stream=None):
    _check_attention(p, q, o_hp=o_hp, lse=lse, workspace=workspace)
    rows = p.batch * p.heads * p.seqlen_kv
    for t, n, per in ((k_codes, "k_codes", p.head_dim // 2), (v_codes, "v_codes", p.head_dim // 2),
                      (k_scales, "k_scales", p.head_dim // 16),
                      (v_scales, "v_scales", p.head_dim // 16)):
        _expect(t, n, torch.uint8, numel=rows * per, device=q.device)
    _check(_lib.attnqat_fwd_packed(ctypes.byref(p), _ptr(q), _ptr(k_codes), _ptr(k_scales),
                                   _ptr(v_codes), _ptr(v_scales), _ptr(o_hp), _ptr(lse),
                                   _ptr(workspace), workspace.numel(), _stream(stream)),
           "attnqat_fwd_packed")


def attnqat_fwd_quantized(p: attnqat_problem, q, k, v, o_hp, lse, o, workspace, stream=None):
    _check_attention(p, q, k, v, o_hp=o_hp, lse=lse, o=o, workspace=workspace)
    _check(_lib.attnqat_fwd_quantized(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp),
                                      _ptr(lse), _ptr(o), _ptr(workspace), workspace.numel(),
                                      _stream(stream)), "attnqat_fwd_quantized")


def attnqat_bwd(p: attnqat_problem, q, k, v, o_hp, d_o, lse, dq, dk, dv, workspace, stream=None):
    _check_attention(p, q, k, v, o_hp=o_hp, d_o=d_o, lse=lse, dq=dq, dk=dk, dv=dv,
                     workspace=workspace)
    _check(_lib.attnqat_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp), _ptr(d_o),
                            _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                            workspace.numel(), _stream(stream)), "attnqat_bwd")


NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20


def attnqat_bwd_noalloc(p: attnqat_problem, q, k, v, o_hp, d_o, lse, dq, dk, dv, stream=None):
    """attnqat_bwd with the library's static device workspace (no allocation)."""
    _check_attention(p, q, k, v, o_hp=o_hp, d_o=d_o, lse=lse, dq=dq, dk=dk, dv=dv)
    _check(_lib.attnqat_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp),
                                    _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _stream(stream)), "attnqat_bwd_noalloc")


def attnqat_fwd_timed(p: attnqat_problem, q, k, v, o_hp, lse, workspace, events, stream=None):
    """``events``: a ctypes array of 4 hipEvent_t handles, a start/stop pair
    per launch (attnqat_instrument.h)."""
    _check_attention(p, q, k, v, o_hp=o_hp, lse=lse, workspace=workspace)
    _check(_lib.attnqat_fwd_timed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp),
                                  _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream),
                                  events), "attnqat_fwd_timed")


def attnqat_fwd_quantized_timed(p: attnqat_problem, q, k, v, o_hp, lse, o, workspace, events,
                                stream=None):
    """``events``: a ctypes array of 6 hipEvent_t handles, a start/stop pair
    per launch (attnqat_instrument.h)."""
    _check_attention(p, q, k, v, o_hp=o_hp, lse=lse, o=o, workspace=workspace)
    _check(_lib.attnqat_fwd_quantized_timed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(o_hp), _ptr(lse), _ptr(o), _ptr(workspace),
                                            workspace.numel(), _stream(stream), events),
           "attnqat_fwd_quantized_timed")


def attnqat_bwd_timed(p: attnqat_problem, q, k, v, o_hp, d_o, lse, dq, dk, dv, workspace,
                      events, stream=None):
    """``events``: a ctypes array of 6 hipEvent_t handles, a start/stop pair
    per launch (attnqat_instrument.h)."""
    _check_attention(p, q, k, v, o_hp=o_hp, d_o=d_o, lse=lse, dq=dq, dk=dk, dv=dv,
                     workspace=workspace)
    _check(_lib.attnqat_bwd_timed(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o_hp),
                                  _ptr(d_o), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _ptr(workspace), workspace.numel(), _stream(stream), events),
           "attnqat_bwd_timed")


def attnqat_probe_mfma_peak(a, b, out, blocks, iters, stream=None):
    """Sustained bf16 MFMA rate probe (attnqat_instrument.h); the caller times
    it.  Returns the flops it executes."""
    need = 32 * 256 * blocks
    _expect(a, "a", torch.bfloat16)
    _expect(b, "b", torch.bfloat16, device=a.device)
    _expect(out, "out", torch.float32, device=a.device)
    if a.numel() < need or b.numel() < need or out.numel() < 256 * blocks:
        raise ValueError("probe buffers too small")
    _device_of(a)
    _check(_lib.attnqat_probe_mfma_peak(_ptr(a), _ptr(b), _ptr(out), blocks, iters,
                                        _stream(stream)), "attnqat_probe_mfma_peak")
    return blocks * 4 * iters * 16 * 32768


def attnqat_probe_issue_mix(mode, valu_per_mfma, agpr, inp, out, blocks, threads, iters,
                            stream=None):
    """MFMA / VALU issue-mix probe (attnqat_instrument.h); the caller times it."""
    _expect(inp, "in", torch.bfloat16)
    _expect(out, "out", torch.float32, device=inp.device)
    if inp.numel() < 8192 or out.numel() < blocks * threads:
        raise ValueError("probe buffers too small")
    _device_of(inp)
    _check(_lib.attnqat_probe_issue_mix(mode, valu_per_mfma, int(bool(agpr)), _ptr(inp),
                                        _ptr(out), blocks, threads, iters, _stream(stream)),
           "attnqat_probe_issue_mix")


def attnqat_probe_lds_write(pattern, out, blocks, iters, stream=None):
    """LDS write-pattern probe (attnqat_instrument.h); the caller times it."""
    _expect(out, "out", torch.float32)
    if out.numel() < blocks * 256:
        raise ValueError("probe buffer too small")
    _device_of(out)
    _check(_lib.attnqat_probe_lds_write(pattern, _ptr(out), blocks, iters, _stream(stream)),
           "attnqat_probe_lds_write")


# ---- conveniences (allocation via torch, then one C call) --------------------

def _check_bhsd(*ts):
    for t in ts:
        if t.dtype != torch.bfloat16 or t.dim() != 4 or not t.is_contiguous():
            raise ValueError("expected contiguous bf16 (B, H, S, D) tensors")


def nvfp4_attention_qat_forward(q, k, v, is_causal=False, softmax_scale=None, p_scale=1.0,
                                workspace=None, current_stream=None, quantized_output=False):
    """Returns ``(high_precision_o, lse)`` of the QAT forward, or
    ``(o, high_precision_o, lse)`` with ``quantized_output=True``, where ``o``
    is the quantized user-visible output fake_nvfp4(P) V^.  Without
    ``softmax_scale`` the page's default 1/sqrt(128) is used (whatever the
    head dim), as in its wrapper; the backward must get the same value."""
    _check_bhsd(q, k, v)
    if softmax_scale is None:
        softmax_scale = PAGE_DEFAULT_SOFTMAX_SCALE
    p = problem_for(q, k, is_causal, softmax_scale, p_scale)
    o_hp = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(attnqat_fwd_workspace_bytes(p), dtype=torch.uint8,
                                device=q.device)
    if not quantized_output:
        attnqat_fwd(p, q, k, v, o_hp, lse, workspace, current_stream)
        return o_hp, lse
    o = torch.empty_like(q)
    attnqat_fwd_quantized(p, q, k, v, o_hp, lse, o, workspace, current_stream)
    return o, o_hp, lse


def nvfp4_attention_qat_backward(do, q, k, v, high_precision_o, lse, is_causal=False,
                                 softmax_scale=None, p_scale=1.0, dq_tensor=None,
                                 dk_tensor=None, dv_tensor=None, workspace=None,
                                 current_stream=None):
    """Returns ``{"dq_tensor", "dk_tensor", "dv_tensor"}``.  Without
    ``softmax_scale`` the page's default 1/sqrt(128) is used, as in its
    wrapper; it must be the forward's."""
    _check_bhsd(do, q, k, v, high_precision_o)
    if softmax_scale is None:
        softmax_scale = PAGE_DEFAULT_SOFTMAX_SCALE
    p = problem_for(q, k, is_causal, softmax_scale, p_scale)
    dq = torch.empty_like(q) if dq_tensor is None else dq_tensor
    dk = torch.empty_like(k) if dk_tensor is None else dk_tensor
    dv = torch.empty_like(v) if dv_tensor is None else dv_tensor
    if workspace is None:
        workspace = torch.empty(attnqat_bwd_workspace_bytes(p), dtype=torch.uint8,
                                device=q.device)
    attnqat_bwd(p, q, k, v, high_precision_o, do, lse, dq, dk, dv, workspace, current_stream)
    return {"dq_tensor": dq, "dk_tensor": dk, "dv_tensor": dv}
