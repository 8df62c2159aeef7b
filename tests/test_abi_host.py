"""Host-side tests of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/*.h declares,
and reject invalid arguments on the host, before any HIP call, with the
documented status codes.  Pointers handed to the library here are never
dereferenced: every call below returns during validation.
"""
from __future__ import annotations

import ctypes
import glob
import math
import os
import re

import pytest

from nvfp4_fake_quantized_amd import binding as B
from tests._util import bwd_plan, fwd_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = []
    for path in HEADERS:
        text = open(path).read()
        names += re.findall(r"ATTNQAT_API\s+[\w\s\*]+?\b(attnqat_\w+)\s*\(", text)
    return names


def test_header_declares_expected_functions():
    names = _declared_functions()
    assert set(names) == set(B.EXPORTED), (names, B.EXPORTED)
    for required in ("attnqat_fake_nvfp4", "attnqat_fwd", "attnqat_bwd"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_struct_layout_matches_header():
    assert ctypes.sizeof(B.attnqat_problem) == 32
    assert ctypes.sizeof(B.attnqat_ws_layout) == 8 * ctypes.sizeof(ctypes.c_size_t)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert B.status_string(code) and B.status_string(code) != "unknown status"
    assert B.status_string(7) == "unknown status"


def _prob(**kw):
    base = dict(batch=1, heads=16, seqlen_q=4096, seqlen_kv=4096, head_dim=128, causal=False,
                softmax_scale=1 / math.sqrt(128), p_scale=1.0)
    base.update(kw)
    return B.make_problem(base["batch"], base["heads"], base["seqlen_q"], base["seqlen_kv"],
                          base["head_dim"], base["causal"], base["softmax_scale"],
                          base["p_scale"])


@pytest.mark.parametrize("kw,code", [
    ({}, B.OK),
    ({"head_dim": 64}, B.OK),
    ({"seqlen_q": 100, "seqlen_kv": 333}, B.OK),
    ({"causal": True}, B.OK),
    ({"head_dim": 96}, B.ERR_UNSUPPORTED),
    ({"head_dim": 256}, B.ERR_UNSUPPORTED),
    ({"causal": True, "seqlen_kv": 2048}, B.ERR_UNSUPPORTED),
    ({"batch": 0}, B.ERR_INVALID_ARGUMENT),
    ({"heads": -1}, B.ERR_INVALID_ARGUMENT),
    ({"seqlen_q": 0}, B.ERR_INVALID_ARGUMENT),
    ({"softmax_scale": 0.0}, B.ERR_INVALID_ARGUMENT),
    ({"softmax_scale": float("nan")}, B.ERR_INVALID_ARGUMENT),
    ({"softmax_scale": float("inf")}, B.ERR_INVALID_ARGUMENT),
    ({"p_scale": -1.0}, B.ERR_INVALID_ARGUMENT),
    ({"batch": 300, "heads": 300}, B.ERR_UNSUPPORTED),
    # at most 2^28 rows per tensor (batch * heads * max(seqlen_q, seqlen_kv))
    ({"batch": 300, "heads": 300, "seqlen_q": 128, "seqlen_kv": 128}, B.OK),
    ({"batch": 1, "heads": 65536}, B.OK),
    ({"batch": 1, "heads": 65537}, B.ERR_UNSUPPORTED),
    ({"batch": 1, "heads": 65536, "seqlen_q": 16, "seqlen_kv": 4097}, B.ERR_UNSUPPORTED),
])
def test_check_support(kw, code):
    assert B.attnqat_check_support(_prob(**kw)) == code


def test_check_support_null():
    assert B._lib.attnqat_check_support(None) == B.ERR_INVALID_ARGUMENT


def test_workspace_sizes_and_layout():
    p = _prob()
    bh, n, d = 16, 4096, 128
    L = B.attnqat_workspace_layout(p, B.WS_BWD)
    assert L["total_bytes"] == B.attnqat_bwd_workspace_bytes(p)
    assert L["q_hat"] == 0
    assert L["k_hat"] >= bh * n * d * 2
    assert L["v_hat"] >= L["k_hat"] + bh * n * d * 2
    assert L["q_scale"] >= L["v_hat"] + bh * n * d * 2
    assert L["delta"] >= L["v_scale"] + bh * n * d // 16
    assert L["total_bytes"] >= L["delta"] + bh * n * 4
    for key in ("q_hat", "k_hat", "v_hat", "q_scale", "k_scale", "v_scale", "delta"):
        assert L[key] % 256 == 0
    F = B.attnqat_workspace_layout(p, B.WS_FWD)
    assert F["delta"] == ctypes.c_size_t(-1).value
    assert F["total_bytes"] == B.attnqat_fwd_workspace_bytes(p)
    with pytest.raises(B.AttnQatError):
        B.attnqat_workspace_layout(p, 5)
    with pytest.raises(B.AttnQatError):
        B.attnqat_bwd_workspace_bytes(_prob(head_dim=80))


def _vp(addr):
    return ctypes.c_void_p(addr)


def test_fwd_bwd_reject_bad_arguments_before_launch():
    lib = B._lib
    p = _prob(batch=1, heads=1, seqlen_q=128, seqlen_kv=128)
    need = B.attnqat_bwd_workspace_bytes(p)
    a = [_vp(0x10000 * (i + 1)) for i in range(10)]  # aligned, never dereferenced
    # null pointer
    args = list(a)
    args[3] = None
    assert lib.attnqat_bwd(ctypes.byref(p), *args[:9], args[9], need, None) == \
        B.ERR_INVALID_ARGUMENT
    # misaligned pointer
    args = list(a)
    args[2] = _vp(0x30008)
    assert lib.attnqat_bwd(ctypes.byref(p), *args[:9], args[9], need, None) == B.ERR_MISALIGNED
    # workspace too small
    assert lib.attnqat_bwd(ctypes.byref(p), *a[:9], a[9], need - 1, None) == \
        B.ERR_WORKSPACE_TOO_SMALL
    # invalid problem wins over everything else
    bad = _prob(head_dim=32)
    assert lib.attnqat_bwd(ctypes.byref(bad), *a[:9], a[9], need, None) == B.ERR_UNSUPPORTED
    assert lib.attnqat_bwd(None, *a[:9], a[9], need, None) == B.ERR_INVALID_ARGUMENT
    # forward
    fneed = B.attnqat_fwd_workspace_bytes(p)
    assert lib.attnqat_fwd(ctypes.byref(p), a[0], a[1], None, a[3], a[4], a[5], fneed, None) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fwd(ctypes.byref(p), a[0], a[1], a[2], _vp(0x40004), a[4], a[5], fneed,
                           None) == B.ERR_MISALIGNED
    assert lib.attnqat_fwd(ctypes.byref(p), *a[:6], fneed - 256, None) == \
        B.ERR_WORKSPACE_TOO_SMALL


def test_fake_nvfp4_rejects_bad_arguments_before_launch():
    lib = B._lib
    x, y, s = _vp(0x10000), _vp(0x20000), _vp(0x30000)
    assert lib.attnqat_fake_nvfp4(x, 7, y, s, 4, 16, None) == B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fake_nvfp4(x, B.DTYPE_BF16, y, s, 4, 24, None) == B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fake_nvfp4(x, B.DTYPE_BF16, y, s, -1, 16, None) == B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fake_nvfp4(x, B.DTYPE_BF16, y, s, 4, 0, None) == B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fake_nvfp4(None, B.DTYPE_BF16, y, s, 4, 16, None) == \
        B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_fake_nvfp4(_vp(0x10002), B.DTYPE_BF16, y, s, 4, 16, None) == \
        B.ERR_MISALIGNED
    # empty input: nothing to do, nothing launched
    assert lib.attnqat_fake_nvfp4(None, B.DTYPE_F32, None, None, 0, 16, None) == B.OK


def test_codec_size_limit():
    """At most 2^35 elements per codec call; beyond: unsupported, decided on
    the host before any pointer is used."""
    lib = B._lib
    big_rows = (1 << 35) // 128 + 1
    assert lib.attnqat_fake_nvfp4(None, B.DTYPE_BF16, None, None, big_rows, 128, None) == \
        B.ERR_UNSUPPORTED
    assert lib.attnqat_fake_nvfp4(None, B.DTYPE_F32, None, None, big_rows, 128, None) == \
        B.ERR_UNSUPPORTED
    assert lib.attnqat_nvfp4_pack(None, None, None, big_rows, 128, None) == B.ERR_UNSUPPORTED
    # at the limit: validation proceeds to the (NULL) pointers
    assert lib.attnqat_fake_nvfp4(None, B.DTYPE_BF16, None, None, (1 << 35) // 128, 128,
                                  None) == B.ERR_INVALID_ARGUMENT


def test_problem_requires_softmax_scale():
    with pytest.raises(ValueError):
        B.make_problem(1, 1, 16, 16, 64, False, None)
    assert abs(B.PAGE_DEFAULT_SOFTMAX_SCALE - 1 / math.sqrt(128)) < 1e-12


def _cpu_case(nq=32, nk=48, d=64, heads=2):
    import torch
    bf = torch.bfloat16
    q = torch.zeros(1, heads, nq, d, dtype=bf)
    k = torch.zeros(1, heads, nk, d, dtype=bf)
    p = B.problem_for(q, k, False, 0.125)
    return p, q, k


@pytest.mark.parametrize("bad", ["k_heads", "v_shape", "lse_dtype", "lse_shape", "dq_dtype",
                                 "dk_shape", "o_hp_shape", "do_noncontig", "ws_dtype"])
def test_binding_rejects_mismatched_tensors(bad):
    """Tensors that do not match the problem raise ValueError in the binding
    (the C ABI cannot see buffer sizes); nothing reaches the library."""
    import torch
    p, q, k = _cpu_case()
    bf = torch.bfloat16
    v = torch.zeros_like(k)
    o = torch.zeros_like(q)
    do = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:3])
    dq, dk, dv = torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v)
    ws = torch.zeros(64, dtype=torch.uint8)
    if bad == "k_heads":
        k = torch.zeros(1, 1, 48, 64, dtype=bf)
    elif bad == "v_shape":
        v = torch.zeros(1, 2, 47, 64, dtype=bf)
    elif bad == "lse_dtype":
        lse = lse.to(bf)
    elif bad == "lse_shape":
        lse = torch.zeros(1, 2, 31)
    elif bad == "dq_dtype":
        dq = dq.float()
    elif bad == "dk_shape":
        dk = torch.zeros(1, 2, 32, 64, dtype=bf)
    elif bad == "o_hp_shape":
        o = torch.zeros(1, 2, 48, 64, dtype=bf)
    elif bad == "do_noncontig":
        do = torch.zeros(1, 2, 64, 32, dtype=bf).transpose(2, 3)
    elif bad == "ws_dtype":
        ws = torch.zeros(16, dtype=torch.int32)
    with pytest.raises(ValueError):
        B.attnqat_bwd(p, q, k, v, o, do, lse, dq, dk, dv, ws)


def test_binding_rejects_host_tensors_and_bad_codec_outputs():
    import torch
    p, q, k = _cpu_case()
    v = torch.zeros_like(k)
    # right shapes on the host: the binding asks for device tensors
    with pytest.raises(ValueError):
        B.attnqat_fwd(p, q, k, v, torch.zeros_like(q), torch.zeros(q.shape[:3]),
                      torch.zeros(64, dtype=torch.uint8))
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # x_hat of the wrong dtype
        B.attnqat_fake_nvfp4(x, x_hat=torch.zeros(4, 32))
    with pytest.raises(ValueError):  # too few scale bytes
        B.attnqat_fake_nvfp4(x, scales=torch.zeros(4, 1, dtype=torch.uint8))
    with pytest.raises(ValueError):  # too few code bytes
        B.attnqat_nvfp4_pack(x, codes=torch.zeros(4, 8, dtype=torch.uint8))


def test_noalloc_rejects_large_workspaces_on_the_host():
    """attnqat_bwd_noalloc refuses a problem whose workspace exceeds its
    static array before any pointer is used."""
    p = _prob(batch=2, heads=40, seqlen_q=8192, seqlen_kv=8192, causal=True)
    assert B.attnqat_bwd_workspace_bytes(p) > B.NOALLOC_MAX_WORKSPACE_BYTES
    rc = B._lib.attnqat_bwd_noalloc(ctypes.byref(p), None, None, None, None, None, None, None,
                                    None, None, None)
    assert rc == B.ERR_UNSUPPORTED
    assert B._lib.attnqat_bwd_noalloc(ctypes.byref(_prob(head_dim=96)), None, None, None, None,
                                      None, None, None, None, None, None) == B.ERR_UNSUPPORTED


def test_instrumentation_entry_points_reject_bad_arguments_before_launch():
    """Timed entry points need 2 events per launch; the probes check their
    ranges and pointers before any HIP call."""
    lib = B._lib
    p = _prob(batch=1, heads=1, seqlen_q=128, seqlen_kv=128)
    need = B.attnqat_bwd_workspace_bytes(p)
    a = [_vp(0x10000 * (i + 1)) for i in range(10)]
    ev5 = (ctypes.c_void_p * 6)(*([0x1000] * 5 + [0]))  # the 6th event is null
    assert lib.attnqat_bwd_timed(ctypes.byref(p), *a[:9], a[9], need, None,
                                 ctypes.cast(ev5, ctypes.c_void_p)) == B.ERR_INVALID_ARGUMENT
    assert lib.attnqat_bwd_timed(ctypes.byref(p), *a[:9], a[9], need, None, None) == \
        B.ERR_INVALID_ARGUMENT
    buf, out = _vp(0x20000), _vp(0x40000)
    # issue mix: mode, FMAs per slot, threads, split mode only with 512 threads, null input
    for args in [(4, 8, 0, buf, out, 1, 256, 1), (0, 12, 0, buf, out, 1, 256, 1),
                 (0, 8, 0, buf, out, 1, 128, 1), (3, 8, 0, buf, out, 1, 256, 1),
                 (0, 8, 0, None, out, 1, 256, 1), (0, 8, 0, buf, out, 0, 256, 1),
                 (0, 8, 0, buf, out, 1, 256, 0)]:
        assert lib.attnqat_probe_issue_mix(*args, None) == B.ERR_INVALID_ARGUMENT, args
    assert lib.attnqat_probe_issue_mix(0, 8, 0, _vp(0x20004), out, 1, 256, 1, None) == \
        B.ERR_MISALIGNED
    # LDS write patterns 0..5
    for args in [(6, out, 1, 1), (-1, out, 1, 1), (0, None, 1, 1), (0, out, 0, 1),
                 (0, out, 1, 1 << 21)]:
        assert lib.attnqat_probe_lds_write(*args, None) == B.ERR_INVALID_ARGUMENT, args
    assert lib.attnqat_probe_lds_write(0, _vp(0x40008), 1, 1, None) == B.ERR_MISALIGNED


def test_backward_workspace_holds_the_split_partials():
    """The backward's workspace grows by the fp32 partial sums of its split
    loops on small problems: s_q * B*H*Nq*D*4 bytes for dQ and
    s_kv * 2 * B*H*Nkv*D*4 for dK/dV (each part 256-byte aligned), and only
    then; large problems (the reference shape, the long workloads) split
    nothing."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    cases = [(1, 16, 1024, 1024, 128, False), (1, 4, 1024, 1024, 64, True), (1, 1, 128, 128, 64, False),
             (1, 2, 333, 333, 128, True), (1, 16, 4096, 4096, 128, False), (2, 40, 8192, 8192, 128, True),
             (1, 40, 32760, 32760, 128, False), (1, 2, 100, 260, 128, False), (1, 1, 1, 5, 128, False),
             (2, 3, 640, 1000, 64, False)]
    kinds = set()
    for b, h, nq, nkv, d, causal in cases:
        p = B.make_problem(b, h, nq, nkv, d, causal, d ** -0.5)
        sq, skv = bwd_plan(b, h, nq, nkv)
        kinds.add((sq > 1, skv > 1))
        bh = b * h
        base = (al(bh * nq * d * 2) + 2 * al(bh * nkv * d * 2) + al(bh * nq * d // 16)
                + 2 * al(bh * nkv * d // 16) + al(bh * nq * 4))
        extra = (al(sq * bh * nq * d * 4) if sq > 1 else 0) + (al(skv * 2 * bh * nkv * d * 4) if skv > 1 else 0)
        assert B.attnqat_bwd_workspace_bytes(p) == base + extra, (b, h, nq, nkv, d, causal, sq, skv)
    assert kinds == {(True, True), (False, False), (True, False)}


def test_forward_workspace_holds_the_key_split_partials():
    """The forward's workspace grows by the partial results of its key runs,
    bh * splits * Nq * (4 D + 8) bytes (each part 256-byte aligned), when it
    splits the keys or takes the 32-query-tile path, and only then."""
    al = lambda x: (x + 255) // 256 * 256  # noqa: E731
    cases = [(1, 2, 16, 4100, 128, False), (1, 4, 64, 3001, 64, False), (2, 3, 100, 8192, 128, False),
             (1, 1, 1, 20000, 128, False), (1, 1, 40, 300, 64, False), (1, 1, 40, 200, 64, False),
             (1, 16, 4096, 4096, 128, False), (1, 1, 128, 128, 64, False),
             (1, 2, 300, 300, 128, True), (2, 40, 8192, 8192, 128, True),
             (1, 1, 32, 100, 64, False), (64, 16, 1, 65536, 128, False), (1, 1, 33, 5000, 128, False),
             (1, 1, 16, 16, 128, True)]
    seen = set()
    for b, h, nq, nkv, d, causal in cases:
        p = B.make_problem(b, h, nq, nkv, d, causal, d ** -0.5)
        S, dec = fwd_plan(b, h, nq, nkv, causal)
        kind = "decode" if dec else ("split" if S > 1 else "plain")
        seen.add(kind)
        bh = b * h
        base = (al(bh * nq * d * 2) + 2 * al(bh * nkv * d * 2) + al(bh * nq * d // 16)
                + 2 * al(bh * nkv * d // 16))
        extra = (al(bh * nq * S * d * 4) + al(bh * nq * S * 8)) if kind != "plain" else 0
        assert B.attnqat_fwd_workspace_bytes(p) == base + extra, (b, h, nq, nkv, d, causal, S, kind)
    assert seen == {"decode", "split", "plain"}
