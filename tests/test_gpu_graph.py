"""The forward and backward recorded in a HIP graph (torch.cuda.graph) and
replayed, as a training step or a serving loop would run them.

Every entry point only launches kernels on the caller's stream: no device
allocation, no memset, no host synchronization inside a call.  So a capture
must succeed, and each replay must reproduce the eager results bit for bit:
after the input buffers are refilled with other data between replays (the
graph reads them when it runs, not when it was recorded), with eager work
between the replays, and with the outputs overwritten before each replay.
The cases take the unsplit backward, the split loops with their reduction
launch, the short causal forward split over keys, the quantized output, the
allocation-free backward, and the packed 32-query-tile forward with its
merge launch and the fused Q fake-quant.
"""
from __future__ import annotations

import math

import pytest
import torch

from nvfp4_fake_quantized_amd import binding as B
from tests._util import bwd_plan, fwd_plan

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _host_inputs(b, h, nq, nkv, d, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, h, nq, d, generator=g).bfloat16()
    k = torch.randn(b, h, nkv, d, generator=g).bfloat16()
    v = torch.randn(b, h, nkv, d, generator=g).bfloat16()
    do = torch.randn(b, h, nq, d, generator=g).bfloat16()
    return q, k, v, do


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


class _Step:
    """Device buffers of one problem and the calls of one step on them."""

    def __init__(self, b, h, nq, nkv, d, causal, kind):
        self.kind = kind
        self.q = torch.empty(b, h, nq, d, dtype=torch.bfloat16, device=DEV)
        self.k = torch.empty(b, h, nkv, d, dtype=torch.bfloat16, device=DEV)
        self.v = torch.empty_like(self.k)
        self.do = torch.empty_like(self.q)
        self.p = B.problem_for(self.q, self.k, causal, 1.0 / math.sqrt(d))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty(b, h, nq, dtype=torch.float32, device=DEV)
        self.wsf = torch.empty(B.attnqat_fwd_workspace_bytes(self.p), dtype=torch.uint8, device=DEV)
        if kind == "packed":
            self.kc = torch.empty(b, h, nkv, d // 2, dtype=torch.uint8, device=DEV)
            self.ks = torch.empty(b, h, nkv, d // 16, dtype=torch.uint8, device=DEV)
            self.vc, self.vs = torch.empty_like(self.kc), torch.empty_like(self.ks)
            self.outs = [self.o, self.lse]
            return
        self.oq = torch.empty_like(self.q) if kind == "quantized" else None
        self.wsb = (None if kind == "noalloc" else
                    torch.empty(B.attnqat_bwd_workspace_bytes(self.p), dtype=torch.uint8, device=DEV))
        self.g = [torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)]
        self.outs = [self.o, self.lse] + ([self.oq] if self.oq is not None else []) + self.g

    def load(self, host):
        """Refills the input buffers (eager copies; for packed K/V the codes
        and scale bytes are made here, outside the step)."""
        for dst, src in zip((self.q, self.k, self.v, self.do), host):
            dst.copy_(src)
        if self.kind == "packed":
            B.attnqat_nvfp4_pack(self.k, self.kc, self.ks)
            B.attnqat_nvfp4_pack(self.v, self.vc, self.vs)

    def run(self):
        """The step's calls, on the current stream."""
        p = self.p
        if self.kind == "packed":
            B.attnqat_fwd_packed(p, self.q, self.kc, self.ks, self.vc, self.vs, self.o, self.lse,
                                 self.wsf)
            return
        if self.kind == "quantized":
            B.attnqat_fwd_quantized(p, self.q, self.k, self.v, self.o, self.lse, self.oq, self.wsf)
        else:
            B.attnqat_fwd(p, self.q, self.k, self.v, self.o, self.lse, self.wsf)
        if self.kind == "noalloc":
            B.attnqat_bwd_noalloc(p, self.q, self.k, self.v, self.o, self.do, self.lse, *self.g)
        else:
            B.attnqat_bwd(p, self.q, self.k, self.v, self.o, self.do, self.lse, *self.g, self.wsb)

    def poison(self):
        for t in self.outs:
            t.fill_(float("nan"))


CASES = [  # b, h, nq, nkv, d, causal, kind
    (1, 16, 2048, 2048, 128, False, "plain"),    # backward loops unsplit
    (1, 2, 512, 512, 64, True, "plain"),         # split backward loops, short causal forward split
    (2, 3, 300, 700, 128, False, "quantized"),   # two-pass forward, cross-attention tails
    (1, 4, 1000, 1000, 128, True, "noalloc"),    # the allocation-free backward
    (1, 8, 16, 8192, 128, False, "packed"),      # 32-query tiles from packed K/V
]


@pytest.mark.parametrize("b,h,nq,nkv,d,causal,kind", CASES)
def test_graph_replays_match_eager_calls(b, h, nq, nkv, d, causal, kind):
    print(f"[graph] B{b} H{h} Nq{nq} Nkv{nkv} D{d} causal={causal} {kind}: "
          f"fwd plan {fwd_plan(b, h, nq, nkv, causal)}, bwd plan {bwd_plan(b, h, nq, nkv)}",
          flush=True)
    st = _Step(b, h, nq, nkv, d, causal, kind)
    data = [_host_inputs(b, h, nq, nkv, d, seed) for seed in (11, 12)]
    # eager results for both input sets
    refs = []
    for host in data:
        st.load(host)
        st.poison()
        st.run()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in st.outs])
    assert not any(_same(a, b_) for a, b_ in zip(refs[0], refs[1]))
    # record the step once (the library was already initialized by the eager calls)
    st.load(data[0])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()
    for rep, i in enumerate((1, 0, 1, 1)):
        st.load(data[i])
        st.poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(range(len(st.outs)), st.outs, refs[i]):
            assert _same(got, ref), f"replay {rep} (inputs {i}): output {name} differs"
    # eager calls still agree after the replays
    st.load(data[0])
    st.poison()
    st.run()
    torch.cuda.synchronize()
    for got, ref in zip(st.outs, refs[0]):
        assert _same(got, ref)
    del graph
