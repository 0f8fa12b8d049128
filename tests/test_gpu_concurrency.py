"""Concurrent calls: two host threads, each with its own HIP stream and
buffers, run independent dispatch + combine steps at the same time (ctypes
releases the GIL during the calls).  Every result must equal the same step run
alone, byte for byte, which checks that the library keeps no state between
calls and that calls on different streams do not interfere.

Every test prints the case it runs before touching the GPU.
"""
import threading

import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
from combine_topk_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

ROUNDS = 6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


class Step:
    """One workload's buffers on one stream (default priority)."""

    def __init__(self, wl, fused):
        wl = wl.replace(expert_output="random")
        self.wl, self.fused = wl, fused
        self.cfg = M.MoeConfig(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.K, num_ranks=wl.R,
                               layout=wl.layout, align=wl.align, capacity=wl.capacity, quant=wl.quant)
        self.stream = torch.cuda.Stream()
        self.d = M.DispatchBuffers(self.cfg, device="cuda")
        inp = W.make_inputs(wl)
        y = W.expert_outputs(wl, inp, rows=self.d.rows)
        self.idx = torch.from_numpy(inp.topk_idx).cuda()
        self.w = torch.from_numpy(inp.topk_w).cuda()
        self.x = torch.from_numpy(inp.x.view(np.int16)).cuda()
        self.y = torch.from_numpy(y.view(np.int16)).cuda()
        self.out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()

    def run(self):
        c, T, d, s = self.cfg, self.wl.T, self.d, self.stream
        if self.fused:
            M.moe_dispatch_fused(c, T, self.idx, self.x, None, d.handle, d.workspace, d.out_x, d.out_scale,
                                 stream=s)
        else:
            M.moe_dispatch_layout(c, T, self.idx, d.handle, d.workspace, stream=s)
            M.moe_dispatch(c, T, self.x, None, d.handle, d.out_x, d.out_scale, stream=s)
        M.moe_combine(c, T, self.y, self.w, d.handle, self.out, stream=s)

    def result(self):
        self.stream.synchronize()
        t = dict(self.d.handle.tensors())
        t.update(out_x=self.d.out_x, out_scale=self.d.out_scale, out=self.out)
        return {k: v.cpu().numpy().view(np.uint8).reshape(-1).copy() for k, v in t.items() if v is not None}

    def clear(self):
        for v in list(self.d.handle.tensors().values()) + [self.d.out_x, self.out]:
            v.view(torch.uint8).fill_(0xA5)
        if self.d.out_scale is not None:
            self.d.out_scale.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()


PAIRS = [
    ("deepseekv3_decode_T256", "qwen3moe_decode_T128", True),
    ("deepseekv3_prefill_T8192", "deepseekv3_decode_T256", True),
    ("deepseekv3_prefill_T8192_mxfp8", "tiny_T64", False),
]


@pytest.mark.parametrize("a,b,fused", PAIRS, ids=[f"{a}+{b}" for a, b, _ in PAIRS])
def test_two_threads_two_streams(a, b, fused):
    _say(f"concurrent steps {a} and {b} (fused={fused}), {ROUNDS} rounds on two host threads")
    steps = [Step(W.WORKLOADS[a], fused), Step(W.WORKLOADS[b], fused)]
    ref = []
    for s in steps:  # each step alone
        s.clear()
        s.run()
        ref.append(s.result())
    for s in steps:
        s.clear()
    errors = []

    def worker(s, k):
        try:
            for _ in range(ROUNDS):
                s.run()
        except Exception as e:  # reported below
            errors.append((k, e))

    th = [threading.Thread(target=worker, args=(s, k)) for k, s in enumerate(steps)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    for k, s in enumerate(steps):
        got = s.result()
        for name in ref[k]:
            assert np.array_equal(got[name], ref[k][name]), f"{s.wl.name}: {name} differs when run concurrently"
    print("  concurrent results equal the single runs", flush=True)
