"""Graph capture of the per-rank deduplicated chain and of the grouped-GEMM
adapter chain, with fixed shapes, the way a decode loop replays them.

Each chain is captured once on one set of buffers and replayed several times;
before each replay new inputs are copied into the captured buffers and every
output is refilled with a 0xA5 sentinel.  The same calls made eagerly on a
second set of buffers with the same inputs must give the same bytes in every
output (handles included).  The first replay is also checked against the
oracle: the per-rank layout and the final reduction for the deduplicated
chain, the per-row experts and the repacked offsets and per-row experts for
the adapters.

Every test prints the case it runs before touching the GPU.
"""
import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
import oracle
from combine_topk_idx_amd import workloads as W
from test_gpu_dedup import _close, _reduce_scale, run_oracle as dedup_oracle

pytestmark = pytest.mark.gpu

SENT = 0xA5
REPLAYS = 3

DEDUP_CASES = {
    "deepseekv3_decode_T256": W.WORKLOADS["deepseekv3_decode_T256"],
    "qwen3moe_decode_T128": W.WORKLOADS["qwen3moe_decode_T128"],
    "contig_ue8m0_T300_H1024": W.WORKLOADS["deepseekv3_prefill_T8192"].replace(
        name="contig_ue8m0_T300_H1024", T=300, H=1024),
    "contig_mxfp8_T200_H512": W.WORKLOADS["deepseekv3_prefill_T8192"].replace(
        name="contig_mxfp8_T200_H512", T=200, H=512, quant=W.QUANT_MXFP8),
}

ADAPTER_CASES = {
    "deepseekv3_decode_T256": W.WORKLOADS["deepseekv3_decode_T256"].replace(H=1024),
    "qwen3moe_decode_T128": W.WORKLOADS["qwen3moe_decode_T128"],
    "masked_ue8m0_T200_C5": W.WORKLOADS["deepseekv3_decode_T256"].replace(
        name="masked_ue8m0_T200_C5", T=200, H=640, capacity=5, quant=W.QUANT_FP8_UE8M0),
}
ALIGN = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()
    oracle._load()


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _cfg(wl):
    return M.MoeConfig(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.K, num_ranks=wl.R,
                       layout=wl.layout, align=wl.align, capacity=wl.capacity, quant=wl.quant)


def _inputs(wl, rep, rows):
    w2 = wl.replace(seed=wl.seed + 1000 * rep, expert_output="random")
    inp = W.make_inputs(w2)
    return inp, W.expert_outputs(w2, inp, rows=rows)


def _host(tensors):
    return {k: v.cpu().numpy().view(np.uint8).reshape(-1).copy() for k, v in tensors.items()}


def _capture(step):
    """Two warm-up calls on a side stream, then one captured call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    return graph


class DedupChain:
    """Buffers of one deduplicated step: per-rank layout, per-expert layout,
    deduplicated dispatch, expansion, partial combine and reduction."""

    def __init__(self, wl, cfg):
        self.wl, self.cfg = wl, cfg
        T, H = wl.T, wl.H
        self.d = M.DispatchBuffers(cfg, device="cuda")
        self.db = M.DedupBuffers(cfg, device="cuda")
        self.idx = torch.empty((T, wl.K), dtype=torch.int32, device="cuda")
        self.w = torch.empty((T, wl.K), dtype=torch.float32, device="cuda")
        self.x = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.y = torch.empty((self.d.rows, H), dtype=torch.int16, device="cuda")
        self.out = torch.empty((T, H), dtype=torch.int16, device="cuda")

    def outputs(self):
        t = dict(self.d.handle.tensors())
        t.update({"rank_" + k: v for k, v in self.db.handle.tensors().items()})
        t.update(out_x=self.d.out_x, out_scale=self.d.out_scale, send_x=self.db.send_x,
                 send_scale=self.db.send_scale, partial=self.db.partial, out=self.out)
        return {k: v for k, v in t.items() if v is not None}

    def load(self, inp, y):
        self.idx.copy_(torch.from_numpy(inp.topk_idx))
        self.w.copy_(torch.from_numpy(inp.topk_w))
        self.x.copy_(torch.from_numpy(inp.x.view(np.int16)))
        self.y.copy_(torch.from_numpy(y.view(np.int16)))
        for v in self.outputs().values():
            v.view(torch.uint8).fill_(SENT)

    def step(self):
        c, T, d, db = self.cfg, self.wl.T, self.d, self.db
        M.moe_rank_layout(c, T, self.idx, db.handle)
        M.moe_dispatch_layout(c, T, self.idx, d.handle, d.workspace)
        M.moe_dispatch_dedup(c, T, self.x, db.handle, db.send_x, db.send_scale)
        M.moe_expand(c, T, self.idx, db.send_x, db.send_scale, db.handle, d.handle, d.out_x, d.out_scale)
        M.moe_combine_partial(c, T, self.idx, self.y, self.w, d.handle, db.handle, db.partial)
        M.moe_combine_reduce(c, T, db.partial, db.handle, self.out)


class AdapterChain:
    """Buffers of one masked dispatch followed by every adapter: per-row
    experts, masked -> contiguous repack, contiguous -> masked repack of
    expert outputs, MN-major scales, and a combine through the slab."""

    def __init__(self, wl, cfg):
        self.wl, self.cfg = wl, cfg
        T, H, E = wl.T, wl.H, wl.E
        self.d = M.DispatchBuffers(cfg, device="cuda")
        rows, crows = self.d.rows, M.moe_repack_rows_capacity(cfg, ALIGN)
        self.crows = crows
        fp8 = wl.quant != W.QUANT_NONE
        self.idx = torch.empty((T, wl.K), dtype=torch.int32, device="cuda")
        self.w = torch.empty((T, wl.K), dtype=torch.float32, device="cuda")
        self.x = torch.empty((T, H), dtype=torch.int16, device="cuda")
        self.y_c = torch.empty((crows, H), dtype=torch.int16, device="cuda")
        self.rex = torch.empty(rows, dtype=torch.int32, device="cuda")
        self.c_x = torch.empty((crows, H), dtype=torch.uint8 if fp8 else torch.int16, device="cuda")
        self.c_scale = M._scale_buffer(cfg, crows, "cuda") if fp8 else None
        self.c_off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        self.c_rex = torch.empty(crows, dtype=torch.int32, device="cuda")
        self.y_m = torch.empty((rows, H), dtype=torch.int16, device="cuda")
        S = M.moe_scale_words(cfg)
        self.mn = torch.empty(S * ((rows + 3) // 4 * 4), dtype=torch.int32, device="cuda") if fp8 else None
        self.out = torch.empty((T, H), dtype=torch.int16, device="cuda")

    def outputs(self):
        t = dict(self.d.handle.tensors())
        t.update(out_x=self.d.out_x, out_scale=self.d.out_scale, rex=self.rex, c_x=self.c_x,
                 c_scale=self.c_scale, c_off=self.c_off, c_rex=self.c_rex, y_m=self.y_m, mn=self.mn,
                 out=self.out)
        return {k: v for k, v in t.items() if v is not None}

    def load(self, inp, y_c):
        self.idx.copy_(torch.from_numpy(inp.topk_idx))
        self.w.copy_(torch.from_numpy(inp.topk_w))
        self.x.copy_(torch.from_numpy(inp.x.view(np.int16)))
        self.y_c.copy_(torch.from_numpy(y_c.view(np.int16)))
        for v in self.outputs().values():
            v.view(torch.uint8).fill_(SENT)

    def step(self):
        c, T, d = self.cfg, self.wl.T, self.d
        M.moe_dispatch_fused(c, T, self.idx, self.x, None, d.handle, d.workspace, d.out_x, d.out_scale)
        M.moe_row_expert(c, d.handle, self.rex)
        M.moe_repack_masked_to_contiguous(c, ALIGN, d.handle, d.out_x, d.out_scale, self.c_x, self.c_scale,
                                          self.c_off, self.c_rex)
        M.moe_repack_contiguous_to_masked(c, d.handle, self.c_off, self.y_c, self.y_m)
        if self.mn is not None:
            M.moe_scales_mn_major(c, d.rows, d.out_scale, self.mn)
        M.moe_combine(c, T, self.y_m, self.w, d.handle, self.out)


def _replay_against_eager(chain_cls, wl, rows_of, oracle_check):
    cfg = _cfg(wl)
    g = chain_cls(wl, cfg)   # captured
    e = chain_cls(wl, cfg)   # eager reference
    rows = rows_of(g)
    inp, y = _inputs(wl, 0, rows)
    g.load(inp, y)
    graph = _capture(g.step)
    for rep in range(REPLAYS):
        inp, y = _inputs(wl, rep, rows)
        g.load(inp, y)
        e.load(inp, y)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _host(g.outputs())
        e.step()
        torch.cuda.synchronize()
        ref = _host(e.outputs())
        assert got.keys() == ref.keys()
        for k in ref:
            assert np.array_equal(got[k], ref[k]), f"replay {rep}: {k} differs from the eager calls"
        if rep == 0:
            oracle_check(e, inp, y)
        print(f"  replay {rep}: equal to eager", flush=True)


@pytest.mark.parametrize("name", list(DEDUP_CASES))
def test_dedup_graph_replays_match_eager(name):
    wl = DEDUP_CASES[name]
    _say(f"dedup graph capture {name}: T={wl.T} H={wl.H} E={wl.E} K={wl.K} R={wl.R} layout={wl.layout} "
         f"quant={wl.quant}, {REPLAYS} replays")

    def check(chain, inp, y):
        o = dedup_oracle(wl, inp.topk_idx, inp.x, inp.topk_w, y, chain.cfg)
        for k in ("rank_token_count", "rank_token_offset", "token_rank_row", "rank_row_to_token"):
            got = getattr(chain.db.handle, k).cpu().numpy()
            assert np.array_equal(got[:o["rk"][k].size], o["rk"][k]), f"{k} differs from the oracle"
        ref = oracle.combine_reduce(o["partial"], o["rk"]["token_rank_row"], wl.R)
        out = chain.out.cpu().numpy().view(np.uint16)
        _close(out, ref, _reduce_scale(o["partial"], o["rk"], wl.R), "reduction")

    _replay_against_eager(DedupChain, wl, lambda c: c.d.rows, check)


@pytest.mark.parametrize("name", list(ADAPTER_CASES))
def test_adapter_graph_replays_match_eager(name):
    wl = ADAPTER_CASES[name]
    assert wl.layout == W.LAYOUT_MASKED
    _say(f"adapter graph capture {name}: T={wl.T} H={wl.H} E={wl.E} K={wl.K} C={wl.capacity} "
         f"quant={wl.quant} align={ALIGN}, {REPLAYS} replays")

    def check(chain, inp, y):
        rows = chain.d.rows
        h = oracle.dispatch_layout(inp.topk_idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
        want = oracle.row_expert(h["expert_offset"], h["recv_count"], rows)
        assert np.array_equal(chain.rex.cpu().numpy(), want), "per-row experts differ from the oracle"
        ox, osc, _ = oracle.dispatch(inp.x, h["pair_to_row"], wl.K, wl.quant, rows)
        _, _, off, rex = oracle.repack_masked_to_contiguous(ox, osc, h["recv_count"], wl.capacity, ALIGN,
                                                            wl.quant, chain.crows)
        assert np.array_equal(chain.c_off.cpu().numpy(), off), "repacked offsets differ from the oracle"
        assert np.array_equal(chain.c_rex.cpu().numpy(), rex), "repacked row experts differ from the oracle"

    _replay_against_eager(AdapterChain, wl, lambda c: c.crows, check)
