"""GPU parity of the grouped-GEMM adapters, through the C ABI.

Per case the GPU runs its dispatch layout and dispatch, then the adapter
under test on its own results; the oracle runs its own layout and dispatch of
the same seeded inputs, then its adapter.  Per-row experts, the
masked-to-contiguous repack (rows, scales, offsets, per-row experts), the
contiguous-to-masked repack of seeded expert outputs and the MN-major scale
transpose are compared byte for byte, on sentinel-filled buffers inside guard
bands; a combine through the repacked slab must equal the oracle's.

Every test prints the case it runs before touching the GPU.
"""
import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
import oracle
from combine_topk_idx_amd import workloads as W
from test_gpu_parity import SENT, Guarded, _sentinel, make_cfg, oracle_scale_view, scale_guard

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()
    oracle._load()


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _inputs(wl):
    """Router ids, weights and activations (no expert outputs: the cases make their own)."""
    inp = W.make_inputs(wl)
    return inp.topk_idx, inp.topk_w, inp.x


def _dispatch_on_gpu(wl, cfg, idx, x):
    """Layout + dispatch on the GPU into zero-filled buffers; returns them."""
    T = idx.shape[0]
    bufs = M.DispatchBuffers(cfg)
    bufs.out_x.zero_()
    if bufs.out_scale is not None:
        bufs.out_scale.zero_()
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    d_x = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace)
    M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale)
    torch.cuda.synchronize()
    return bufs


def _dispatch_on_oracle(wl, cfg, idx, x):
    """The oracle's layout and dispatch of the same inputs into zero-filled buffers."""
    rows = M.moe_rows_capacity(cfg)
    h = oracle.dispatch_layout(idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    ox, osc, _ = oracle.dispatch(x, h["pair_to_row"], wl.K, wl.quant, rows)
    return h, ox, osc


MASKED = [
    ("deepseekv3_decode_T256", {}),
    ("qwen3moe_decode_T128", {}),
    ("skewed_prefill_T16384_masked_fp8", dict(H=1024)),           # capacity drops
    ("skewed_prefill_T16384_masked_bf16", dict(T=3000)),
    ("deepseekv3_decode_T256", dict(name="decode_mxfp8", quant=W.QUANT_MXFP8, H=1024)),
    ("deepseekv3_decode_T256", dict(name="decode_ue8m0_c5", quant=W.QUANT_FP8_UE8M0, capacity=5, H=640)),
    ("deepseekv3_decode_T256", dict(name="wide_bf16", quant=W.QUANT_NONE, T=32, H=32768, capacity=8)),
    ("deepseekv3_decode_T256", dict(name="wide_mxfp8", quant=W.QUANT_MXFP8, T=32, H=32768, capacity=8)),
]


@pytest.mark.parametrize("align", [1, 128])
@pytest.mark.parametrize("base,kw", MASKED, ids=[f"{b}-{kw.get('name', kw.get('T', ''))}" for b, kw in MASKED])
def test_repack_round_trip(base, kw, align):
    wl = W.WORKLOADS[base].replace(**kw)
    _say(f"repack {wl.name} T={wl.T} H={wl.H} E={wl.E} C={wl.capacity} quant={wl.quant} align={align}")
    idx, w, x = _inputs(wl)
    cfg = make_cfg(wl)
    E, C, H = wl.E, wl.capacity, wl.H
    fp8 = wl.quant != W.QUANT_NONE
    bufs = _dispatch_on_gpu(wl, cfg, idx, x)
    h, mx, ms = _dispatch_on_oracle(wl, cfg, idx, x)
    recv = h["recv_count"]
    mrows = E * C
    crows = M.moe_repack_rows_capacity(cfg, align)

    # masked -> contiguous: the GPU repacks its dispatch, the oracle repacks its own
    eb = 1 if fp8 else 2
    out_x = Guarded(crows * H * eb, torch.uint8 if fp8 else torch.int16, (crows, H))
    out_s = scale_guard(wl, crows) if fp8 else None
    out_off = Guarded(4 * (E + 1), torch.int32, (E + 1,))
    out_rex = Guarded(4 * crows, torch.int32, (crows,))
    M.moe_repack_masked_to_contiguous(cfg, align, bufs.handle, bufs.out_x,
                                      bufs.out_scale, out_x.view, None if out_s is None else out_s.view,
                                      out_off.view, out_rex.view)
    torch.cuda.synchronize()
    ox = _sentinel(crows * H * eb)
    osc = _sentinel(out_s.nbytes) if fp8 else None
    _, _, off, rex = oracle.repack_masked_to_contiguous(
        mx, ms, recv, C, align, wl.quant, crows,
        out_x=ox.view(np.uint8 if fp8 else np.uint16).reshape(crows, H),
        out_scale=oracle_scale_view(wl.quant, osc, crows) if fp8 else None)
    assert np.array_equal(out_off.host().view(np.int32), off), "offsets differ"
    assert np.array_equal(out_rex.host().view(np.int32), rex), "per-row experts differ"
    assert np.array_equal(out_x.host(), ox), "repacked rows differ"
    if fp8:
        assert np.array_equal(out_s.host(), osc), "repacked scales differ"

    # contiguous -> masked, on seeded stand-in expert outputs in the contiguous layout
    rng = np.random.default_rng(int(align) + wl.seed)
    y_c = W.f32_to_bf16_bits(rng.standard_normal((crows, H)).astype(np.float32))
    d_yc = torch.from_numpy(y_c.view(np.int16)).cuda()
    y_m = Guarded(mrows * H * 2, torch.int16, (mrows, H))
    M.moe_repack_contiguous_to_masked(cfg, bufs.handle, out_off.view, d_yc, y_m.view)
    torch.cuda.synchronize()
    ref = _sentinel(mrows * H * 2).view(np.uint16).reshape(mrows, H)
    oracle.repack_contiguous_to_masked(y_c, recv, off, C, out=ref)
    got = y_m.host().view(np.uint16).reshape(mrows, H)
    assert np.array_equal(got, ref), "slab rows differ"

    # combine through the slab (masked handle) against the oracle's combine of its slab
    T = idx.shape[0]
    d_w = torch.from_numpy(w).cuda()
    out = torch.empty((T, H), dtype=torch.int16, device="cuda")
    M.moe_combine(cfg, T, y_m.view, d_w, bufs.handle, out)
    torch.cuda.synchronize()
    want = oracle.combine(ref, w, h["pair_to_row"])   # combine reads kept rows only, all of them written
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want), "combine through the slab differs"
    print(f"  kept rows {int(recv.sum())}, contiguous rows used {int(off[-1])} of {crows}", flush=True)


ROWEXP = ["deepseekv3_prefill_T8192", "deepseekv3_decode_T256", "skewed_prefill_T16384_contig_fp8",
          "skewed_prefill_T16384_masked_fp8", "tiny_T64"]


@pytest.mark.parametrize("name", ROWEXP)
def test_row_expert(name):
    wl = W.WORKLOADS[name]
    _say(f"row experts {name}")
    idx, _, x = _inputs(wl)
    cfg = make_cfg(wl)
    bufs = _dispatch_on_gpu(wl, cfg, idx, x)
    rows = M.moe_rows_capacity(cfg)
    g = Guarded(4 * rows, torch.int32, (rows,))
    M.moe_row_expert(cfg, bufs.handle, g.view)
    torch.cuda.synchronize()
    h = oracle.dispatch_layout(idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    want = oracle.row_expert(h["expert_offset"], h["recv_count"], rows)
    assert np.array_equal(g.host().view(np.int32), want)


MNMAJOR = [("deepseekv3_prefill_T8192", None), ("deepseekv3_prefill_T8192_mxfp8", None),
           ("deepseekv3_decode_T256", None), ("skewed_prefill_T16384_contig_fp8", None),
           ("deepseekv3_decode_T256", 4097), ("deepseekv3_decode_T256", 3)]


@pytest.mark.parametrize("name,rows", MNMAJOR, ids=[f"{n}-{r}" for n, r in MNMAJOR])
def test_scales_mn_major(name, rows):
    wl = W.WORKLOADS[name]
    _say(f"MN-major scales {name} rows={rows}")
    idx, _, x = _inputs(wl)
    cfg = make_cfg(wl)
    bufs = _dispatch_on_gpu(wl, cfg, idx, x)
    n = bufs.rows if rows is None else rows
    S = M.moe_scale_words(cfg)
    ld = -(-n // 4) * 4
    g = Guarded(4 * S * ld, torch.int32, (S * ld,))
    g.view.view(torch.uint8).fill_(SENT)
    M.moe_scales_mn_major(cfg, n, bufs.out_scale, g.view)
    torch.cuda.synchronize()
    _, _, osc = _dispatch_on_oracle(wl, cfg, idx, x)   # the oracle's scales of the same inputs
    words = np.ascontiguousarray(osc).view(np.uint32).reshape(bufs.rows, S)[:n]
    want = oracle.scales_mn_major(words)
    assert np.array_equal(g.host().view(np.uint32).reshape(S, ld), want)
