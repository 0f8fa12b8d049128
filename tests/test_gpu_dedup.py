"""GPU parity of the per-rank deduplicated exchange, through the C ABI.

Per case: the per-rank layout (all four arrays), the deduplicated dispatch
(send rows and scales), the receive-side expansion (which must also equal
moe_dispatch's rows byte for byte), the partial combine and the final
reduction, each against the CPU oracle run on the same seeded inputs.  Every output
buffer starts as a 0xA5 sentinel on both sides and is compared whole, inside
guard bands that must survive.  Integer and byte outputs are bit-exact.  The
partial sums and the reduction use the same fp32 operation order as the
oracle, so they are expected bit-exact as well; they are checked with the
tolerance |g - o| <= 1e-2 |o| + 1e-5 S (S = sum of |terms|) and the count of
unequal elements is reported.

Every test prints the case it runs before touching the GPU.
"""
import zlib

import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
import oracle
from combine_topk_idx_amd import workloads as W
from test_gpu_parity import SENT, Guarded, _sentinel, make_cfg, oracle_scale_view, random_case, scale_cols, scale_guard

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()
    oracle._load()


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


def _scale_view(quant, buf, rows):
    return oracle_scale_view(quant, buf, rows)


def run_gpu(wl, idx, x, w, y, cfg):
    T, H, R = idx.shape[0], wl.H, wl.R
    fp8 = wl.quant != W.QUANT_NONE
    qrows = M.moe_rank_rows_capacity(cfg)
    rows = M.moe_rows_capacity(cfg)
    nsc = scale_cols(wl)
    eb = 1 if fp8 else 2
    rh = M.RankHandle.__new__(M.RankHandle)
    rbufs = {}
    for name, n in (("rank_token_count", R), ("rank_token_offset", R + 1),
                    ("token_rank_row", cfg.max_tokens * R), ("rank_row_to_token", qrows)):
        g = Guarded(4 * n, torch.int32, (n,))
        rbufs[name] = g
        setattr(rh, name, g.view)
    rh.c = M.MoeRankHandle(*(rbufs[n].view.data_ptr() for n, _ in M.MoeRankHandle._fields_))
    h = M.Handle(cfg)
    ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    send_x = Guarded(qrows * H * eb, torch.uint8 if fp8 else torch.int16, (qrows, H))
    send_sc = scale_guard(wl, qrows) if fp8 else None
    exp_x = Guarded(rows * H * eb, torch.uint8 if fp8 else torch.int16, (rows, H))
    exp_sc = scale_guard(wl, rows) if fp8 else None
    dir_x = Guarded(rows * H * eb, torch.uint8 if fp8 else torch.int16, (rows, H))
    dir_sc = scale_guard(wl, rows) if fp8 else None
    partial = Guarded(qrows * H * 2, torch.int16, (qrows, H))
    out = Guarded(T * H * 2, torch.int16, (T, H))
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    d_w = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    d_x = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    d_y = torch.from_numpy(np.ascontiguousarray(y).view(np.int16)).cuda()
    sv = lambda g: None if g is None else g.view
    M.moe_rank_layout(cfg, T, d_idx, rh)
    M.moe_dispatch_layout(cfg, T, d_idx, h, ws)
    M.moe_dispatch_dedup(cfg, T, d_x, rh, send_x.view, sv(send_sc))
    M.moe_expand(cfg, T, d_idx, send_x.view, sv(send_sc), rh, h, exp_x.view, sv(exp_sc))
    M.moe_dispatch(cfg, T, d_x, None, h, dir_x.view, sv(dir_sc))
    M.moe_combine_partial(cfg, T, d_idx, d_y, d_w, h, rh, partial.view)
    M.moe_combine_reduce(cfg, T, partial.view, rh, out.view)
    torch.cuda.synchronize()
    res = {n: g.host().view(np.int32) for n, g in rbufs.items()}
    res["pair_to_row"] = h.pair_to_row.cpu().numpy()[:T * wl.K]
    for name, g in (("send_x", send_x), ("send_scale", send_sc), ("exp_x", exp_x), ("exp_scale", exp_sc),
                    ("dir_x", dir_x), ("dir_scale", dir_sc)):
        res[name] = None if g is None else g.host()
    res["partial"] = partial.host().view(np.uint16).reshape(qrows, H)
    res["out"] = out.host().view(np.uint16).reshape(T, H)
    return res


def run_oracle(wl, idx, x, w, y, cfg):
    T, H, R, E, K = idx.shape[0], wl.H, wl.R, wl.E, wl.K
    fp8 = wl.quant != W.QUANT_NONE
    qrows = M.moe_rank_rows_capacity(cfg)
    rows = M.moe_rows_capacity(cfg)
    nsc = scale_cols(wl)
    rk = oracle.rank_layout(idx, E, R, rows_cap=qrows)
    res = {}
    for name, n in (("rank_token_count", R), ("rank_token_offset", R + 1),
                    ("token_rank_row", cfg.max_tokens * R), ("rank_row_to_token", qrows)):
        a = _sentinel(4 * n).view(np.int32)
        a[:rk[name].size] = rk[name]
        res[name] = a
    lay = oracle.dispatch_layout(idx, E, R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    sx = _sentinel(qrows * H * (1 if fp8 else 2))
    ss = _sentinel(qrows * nsc * 4) if fp8 else None
    oracle.dispatch_dedup(x, rk["token_rank_row"], R, wl.quant, qrows,
                          out_x=sx.view(np.uint8 if fp8 else np.uint16).reshape(qrows, H),
                          out_scale=_scale_view(wl.quant, ss, qrows) if fp8 else None)
    ex = _sentinel(rows * H * (1 if fp8 else 2))
    es = _sentinel(rows * nsc * 4) if fp8 else None
    oracle.expand(idx, E, R, wl.quant, sx.view(np.uint8 if fp8 else np.uint16).reshape(qrows, H),
                  _scale_view(wl.quant, ss, qrows) if fp8 else None, rk["token_rank_row"], lay["pair_to_row"],
                  rows, out_x=ex.view(np.uint8 if fp8 else np.uint16).reshape(rows, H),
                  out_scale=_scale_view(wl.quant, es, rows) if fp8 else None)
    part = _sentinel(qrows * H * 2).view(np.uint16).reshape(qrows, H)
    oracle.combine_partial(idx, E, R, y, w, lay["pair_to_row"], rk["token_rank_row"], qrows, out=part)
    res.update(send_x=sx, send_scale=ss, exp_x=ex, exp_scale=es, partial=part, lay=lay, rk=rk)
    return res


def _close(got, ref, S, what):
    g = W.bf16_bits_to_f32(got).astype(np.float64)
    o = W.bf16_bits_to_f32(ref).astype(np.float64)
    bad = np.abs(g - o) > 1e-2 * np.abs(o) + 1e-5 * S
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside the tolerance"
    return int((got != ref).sum())


def _partial_scale(idx, w, y, lay, rk, E, R, used):
    """S per partial element: sum of |w y| over the kept pairs of its (token, rank)."""
    T, K = idx.shape
    L = E // R
    S = np.zeros((used, y.shape[1]), np.float32)
    trr = rk["token_rank_row"].reshape(T, R)
    p2r = lay["pair_to_row"].reshape(T, K)
    for k in range(K):
        e, row = idx[:, k], p2r[:, k]
        m = (e >= 0) & (e < E) & (row >= 0)
        t = np.nonzero(m)[0]
        q = trr[t, e[m] // L]          # distinct for distinct tokens
        S[q] += np.abs(w[m, k][:, None] * W.bf16_bits_to_f32(y[row[m]]))
    return S


def _reduce_scale_of(S, rk, R):
    """Sum over a token's ranks of the partial-sum scales S (rows of S are (token, rank) rows)."""
    trr = rk["token_rank_row"].reshape(-1, R)
    out = np.zeros((trr.shape[0], S.shape[1]), np.float32)
    for r in range(R):
        m = trr[:, r] >= 0
        out[m] += S[trr[m, r]]
    return out


def _reduce_scale(partial, rk, R):
    trr = rk["token_rank_row"].reshape(-1, R)
    S = np.zeros((trr.shape[0], partial.shape[1]), np.float32)
    for r in range(R):
        m = trr[:, r] >= 0
        S[m] += np.abs(W.bf16_bits_to_f32(partial[trr[m, r]]))
    return S


def check(wl, idx, w, x, y, cfg):
    g = run_gpu(wl, idx, x, w, y, cfg)
    o = run_oracle(wl, idx, x, w, y, cfg)
    for k in ("rank_token_count", "rank_token_offset", "token_rank_row", "rank_row_to_token"):
        assert np.array_equal(g[k], o[k]), f"{k} differs"
    assert np.array_equal(g["pair_to_row"], o["lay"]["pair_to_row"]), "pair_to_row differs"
    assert np.array_equal(g["send_x"], o["send_x"]), "send rows differ"
    if o["send_scale"] is not None:
        assert np.array_equal(g["send_scale"], o["send_scale"]), "send scales differ"
    assert np.array_equal(g["exp_x"], o["exp_x"]), "expanded rows differ"
    assert np.array_equal(g["exp_x"], g["dir_x"]), "expanded rows differ from moe_dispatch"
    if o["exp_scale"] is not None:
        assert np.array_equal(g["exp_scale"], o["exp_scale"]), "expanded scales differ"
        assert np.array_equal(g["exp_scale"], g["dir_scale"]), "expanded scales differ from moe_dispatch"
    qrows = g["partial"].shape[0]
    used = int(o["rk"]["rank_token_offset"][-1])
    assert np.all(g["partial"][used:].view(np.uint8) == SENT), "partial rows past the end were written"
    S = _partial_scale(idx, w, y, o["lay"], o["rk"], wl.E, wl.R, used)
    n_part = _close(g["partial"][:used], o["partial"][:used], S, "partial sums")
    ref_out = oracle.combine_reduce(o["partial"], o["rk"]["token_rank_row"], wl.R)
    # S of the reduction: the oracle's partials, plus the partial tolerance they carry
    n_out = _close(g["out"], ref_out, _reduce_scale(o["partial"], o["rk"], wl.R) + _reduce_scale_of(S, o["rk"], wl.R),
                   "reduction")
    print(f"  dedup rows {used} of {qrows}; unequal partial elements {n_part}, unequal outputs {n_out}",
          flush=True)


FULL = ["deepseekv3_prefill_T8192", "deepseekv3_decode_T256", "qwen3moe_decode_T128",
        "skewed_prefill_T16384_masked_fp8", "skewed_prefill_T16384_contig_bf16"]


@pytest.mark.parametrize("name", FULL)
def test_dedup_full_size(name):
    wl = W.WORKLOADS[name].replace(expert_output="random")
    _say(f"dedup full size {name}: T={wl.T} H={wl.H} E={wl.E} K={wl.K} R={wl.R} layout={wl.layout} "
         f"quant={wl.quant}")
    inp = W.make_inputs(wl)
    y = W.expert_outputs(wl, inp)
    check(wl, inp.topk_idx, inp.topk_w, inp.x, y, make_cfg(wl))


SMALL = [
    # name, base workload, overrides
    ("tiny_bf16_R2", "tiny_T64", dict()),
    ("one_expert_per_rank_R32", "tiny_T64", dict(T=200, E=32, R=32, K=8, H=384,
                                                 quant=W.QUANT_FP8_UE8M0, align=4)),
    ("one_rank", "tiny_T64", dict(T=77, E=16, R=1, K=4, H=264)),
    ("single_token_K1", "tiny_T64", dict(T=1, E=8, R=4, K=1, H=128, quant=W.QUANT_FP8_F32)),
    ("K32_R8", "tiny_T64", dict(T=50, E=64, R=8, K=32, H=256, quant=W.QUANT_FP8_F32)),
    ("masked_drops_ue8m0", "deepseekv3_decode_T256", dict(T=300, H=512, capacity=3,
                                                          quant=W.QUANT_FP8_UE8M0)),
    ("mxfp8_contig", "deepseekv3_prefill_T8192", dict(T=500, H=1024, quant=W.QUANT_MXFP8)),
    ("wide_rows_ue8m0", "tiny_T64", dict(T=40, E=16, R=4, K=4, H=32768, quant=W.QUANT_FP8_UE8M0, align=4)),
    ("wide_rows_bf16", "tiny_T64", dict(T=40, E=16, R=4, K=4, H=32768, align=4)),
    ("many_chunks_T140000", "tiny_T64", dict(T=140000, E=64, R=16, K=2, H=64)),
    ("lds_budget_T1100000_R32", "tiny_T64", dict(T=1100000, E=32, R=32, K=1, H=8)),
]


@pytest.mark.parametrize("name,base,kw", SMALL, ids=[s[0] for s in SMALL])
def test_dedup_small(name, base, kw):
    wl = W.WORKLOADS[base].replace(name=name, expert_output="random", **kw)
    _say(f"dedup {name}: T={wl.T} H={wl.H} E={wl.E} K={wl.K} R={wl.R} layout={wl.layout} quant={wl.quant}")
    inp = W.make_inputs(wl)
    y = W.expert_outputs(wl, inp)
    check(wl, inp.topk_idx, inp.topk_w, inp.x, y, make_cfg(wl))


@pytest.mark.parametrize("i", range(16, 24))
def test_dedup_random_configs(i):
    """Seeded random configurations (the generator of the direct-path sweep,
    other seeds): odd rank and expert counts, both layouts, every
    quantization, T below max_tokens."""
    c = random_case(i)
    wl = W.Workload(f"random{i}", T=c["T"], H=c["H"], E=c["E"], K=c["K"], R=c["R"], layout=c["layout"],
                    align=c["align"], capacity=c["capacity"], quant=c["quant"], routing=c["routing"],
                    seed=c["seed"], expert_output="random")
    _say(f"dedup random config {i}: {c}")
    inp = W.make_inputs(wl)
    cfg = make_cfg(wl, T_max=c["T_max"], num_cus=c["num_cus"])
    y = W.expert_outputs(wl, inp, rows=M.moe_rows_capacity(cfg))
    check(wl, inp.topk_idx, inp.topk_w, inp.x, y, cfg)


def test_dedup_edge_routing():
    """Unrouted and invalid ids, one expert repeated, two experts of one rank,
    a token in no rank, and T < max_tokens."""
    wl = W.WORKLOADS["tiny_T64"].replace(name="edge", T=40, E=16, R=4, K=4, H=256,
                                         quant=W.QUANT_FP8_UE8M0, expert_output="random")
    _say("dedup edge routing: -1, invalid ids, repeats, empty tokens, T < max_tokens")
    rng = np.random.default_rng(zlib.crc32(b"dedup-edge"))
    inp = W.make_inputs(wl)
    idx = inp.topk_idx.copy()
    idx[0] = [-1, -1, -1, -1]
    idx[1] = [3, 3, 3, 3]
    idx[2] = [0, 1, 2, 3]            # four experts, one rank
    idx[3] = [16, -5, 4, -1]         # two invalid ids, one valid
    idx[4] = [15, 0, 15, 12]
    idx[rng.random(idx.shape) < 0.05] = -1
    cfg = make_cfg(wl, T_max=64)
    y = W.expert_outputs(wl, inp, rows=M.moe_rows_capacity(cfg))
    check(wl, idx, inp.topk_w, inp.x, y, cfg)


def test_rank_layout_zero_tokens():
    wl = W.WORKLOADS["tiny_T64"].replace(name="zero", E=8, R=4, K=2)
    _say("rank layout with zero tokens")
    cfg = make_cfg(wl, T_max=16)
    rh = M.RankHandle(cfg)
    for t in rh.tensors().values():
        t.fill_(0x5A5A5A5A)
    M.moe_rank_layout(cfg, 0, torch.empty(0, dtype=torch.int32, device="cuda"), rh)
    torch.cuda.synchronize()
    assert rh.rank_token_count.cpu().tolist() == [0] * 4
    assert rh.rank_token_offset.cpu().tolist() == [0] * 5
    assert np.all(rh.rank_row_to_token.cpu().numpy() == -1)
