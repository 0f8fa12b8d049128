"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for every integer and byte output (counts, offsets, both maps,
status, every dispatched bf16 / E4M3 byte, every scale, every row weight) and
for the bytes that must stay untouched: all output buffers start filled with a
0xA5 sentinel on both sides and are compared whole, and 256-byte guard bands
around each device buffer must survive.  Combine is checked against the
tolerance |g - o| <= 1e-2 |o| + 1e-5 S, S = sum_k |w_k y_k| per element (the
fp32 accumulation order is identical on both sides, so the expected result is
exact equality; the count of unequal elements is reported).

Every test prints the case it runs before touching the GPU.
"""
import zlib

import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
import oracle
from combine_topk_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

SENT = 0xA5
GUARD = 256  # bytes


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()  # raises if libmoe_dispatch.so is not built
    oracle._load()


def _say(msg):
    print(f"\n[case] {msg}", flush=True)


class Guarded:
    """A device buffer of `nbytes` inside 0xA5-filled guard bands."""

    def __init__(self, nbytes, dtype, shape):
        nbytes = int(nbytes)
        self.nbytes = nbytes
        self.full = torch.full((nbytes + 2 * GUARD,), SENT, dtype=torch.uint8, device="cuda")
        self.view = self.full[GUARD:GUARD + nbytes].view(dtype).view(shape)

    def host(self):
        b = self.full.cpu().numpy()
        assert np.all(b[:GUARD] == SENT) and np.all(b[GUARD + self.nbytes:] == SENT), \
            "write outside the buffer (guard band changed)"
        return b[GUARD:GUARD + self.nbytes]


def _sentinel(nbytes):
    return np.full(int(nbytes), SENT, np.uint8)


def make_cfg(wl, T_max=None, num_cus=0):
    return M.MoeConfig(max_tokens=wl.T if T_max is None else T_max, hidden=wl.H,
                       num_experts=wl.E, num_topk=wl.K, num_ranks=wl.R, layout=wl.layout,
                       align=wl.align, capacity=wl.capacity, quant=wl.quant, num_cus=num_cus)


def scale_cols(wl):
    """32-bit words of scales per dispatched row."""
    nb = wl.H // 128
    return {W.QUANT_NONE: 0, W.QUANT_FP8_F32: nb, W.QUANT_FP8_UE8M0: (nb + 3) // 4,
            W.QUANT_MXFP8: nb}[wl.quant]


def scale_guard(wl, rows):
    """A guarded device scale buffer in the element type the binding expects."""
    if wl.quant == W.QUANT_MXFP8:
        return Guarded(rows * wl.H // 32, torch.uint8, (rows, wl.H // 32))
    nsc = scale_cols(wl)
    return Guarded(rows * nsc * 4, torch.int32, (rows, nsc))


def oracle_scale_view(quant, buf, rows):
    """The oracle's view of a scale buffer: fp32, packed UE8M0 words or MX bytes."""
    if quant == W.QUANT_FP8_F32:
        return buf.view(np.float32).reshape(rows, -1)
    if quant == W.QUANT_FP8_UE8M0:
        return buf.view(np.uint32).reshape(rows, -1)
    if quant == W.QUANT_MXFP8:
        return buf.view(np.uint8).reshape(rows, -1)
    return None


def run_gpu(wl, idx, w, x, y, cfg, fused=False):
    """One layout + dispatch + combine through the ABI (layout and dispatch as
    two calls, or as the one fused call); returns host arrays."""
    T, K, E, R, H = idx.shape[0], wl.K, wl.E, wl.R, wl.H
    rows = M.moe_rows_capacity(cfg)
    handle = M.Handle.__new__(M.Handle)
    bufs = {}
    for name, n in (("expert_count", E), ("recv_count", E), ("expert_offset", E + 1),
                    ("rank_offset", R + 1), ("pair_to_row", cfg.max_tokens * K),
                    ("row_to_pair", rows), ("status", 2)):
        g = Guarded(4 * n, torch.int32, (n,))
        bufs[name] = g
        setattr(handle, name, g.view)
    handle.c = M.MoeHandle(*(bufs[n].view.data_ptr() for n, _ in M.MoeHandle._fields_))
    ws = torch.empty(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    fp8 = wl.quant != W.QUANT_NONE
    ebytes = 1 if fp8 else 2
    out_x = Guarded(rows * H * ebytes, torch.uint8 if fp8 else torch.int16, (rows, H))
    nsc = scale_cols(wl)
    out_scale = scale_guard(wl, rows) if fp8 else None
    out_rw = Guarded(rows * 4, torch.float32, (rows,))
    out = Guarded(T * H * 2, torch.int16, (T, H))
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    d_w = torch.from_numpy(np.ascontiguousarray(w, np.float32)).cuda()
    d_x = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    d_y = torch.from_numpy(np.ascontiguousarray(y).view(np.int16)).cuda()
    if fused:
        M.moe_dispatch_fused(cfg, T, d_idx, d_x, d_w, handle, ws, out_x.view,
                             out_scale.view if fp8 else None, out_rw.view)
    else:
        M.moe_dispatch_layout(cfg, T, d_idx, handle, ws)
        M.moe_dispatch(cfg, T, d_x, d_w, handle, out_x.view,
                       out_scale.view if fp8 else None, out_rw.view)
    M.moe_combine(cfg, T, d_y, d_w, handle, out.view)
    torch.cuda.synchronize()
    res = {n: g.host().view(np.int32) for n, g in bufs.items()}
    res["out_x"] = out_x.host()
    res["out_scale"] = out_scale.host() if fp8 else None
    res["out_row_weight"] = out_rw.host()
    res["out"] = out.host().view(np.uint16).reshape(T, H)
    return res


def run_oracle(wl, idx, w, x, y, cfg):
    T, K, E, R, H = idx.shape[0], wl.K, wl.E, wl.R, wl.H
    rows = M.moe_rows_capacity(cfg)
    h = oracle.dispatch_layout(idx, E, R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    res = {}
    for name, n in (("expert_count", E), ("recv_count", E), ("expert_offset", E + 1),
                    ("rank_offset", R + 1), ("pair_to_row", cfg.max_tokens * K),
                    ("row_to_pair", rows), ("status", 2)):
        a = _sentinel(4 * n).view(np.int32)
        a[:h[name].size] = h[name]
        res[name] = a
    fp8 = wl.quant != W.QUANT_NONE
    ox = _sentinel(rows * H * (1 if fp8 else 2))
    nsc = scale_cols(wl)
    osc = _sentinel(rows * nsc * 4) if fp8 else None
    orw = _sentinel(rows * 4)
    out_x = ox.view(np.uint8 if fp8 else np.uint16).reshape(rows, H)
    out_scale = oracle_scale_view(wl.quant, osc, rows) if fp8 else None
    oracle.dispatch(x, h["pair_to_row"], K, wl.quant, rows, topk_w=w, out_x=out_x,
                    out_scale=out_scale, out_row_weight=orw.view(np.float32))
    res["out_x"] = ox
    res["out_scale"] = osc
    res["out_row_weight"] = orw
    res["out"] = oracle.combine(y, w, h["pair_to_row"]) if T > 0 else np.zeros((0, H), np.uint16)
    return res


def assert_combine_close(g, o, y, w, p2r, K):
    """Q20 tolerance, evaluated where the bf16 results differ."""
    diff = np.nonzero(g.reshape(-1) != o.reshape(-1))[0]
    if diff.size == 0:
        return 0
    T, H = o.shape
    t, j = diff // H, diff % H
    gf = W.bf16_bits_to_f32(g.reshape(-1)[diff]).astype(np.float64)
    of = W.bf16_bits_to_f32(o.reshape(-1)[diff]).astype(np.float64)
    S = np.zeros(diff.size)
    for k in range(K):
        r = p2r.reshape(T, K)[t, k]
        ok = r >= 0
        yv = W.bf16_bits_to_f32(y[r[ok], j[ok]]).astype(np.float64)
        S[ok] += np.abs(w[t[ok], k].astype(np.float64) * yv)
    bad = np.abs(gf - of) > 1e-2 * np.abs(of) + 1e-5 * S
    assert not bad.any(), f"{int(bad.sum())} combine elements outside tolerance"
    return int(diff.size)


def check_parity(wl, idx, w, x, y, cfg, label, fused=False):
    label = f"{label} [{'fused' if fused else 'separate'}]"
    g = run_gpu(wl, idx, w, x, y, cfg, fused)
    o = run_oracle(wl, idx, w, x, y, cfg)
    for name in ("expert_count", "recv_count", "expert_offset", "rank_offset", "status",
                 "pair_to_row", "row_to_pair"):
        if not np.array_equal(g[name], o[name]):
            bad = np.nonzero(g[name] != o[name])[0]
            raise AssertionError(f"{label}: {name} differs at {bad[:8]}: gpu {g[name][bad[:8]]} "
                                 f"oracle {o[name][bad[:8]]}")
    for name in ("out_x", "out_scale", "out_row_weight"):
        if g[name] is None:
            continue
        if not np.array_equal(g[name], o[name]):
            bad = np.nonzero(g[name] != o[name])[0]
            raise AssertionError(f"{label}: {name} differs at {bad.size} bytes, first {bad[:8]}: "
                                 f"gpu {g[name][bad[:8]]} oracle {o[name][bad[:8]]}")
    n_ne = assert_combine_close(g["out"], o["out"], y, w, o["pair_to_row"], wl.K)
    print(f"[ok] {label}: layout/dispatch bit-exact, combine unequal elements {n_ne}", flush=True)
    return g, o


def inputs_for(wl, row_to_pair=None):
    inp = W.make_inputs(wl)
    if wl.expert_output == "scaled":
        h = oracle.dispatch_layout(inp.topk_idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity)
        y = W.expert_outputs(wl, inp, h["row_to_pair"])
    else:
        y = W.expert_outputs(wl, inp)
    return inp.topk_idx, inp.topk_w, inp.x, y


# ---- every workload at its full size, in the launch configuration the benchmark times

MODES = [False, True]
MODE_IDS = ["separate", "fused"]


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size(name, fused):
    wl = W.WORKLOADS[name]
    _say(f"full-size workload {name} fused={fused}")
    idx, w, x, y = inputs_for(wl)
    cfg = make_cfg(wl)
    g, o = check_parity(wl, idx, w, x, y, cfg, name, fused)
    if wl.layout == W.LAYOUT_MASKED:
        print(f"[info] {name}: dropped pairs {int(g['status'][0])}", flush=True)
    # determinism: a second run is bitwise identical
    g2 = run_gpu(wl, idx, w, x, y, cfg, fused)
    for k in g:
        if g[k] is not None:
            assert np.array_equal(g[k], g2[k]), f"{name}: {k} not deterministic"


# ---- scaled expert outputs at full size: oracle parity plus a closed form

@pytest.mark.parametrize("name", ["deepseekv3_prefill_T8192", "deepseekv3_decode_T256", "qwen3moe_decode_T128"])
def test_scaled_experts_full_size(name):
    """Expert e returns bf16((e + 1) / 2 * x): combine must match the oracle
    and, independently of it, the closed form x * sum over kept pairs of
    w_k (e_k + 1) / 2 evaluated in float64.  All terms of a token share the
    sign of x, so the relative error is at most the two bf16 roundings (y and
    the output, 2^-8 each) plus the fp32 accumulation: 2^-7 + 2^-12 covers it."""
    wl = W.WORKLOADS[name].replace(expert_output="scaled")
    _say(f"full-size workload {name} with scaled expert outputs (fused)")
    idx, w, x, y = inputs_for(wl)
    cfg = make_cfg(wl)
    g, o = check_parity(wl, idx, w, x, y, cfg, name + " scaled experts", fused=True)
    T, K = idx.shape
    p2r = o["pair_to_row"][:T * K].reshape(T, K)
    kept = p2r >= 0
    factor = np.where(kept, w.astype(np.float64) * (idx.astype(np.float64) + 1.0) * 0.5, 0.0).sum(axis=1)
    ref = W.bf16_bits_to_f32(x).astype(np.float64) * factor[:, None]
    got = W.bf16_bits_to_f32(g["out"]).astype(np.float64)
    err = np.abs(got - ref)
    tol = (2.0 ** -7 + 2.0 ** -12) * np.abs(ref)
    assert np.all(err <= tol), f"{int((err > tol).sum())} elements off the closed form"
    print(f"[ok] {name}: closed form, max relative error "
          f"{float(np.max(err / np.maximum(np.abs(ref), 1e-300))):.3e}", flush=True)


# ---- small cases spanning several tiles and ragged tails

SMALL = [
    # T, H, E, K, R, layout, align, capacity, quant
    (37, 384, 24, 6, 4, W.LAYOUT_CONTIGUOUS, 16, 1, W.QUANT_FP8_UE8M0),
    (37, 384, 24, 6, 4, W.LAYOUT_CONTIGUOUS, 16, 1, W.QUANT_FP8_F32),
    (37, 384, 24, 6, 4, W.LAYOUT_CONTIGUOUS, 16, 1, W.QUANT_MXFP8),
    (300, 640, 40, 7, 8, W.LAYOUT_MASKED, 1, 33, W.QUANT_MXFP8),         # MX, overflow
    (2000, 128, 96, 32, 8, W.LAYOUT_CONTIGUOUS, 8, 1, W.QUANT_MXFP8),    # MX, K = 32, one group
    (300, 640, 40, 7, 8, W.LAYOUT_CONTIGUOUS, 3, 1, W.QUANT_FP8_UE8M0),   # 5 blocks: partial word
    (300, 1152, 40, 7, 5, W.LAYOUT_MASKED, 1, 33, W.QUANT_FP8_F32),       # overflow
    (513, 72, 17, 3, 17, W.LAYOUT_CONTIGUOUS, 5, 1, W.QUANT_NONE),        # H % 512 ragged
    (513, 1032, 64, 5, 2, W.LAYOUT_MASKED, 1, 20, W.QUANT_NONE),
    (2000, 256, 96, 32, 8, W.LAYOUT_CONTIGUOUS, 8, 1, W.QUANT_FP8_F32),   # K = 32
    (4100, 128, 8, 1, 1, W.LAYOUT_MASKED, 1, 700, W.QUANT_FP8_UE8M0),     # K = 1, H = 128
    (2048, 264, 64, 32, 8, W.LAYOUT_CONTIGUOUS, 4, 1, W.QUANT_NONE),     # fused: half the CUs, K = 32
    (3000, 384, 96, 8, 8, W.LAYOUT_MASKED, 1, 200, W.QUANT_FP8_F32),      # fused: half the CUs, overflow
    (2600, 640, 64, 6, 4, W.LAYOUT_CONTIGUOUS, 32, 1, W.QUANT_MXFP8),     # fused: 7/16 of the CUs
    (2048, 16384, 32, 4, 4, W.LAYOUT_CONTIGUOUS, 8, 1, W.QUANT_FP8_UE8M0),  # token runs, two-iteration items
    (2100, 16384, 40, 3, 5, W.LAYOUT_MASKED, 1, 120, W.QUANT_MXFP8),     # token runs, MX, overflow
    (8200, 8448, 64, 7, 8, W.LAYOUT_CONTIGUOUS, 16, 1, W.QUANT_FP8_UE8M0),  # x > 128 MiB: every CU, ragged row
    (9000, 512, 256, 8, 8, W.LAYOUT_CONTIGUOUS, 128, 1, W.QUANT_FP8_UE8M0),  # > 64 layout chunks
    (1, 2048, 128, 8, 8, W.LAYOUT_MASKED, 1, 128, W.QUANT_FP8_F32),       # T = 1
    (64, 8, 4, 4, 4, W.LAYOUT_CONTIGUOUS, 1, 1, W.QUANT_NONE),            # H = 8, E = R
    (3000, 128, 600, 4, 8, W.LAYOUT_CONTIGUOUS, 2, 1, W.QUANT_FP8_UE8M0),  # E > 512: 8-wave layout blocks
    (5000, 256, 2048, 6, 16, W.LAYOUT_MASKED, 1, 3, W.QUANT_FP8_F32),     # E = 2048: 4-wave blocks
    (140000, 8, 64, 8, 8, W.LAYOUT_CONTIGUOUS, 4, 1, W.QUANT_NONE),       # > 1M pairs: multi-tile waves
    (64, 32768, 16, 4, 4, W.LAYOUT_CONTIGUOUS, 4, 1, W.QUANT_FP8_UE8M0),  # wide rows: multi-iteration items
    (64, 32768, 16, 4, 4, W.LAYOUT_CONTIGUOUS, 4, 1, W.QUANT_NONE),
    (48, 32768, 16, 4, 4, W.LAYOUT_MASKED, 1, 9, W.QUANT_MXFP8),
    (33, 20480, 16, 6, 2, W.LAYOUT_MASKED, 1, 20, W.QUANT_FP8_F32),       # 160 blocks: 40 UE8M0-size words
]


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_H{c[1]}_E{c[2]}_K{c[3]}_L{c[5]}_Q{c[8]}"
                                             for c in SMALL])
def test_small_ragged(case, fused):
    T, H, E, K, R, layout, align, cap, quant = case
    _say(f"small {case} fused={fused}")
    wl = W.Workload("small", T=T, H=H, E=E, K=K, R=R, layout=layout, align=align,
                    capacity=cap, quant=quant, routing="softmax", seed=1000 + T)
    idx, w, x, y = inputs_for(wl)
    check_parity(wl, idx, w, x, y, make_cfg(wl), f"small {case}", fused)


# ---- seeded random configurations: every layout and quantization, odd expert
# and rank counts, T below max_tokens, forced compute-unit counts (the fused
# call's block count), with sizes kept small enough for the oracle

def random_case(i):
    rng = np.random.default_rng(9100 + i)
    R = int(rng.choice([1, 2, 3, 4, 8, 16]))
    E = R * int(rng.integers(1, 48))
    K = int(rng.integers(1, min(16, E) + 1))
    quant = int(rng.choice([W.QUANT_NONE, W.QUANT_FP8_F32, W.QUANT_FP8_UE8M0, W.QUANT_MXFP8]))
    H = 128 * int(rng.integers(1, 9)) if quant != W.QUANT_NONE else 8 * int(rng.integers(1, 129))
    layout = int(rng.choice([W.LAYOUT_CONTIGUOUS, W.LAYOUT_MASKED]))
    align = int(rng.choice([1, 2, 7, 32, 128]))
    if E * align > 20000:
        align = 7
    T = int(rng.integers(1, 1500))
    capacity = int(rng.integers(1, T * K // E + 9))
    routing = "zipf" if rng.random() < 0.3 else "softmax"
    return dict(T=T, H=H, E=E, K=K, R=R, layout=layout, align=align, capacity=capacity, quant=quant,
                routing=routing, T_max=T + int(rng.integers(0, 100)),
                num_cus=int(rng.choice([0, 1, 5, 64, 256])), seed=9100 + i)


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("i", range(16))
def test_random_configs(i, fused):
    c = random_case(i)
    _say(f"random config {i}: {c} fused={fused}")
    wl = W.Workload(f"random{i}", T=c["T"], H=c["H"], E=c["E"], K=c["K"], R=c["R"], layout=c["layout"],
                    align=c["align"], capacity=c["capacity"], quant=c["quant"], routing=c["routing"],
                    seed=c["seed"])
    cfg = make_cfg(wl, T_max=c["T_max"], num_cus=c["num_cus"])
    inp = W.make_inputs(wl)
    y = W.expert_outputs(wl, inp, rows=M.moe_rows_capacity(cfg))  # rows for max_tokens, not T
    check_parity(wl, inp.topk_idx, inp.topk_w, inp.x, y, cfg, f"random config {i}", fused)


def _edge_inputs(kind, T, H, E, K, rng):
    if kind == "one_expert":
        idx = np.zeros((T, K), np.int32)
        idx[:, 1:] = -1
    elif kind == "invalid_and_unrouted":
        idx = rng.integers(0, E, (T, K)).astype(np.int32)
        m = rng.random((T, K))
        idx[m < 0.2] = -1
        idx[(m >= 0.2) & (m < 0.3)] = E + 5
        idx[(m >= 0.3) & (m < 0.35)] = -7
        idx[7] = -1
    elif kind == "duplicates":
        idx = rng.integers(0, 3, (T, K)).astype(np.int32)
    else:
        raise ValueError(kind)
    w = rng.standard_normal((T, K)).astype(np.float32)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[0] *= 1e-39          # bf16 subnormals
    xf[1, :128] = 0.0       # zero block
    xf[2, :128] = -0.0      # negative zero block
    xf[3] *= 3e-11          # block maxima around the amax floor
    xf[4] *= 1e30
    return idx, w, W.f32_to_bf16_bits(xf)


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
@pytest.mark.parametrize("kind", ["one_expert", "invalid_and_unrouted", "duplicates"])
@pytest.mark.parametrize("layout,quant", [(W.LAYOUT_CONTIGUOUS, W.QUANT_FP8_UE8M0),
                                          (W.LAYOUT_MASKED, W.QUANT_FP8_F32),
                                          (W.LAYOUT_MASKED, W.QUANT_MXFP8),
                                          (W.LAYOUT_MASKED, W.QUANT_NONE)])
def test_edge_routing(kind, layout, quant, fused):
    T, H, E, K, R = 200, 256, 12, 4, 3
    _say(f"edge {kind} layout {layout} quant {quant} fused={fused}")
    rng = np.random.default_rng(zlib.crc32(f"{kind}/{layout}/{quant}".encode()))
    wl = W.Workload("edge", T=T, H=H, E=E, K=K, R=R, layout=layout, align=4, capacity=9,
                    quant=quant)
    idx, w, x = _edge_inputs(kind, T, H, E, K, rng)
    y = W.f32_to_bf16_bits(rng.standard_normal((wl.rows_capacity, H)).astype(np.float32))
    g, o = check_parity(wl, idx, w, x, y, make_cfg(wl), f"edge {kind}", fused)
    if kind == "invalid_and_unrouted":
        assert g["status"][1] > 0


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
def test_capacity_one_masked(fused):
    T, H, E, K, R = 100, 128, 8, 2, 8
    _say(f"masked capacity 1 fused={fused}")
    wl = W.Workload("cap1", T=T, H=H, E=E, K=K, R=R, layout=W.LAYOUT_MASKED, capacity=1,
                    quant=W.QUANT_FP8_UE8M0, seed=7)
    idx, w, x, y = inputs_for(wl)
    g, _ = check_parity(wl, idx, w, x, y, make_cfg(wl), "masked capacity 1", fused)
    assert g["status"][0] == T * K - E


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
def test_fewer_tokens_than_max_and_num_cus(fused):
    """A call with num_tokens < max_tokens, and a restricted compute-unit budget."""
    wl = W.WORKLOADS["deepseekv3_decode_T256"].replace(T=200)
    _say(f"T=200 of max 256, num_cus=7 fused={fused}")
    idx, w, x, y = inputs_for(wl.replace(T=200))
    cfg = make_cfg(wl, T_max=256, num_cus=7)
    check_parity(wl, idx, w, x, y, cfg, "T<max, num_cus=7", fused)


@pytest.mark.parametrize("T", [2048, 2049])
def test_combine_load_policy_boundary(T):
    """Combines reading at most 64 MiB of expert rows (T*K*H*2) use cache-
    allocating loads, larger ones non-temporal loads: both sides of the switch
    (exactly 64 MiB and one token more) against the oracle."""
    wl = W.WORKLOADS["qwen3moe_decode_T128"].replace(T=T, layout=W.LAYOUT_CONTIGUOUS, align=16,
                                                     quant=W.QUANT_NONE)
    assert wl.K * wl.H * 2 * 2048 == 64 << 20
    _say(f"combine load-policy boundary T={T} H={wl.H} K={wl.K}")
    idx, w, x, y = inputs_for(wl)
    check_parity(wl, idx, w, x, y, make_cfg(wl), f"load-policy boundary T={T}")


def test_fused_unaligned_ids():
    """topk_idx that is only 4-byte aligned takes the scalar histogram path."""
    wl = W.Workload("unaligned", T=300, H=512, E=32, K=4, R=4, layout=W.LAYOUT_CONTIGUOUS,
                    align=8, quant=W.QUANT_FP8_UE8M0, seed=31)
    _say("fused call with topk_idx at a 4-byte offset")
    idx, w, x, y = inputs_for(wl)
    cfg = make_cfg(wl)
    T, K = idx.shape
    rows = M.moe_rows_capacity(cfg)
    base = torch.full((T * K + 4,), -1, dtype=torch.int32, device="cuda")
    base[1:1 + T * K] = torch.from_numpy(idx.reshape(-1)).cuda()
    d_idx = base[1:1 + T * K]
    assert d_idx.data_ptr() % 16 != 0
    b = M.DispatchBuffers(cfg, device="cuda")
    d_x = torch.from_numpy(x.view(np.int16)).cuda()
    M.moe_dispatch_fused(cfg, T, d_idx, d_x, None, b.handle, b.workspace, b.out_x, b.out_scale)
    torch.cuda.synchronize()
    h = oracle.dispatch_layout(idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    for k, v in b.handle.tensors().items():
        assert np.array_equal(v.cpu().numpy()[:h[k].size], h[k]), k
    ox, osc, _ = oracle.dispatch(x, h["pair_to_row"], K, wl.quant, rows)
    kept = h["pair_to_row"][h["pair_to_row"] >= 0]
    assert np.array_equal(b.out_x.cpu().numpy()[kept], ox[kept])
    assert np.array_equal(b.out_scale.cpu().numpy().view(np.uint32)[kept], osc[kept])


@pytest.mark.parametrize("fused", MODES, ids=MODE_IDS)
def test_zero_tokens_layout(fused):
    wl = W.Workload("empty", T=0, H=256, E=16, K=4, R=4, layout=W.LAYOUT_CONTIGUOUS, align=8)
    _say(f"zero tokens fused={fused}")
    cfg = make_cfg(wl, T_max=50)
    idx = np.zeros((0, 4), np.int32)
    w = np.zeros((0, 4), np.float32)
    x = np.zeros((0, 256), np.uint16)
    y = np.zeros((M.moe_rows_capacity(cfg), 256), np.uint16)
    g, _ = check_parity(wl, idx, w, x, y, cfg, "zero tokens", fused)
    assert np.all(g["row_to_pair"] == -1) and not g["expert_offset"].any()


def test_quant_sweep_all_bf16_magnitudes():
    """Every bf16 value with |x| <= 448 goes through the E4M3 conversion with
    scale exactly 1 (UE8M0 k = 0 and fp32 s = 1): block element 0 is 448, the
    other 127 carry the sweep.  Blocks whose maximum is 448 * 2^j sweep the
    same values scaled by powers of two (exact ties included)."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(b)
    vals = f[np.isfinite(f) & (np.abs(f) <= 448)]
    per = 127
    nblk = -(-vals.size // per)
    pad = np.zeros(nblk * per, np.float32)
    pad[:vals.size] = vals
    blocks = np.concatenate([np.full((nblk, 1), 448.0, np.float32), pad.reshape(nblk, per)], 1)
    scaled = [blocks * np.float32(2.0 ** j) for j in (0, -3, 5)]
    allb = np.concatenate(scaled).reshape(-1)
    H = 7168
    T = -(-allb.size // H)
    xf = np.zeros(T * H, np.float32)
    xf[:allb.size] = allb
    x = W.f32_to_bf16_bits(xf.reshape(T, H))
    rng = np.random.default_rng(77)
    for quant in (W.QUANT_FP8_UE8M0, W.QUANT_FP8_F32, W.QUANT_MXFP8):
        _say(f"bf16 magnitude sweep quant {quant} T={T}")
        wl = W.Workload("sweep", T=T, H=H, E=4, K=2, R=2, layout=W.LAYOUT_CONTIGUOUS,
                        align=1, quant=quant)
        idx = np.stack([np.arange(T) % 4, (np.arange(T) + 1) % 4], 1).astype(np.int32)
        w = np.full((T, 2), 0.5, np.float32)
        y = W.f32_to_bf16_bits(rng.standard_normal((wl.rows_capacity, H)).astype(np.float32))
        check_parity(wl, idx, w, x, y, make_cfg(wl), f"sweep quant {quant}", fused=True)


def test_determinism_ten_runs():
    """Ten runs of the headline step (fused dispatch + combine) leave every
    output bitwise identical, compared on the device."""
    wl = W.WORKLOADS[W.HEADLINE]
    _say(f"determinism over 10 runs: {wl.name}")
    inp = W.make_inputs(wl)
    y = W.expert_outputs(wl, inp)
    cfg = make_cfg(wl)
    bufs = M.DispatchBuffers(cfg, row_weight=True)
    d_idx = torch.from_numpy(inp.topk_idx).cuda()
    d_w = torch.from_numpy(inp.topk_w).cuda()
    d_x = torch.from_numpy(inp.x.view(np.int16)).cuda()
    d_y = torch.from_numpy(y.view(np.int16)).cuda()
    out = torch.empty((wl.T, wl.H), dtype=torch.int16, device="cuda")
    first = None
    for run in range(10):
        for t in (bufs.out_x, bufs.out_scale, bufs.out_row_weight, out):
            t.view(torch.uint8).fill_(SENT)
        M.moe_dispatch_fused(cfg, wl.T, d_idx, d_x, d_w, bufs.handle, bufs.workspace, bufs.out_x,
                             bufs.out_scale, bufs.out_row_weight)
        M.moe_combine(cfg, wl.T, d_y, d_w, bufs.handle, out)
        snap = [t.clone() for t in list(bufs.handle.tensors().values()) +
                [bufs.out_x, bufs.out_scale, bufs.out_row_weight, out]]
        torch.cuda.synchronize()
        if first is None:
            first = snap
        else:
            for a, b in zip(first, snap):
                assert torch.equal(a, b), f"run {run} differs from run 0"


def test_fp32_scale_sweep_non_power_of_two():
    """The fp32-scale path with scales that are not powers of two: every
    bf16 value up to 448 c in blocks whose maximum is 448 c, so x / s lands on
    fp32 values with mantissa bits beyond bf16, near E4M3 rounding ties
    included; the hardware conversion must match the oracle's encoder."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = W.bf16_bits_to_f32(b)
    rng = np.random.default_rng(78)
    H = 7168
    blocks = []
    for c in (1.1, 1.37, 1.5, 1.9921875, 3.0, 0.7, 1e-3, 1e5):
        amax = np.float32(448.0 * c)
        amax_bf = W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([amax], np.float32)))[0]
        vals = f[np.isfinite(f) & (np.abs(f) <= amax_bf)]
        per = 127
        nblk = -(-vals.size // per)
        pad = np.zeros(nblk * per, np.float32)
        pad[:vals.size] = rng.permutation(vals)
        blocks.append(np.concatenate([np.full((nblk, 1), amax_bf, np.float32), pad.reshape(nblk, per)], 1))
    allb = np.concatenate(blocks).reshape(-1)
    T = -(-allb.size // H)
    xf = np.zeros(T * H, np.float32)
    xf[:allb.size] = allb
    x = W.f32_to_bf16_bits(xf.reshape(T, H))
    _say(f"fp32-scale sweep with non-power-of-two scales, T={T}")
    wl = W.Workload("sweep_f32", T=T, H=H, E=4, K=2, R=2, layout=W.LAYOUT_CONTIGUOUS, align=1,
                    quant=W.QUANT_FP8_F32)
    idx = np.stack([np.arange(T) % 4, (np.arange(T) + 1) % 4], 1).astype(np.int32)
    w = np.full((T, 2), 0.5, np.float32)
    y = W.f32_to_bf16_bits(rng.standard_normal((wl.rows_capacity, H)).astype(np.float32))
    check_parity(wl, idx, w, x, y, make_cfg(wl), "fp32-scale sweep", fused=False)
