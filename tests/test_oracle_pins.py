"""Pins for the CPU oracle (no GPU needed).

The oracle is checked against things other than itself: hand-worked fixtures
(tests/golden/), library routines (torch's float8/bfloat16 casts, numpy's
stable argsort and bincount), independent formulations (value-domain nearest
search, exponent-bit shortcuts), brute force on tiny inputs, closed forms and
invariants.  Each check is chosen so that a plausible slip in the oracle (a
wrong tie rule, a dropped sign, an off-by-one in a slot or offset, a transposed
index) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _f32(bits):
    return W.bf16_bits_to_f32(bits)


# ----------------------------------------------------------------------------
# Codecs
# ----------------------------------------------------------------------------

def _torch_e4m3(v):
    """torch's float8_e4m3fn cast (round to nearest even), as bytes."""
    t = torch.from_numpy(np.ascontiguousarray(v, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_e4m3_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


_CODE_VALUES = _torch_e4m3_decode(np.arange(0x7F, dtype=np.uint8))  # 0x00..0x7E


def _nearest_e4m3(v):
    """Independent value-domain encoder: nearest of the 127 finite magnitudes,
    ties to the even code, sign copied from the input."""
    v = np.asarray(v, np.float32)
    a = np.abs(v.astype(np.float64))
    c = np.searchsorted(_CODE_VALUES, a, side="right") - 1
    c = np.clip(c, 0, 0x7E)
    up = np.minimum(c + 1, 0x7E)
    dlo = a - _CODE_VALUES[c]
    dhi = _CODE_VALUES[up] - a
    take_up = (up != c) & ((dhi < dlo) | ((dhi == dlo) & (c % 2 == 1)))
    code = np.where(take_up, up, c).astype(np.uint8)
    return code | np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))


def _e4m3_sweep_inputs():
    rng = np.random.default_rng(11)
    parts = []
    # every bf16 pattern with finite magnitude <= 448
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = _f32(b)
    parts.append(f[np.isfinite(f) & (np.abs(f) <= 448)])
    # structured fp32 sweep: every exponent up to 2^8, every top-12 mantissa
    # pattern, and low-bit patterns around the rounding point (exact ties
    # included), both signs
    exps = np.arange(0, 136, dtype=np.uint32)
    top = np.arange(1 << 12, dtype=np.uint32) << 11
    low = np.array([0, 1, 0x3FF, 0x400, 0x401, 0x7FF], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | top[None, :, None] | low[None, None, :]
    bits = bits.reshape(-1)
    s = np.concatenate([bits, bits | np.uint32(0x80000000)])
    f = s.view(np.float32)
    parts.append(f[np.abs(f) <= 448])
    # random values, uniform and log-uniform magnitudes
    parts.append(rng.uniform(-448, 448, 1 << 20).astype(np.float32))
    mag = np.exp2(rng.uniform(-30, np.log2(448.0), 1 << 20)).astype(np.float32)
    mag = np.minimum(mag, np.float32(448))
    parts.append(mag * rng.choice(np.array([-1, 1], np.float32), mag.size))
    return np.concatenate(parts)


def test_e4m3_golden_ocp_values(oracle_lib):
    g = _golden("e4m3_ocp_values.json")
    vals = np.array([c["value"] for c in g["cases"]], np.float32)
    want = np.array([int(c["code"], 16) for c in g["cases"]], np.uint8)
    got = oracle.e4m3_encode(vals)
    bad = [(c["value"], c["code"], hex(x)) for c, x, w in zip(g["cases"], got, want) if x != w]
    assert not bad, bad


def test_e4m3_roundtrip_all_finite_codes(oracle_lib):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = _torch_e4m3_decode(codes).astype(np.float32)
    # -0 decodes to -0.0 and must come back as 0x80
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    # the oracle's own decode of the positive codes agrees with torch's
    ours = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    assert np.array_equal(ours, _CODE_VALUES)


def test_e4m3_sweep_vs_torch_and_nearest(oracle_lib):
    v = _e4m3_sweep_inputs()
    got = oracle.e4m3_encode(v)
    ref_t = _torch_e4m3(v)
    ref_n = _nearest_e4m3(v)
    assert np.array_equal(ref_t, ref_n)  # the two references agree
    mism = np.nonzero(got != ref_t)[0]
    assert mism.size == 0, [(float(v[i]), hex(got[i]), hex(ref_t[i])) for i in mism[:10]]


def test_bf16_rne_vs_torch(oracle_lib):
    rng = np.random.default_rng(12)
    exps = np.arange(0, 255, dtype=np.uint32)
    hi = np.arange(1 << 7, dtype=np.uint32) << 16
    low = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = ((exps[:, None, None] << 23) | hi[None, :, None] | low[None, None, :]).reshape(-1)
    rnd = rng.integers(0, 1 << 32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    rnd = rnd[(rnd & 0x7F800000) != 0x7F800000]
    bits = np.concatenate([bits, bits | np.uint32(0x80000000), rnd])
    f = bits.view(np.float32)
    got = oracle.bf16_rne(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    mism = np.nonzero(got != ref)[0]
    assert mism.size == 0, [(hex(bits[i]), hex(got[i]), hex(ref[i])) for i in mism[:10]]


def test_ue8m0_exponent_exhaustive_over_bf16(oracle_lib):
    b = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)  # positive finite bf16
    a = np.maximum(_f32(b), np.float32(1e-10))
    a = np.concatenate([a, np.array([1e-10, 448, 448 * 2.0 ** -42], np.float32)])
    k = oracle.ue8m0_exponent(a)
    # independent shortcut from the binary32 fields of a (always normal here):
    # a = m * 2^e with m in [1,2); 448 = 1.75 * 2^8, so k = e - 8 when m <= 1.75
    # and e - 7 otherwise.
    bits = a.view(np.uint32)
    e = ((bits >> 23) & 0xFF).astype(np.int64) - 127
    m = bits & 0x7FFFFF
    k_short = e - 8 + (m > 0x600000)
    assert np.array_equal(k, k_short)
    # defining inequality, evaluated in float64 (exact)
    ad = a.astype(np.float64)
    assert np.all(ad <= np.ldexp(448.0, k)) and np.all(ad > np.ldexp(448.0, k - 1))
    # the stored byte k + 127 decodes (torch float8_e8m0fnu) to the scale 2^k
    byte = torch.from_numpy((k + 127).astype(np.uint8)).view(torch.float8_e8m0fnu)
    assert np.array_equal(byte.to(torch.float64).numpy(), np.ldexp(1.0, k))


# ----------------------------------------------------------------------------
# Layout
# ----------------------------------------------------------------------------

LAYOUT_KEYS = ("expert_count", "recv_count", "expert_offset", "rank_offset",
               "pair_to_row", "row_to_pair", "status")


@pytest.mark.parametrize("name", ["layout_contiguous_T4_E4_K2_A2.json",
                                  "layout_masked_T4_E4_K2_C2.json"])
def test_layout_golden(oracle_lib, name):
    g = _golden(name)
    lay = oracle.CONTIGUOUS if g["layout"] == "contiguous" else oracle.MASKED
    h = oracle.dispatch_layout(np.array(g["topk_idx"], np.int32), g["E"], g["R"], lay,
                               g["align"], g["capacity"])
    for k in LAYOUT_KEYS:
        assert h[k].tolist() == g["expected"][k], k


def test_dispatch_combine_golden_bf16(oracle_lib):
    g = _golden("layout_contiguous_T4_E4_K2_A2.json")
    ex = g["expected"]
    idx = np.array(g["topk_idx"], np.int32)
    h = oracle.dispatch_layout(idx, g["E"], g["R"], oracle.CONTIGUOUS, g["align"])
    x = _bf16(g["x"])
    rows = len(ex["row_to_pair"])
    sentinel = np.uint16(0xA5A5)
    out_x = np.full((rows, g["H"]), sentinel, np.uint16)
    oracle.dispatch(x, h["pair_to_row"], g["K"], oracle.QUANT_NONE, rows, out_x=out_x)
    for r, v in ex["out_x_rows"].items():
        assert np.array_equal(out_x[int(r)], _bf16(v)), r
    for r in ex["untouched_rows"]:
        assert np.all(out_x[r] == sentinel)
    y = np.zeros((rows, g["H"]), np.uint16)
    for r, v in ex["y_scaled_rows"].items():
        y[int(r)] = _bf16(v)
    out = oracle.combine(y, np.array(g["topk_w"], np.float32), h["pair_to_row"])
    assert np.array_equal(out, _bf16(ex["out"]))


def _brute_layout(idx, E, R, layout, align, capacity):
    """Tiny-input brute force straight from the definitions (quadratic)."""
    flat = idx.reshape(-1)
    P = flat.size
    routed = [(0 <= e < E) for e in flat]
    count = [sum(1 for p in range(P) if routed[p] and flat[p] == e) for e in range(E)]
    invalid = sum(1 for p in range(P) if not routed[p] and flat[p] != -1)
    if layout == oracle.CONTIGUOUS:
        off = [0]
        for e in range(E):
            off.append(off[-1] + -(-count[e] // align) * align)
        recv = list(count)
        overflow = 0
    else:
        off = [e * capacity for e in range(E + 1)]
        recv = [min(c, capacity) for c in count]
        overflow = sum(max(0, c - capacity) for c in count)
    rows = P + E * (align - 1) if layout == oracle.CONTIGUOUS else E * capacity
    p2r = []
    for p in range(P):
        if not routed[p]:
            p2r.append(-1)
            continue
        slot = sum(1 for q in range(p) if routed[q] and flat[q] == flat[p])
        if layout == oracle.CONTIGUOUS:
            p2r.append(off[flat[p]] + slot)
        else:
            p2r.append(flat[p] * capacity + slot if slot < capacity else -1)
    r2p = [-1] * rows
    for p, r in enumerate(p2r):
        if r >= 0:
            r2p[r] = p
    L = E // R
    return dict(expert_count=count, recv_count=recv, expert_offset=off,
                rank_offset=[off[r * L] for r in range(R + 1)], pair_to_row=p2r,
                row_to_pair=r2p, status=[overflow, invalid])


def _random_ids(rng, T, K, E, allow_bad):
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    if allow_bad:
        m = rng.random((T, K))
        idx[m < 0.1] = -1
        idx[(m >= 0.1) & (m < 0.15)] = E + rng.integers(0, 3)
        idx[(m >= 0.15) & (m < 0.17)] = -2 - rng.integers(0, 3)
    return idx


def test_layout_brute_force_tiny(oracle_lib):
    rng = np.random.default_rng(21)
    n = 0
    for E in (1, 2, 3, 4, 6, 8):
        for R in [r for r in (1, 2, 3, 4, 8) if E % r == 0]:
            for K in (1, 2, 3, 4):
                for T in (0, 1, 5, 13):
                    for layout, align, cap in ((0, 1, 1), (0, 2, 1), (0, 4, 1),
                                               (1, 1, 1), (1, 1, 2), (1, 1, 5)):
                        idx = _random_ids(rng, T, K, E, allow_bad=(n % 2 == 0))
                        h = oracle.dispatch_layout(idx, E, R, layout, align, cap)
                        b = _brute_layout(idx, E, R, layout, align, cap)
                        for k in LAYOUT_KEYS:
                            assert h[k].tolist() == b[k], (k, E, R, K, T, layout, align, cap)
                        n += 1
    assert n > 500


def test_layout_align1_equals_stable_argsort(oracle_lib):
    rng = np.random.default_rng(22)
    for E, K, T in ((8, 2, 64), (128, 8, 300), (256, 8, 1000)):
        idx = _random_ids(rng, T, K, E, allow_bad=True)
        h = oracle.dispatch_layout(idx, E, 1, oracle.CONTIGUOUS, 1)
        flat = idx.reshape(-1)
        valid = np.nonzero((flat >= 0) & (flat < E))[0]
        order = valid[np.argsort(flat[valid], kind="stable")]
        n = order.size
        assert np.array_equal(h["row_to_pair"][:n], order)
        assert np.all(h["row_to_pair"][n:] == -1)
        assert np.array_equal(h["expert_count"], np.bincount(flat[valid], minlength=E))


def check_layout_invariants(h, idx, E, R, layout, align, capacity, rows_cap):
    """Properties any correct layout has; shared by the CPU and GPU tests."""
    flat = idx.reshape(-1).astype(np.int64)
    P = flat.size
    valid = (flat >= 0) & (flat < E)
    cnt = np.bincount(flat[valid], minlength=E)
    assert np.array_equal(h["expert_count"], cnt)
    assert h["status"][1] == int(np.sum(~valid & (flat != -1)))
    off = h["expert_offset"].astype(np.int64)
    assert off[0] == 0 and np.all(np.diff(off) >= 0)
    if layout == oracle.CONTIGUOUS:
        assert np.all(off % align == 0)
        assert np.array_equal(np.diff(off), -(-cnt // align) * align)
        assert np.array_equal(h["recv_count"], cnt)
        assert h["status"][0] == 0
    else:
        assert np.array_equal(off, np.arange(E + 1) * capacity)
        assert np.array_equal(h["recv_count"], np.minimum(cnt, capacity))
        assert h["status"][0] == int(np.sum(np.maximum(cnt - capacity, 0)))
    L = E // R
    assert np.array_equal(h["rank_offset"], h["expert_offset"][::L])
    p2r = h["pair_to_row"].astype(np.int64)
    r2p = h["row_to_pair"].astype(np.int64)
    assert r2p.size == rows_cap
    kept = np.nonzero(p2r >= 0)[0]
    assert np.all(valid[kept])
    assert np.unique(p2r[kept]).size == kept.size          # injective
    assert np.array_equal(r2p[p2r[kept]], kept)             # bijection on kept pairs
    assert int(np.sum(r2p >= 0)) == kept.size               # no other row claims a pair
    e_of = flat[kept]
    rows = p2r[kept]
    assert np.all(rows >= off[e_of]) and np.all(rows < off[e_of] + h["recv_count"][e_of])
    # rows of one expert are consecutive from the segment start, in ascending p
    for e in np.unique(e_of):
        sel = kept[e_of == e]
        assert np.array_equal(p2r[sel], off[e] + np.arange(sel.size))
    if layout == oracle.MASKED:
        # dropped pairs are exactly the routed ones whose slot >= capacity
        dropped = np.nonzero(valid & (p2r < 0))[0]
        for p in dropped[:200]:
            assert np.sum(flat[:p] == flat[p]) >= capacity


def test_layout_invariants_random(oracle_lib):
    rng = np.random.default_rng(23)
    for E, R, K, T, layout, align, cap in ((256, 8, 8, 2048, 0, 128, 1),
                                           (256, 8, 8, 2048, 1, 1, 64),
                                           (128, 8, 8, 700, 0, 16, 1),
                                           (5, 5, 3, 999, 1, 1, 7),
                                           (64, 4, 32, 100, 0, 3, 1)):
        idx = _random_ids(rng, T, K, E, allow_bad=True)
        rows_cap = oracle.rows_capacity(T, K, E, layout, align, cap)
        h = oracle.dispatch_layout(idx, E, R, layout, align, cap)
        check_layout_invariants(h, idx, E, R, layout, align, cap, rows_cap)


def test_layout_empty_batch(oracle_lib):
    idx = np.zeros((0, 8), np.int32)
    h = oracle.dispatch_layout(idx, 16, 4, oracle.CONTIGUOUS, 4, rows_cap=100)
    assert not h["expert_count"].any() and not h["expert_offset"].any()
    assert not h["rank_offset"].any() and np.all(h["row_to_pair"] == -1)
    h = oracle.dispatch_layout(idx, 16, 4, oracle.MASKED, 1, 3)
    assert h["expert_offset"].tolist() == [3 * e for e in range(17)]
    assert not h["recv_count"].any() and np.all(h["row_to_pair"] == -1)
    assert h["status"].tolist() == [0, 0]


# ----------------------------------------------------------------------------
# Dispatch
# ----------------------------------------------------------------------------

def test_quant_golden_blocks(oracle_lib):
    g = _golden("quant_blocks_H384.json")
    H = g["H"]
    xf = np.zeros(H, np.float32)
    for j, v in g["x_nonzero"].items():
        xf[int(j)] = v
    x = _bf16(xf)[None, :]
    p2r = np.array([0], np.int32)
    q, s, _ = oracle.dispatch(x, p2r, 1, oracle.QUANT_FP8_F32, 1)
    ex = g["expected_fp32"]
    sb = s[0].view(np.uint32)
    for b, want in enumerate(ex["scales_bits"]):
        if want is not None:
            assert sb[b] == int(want, 16), (b, hex(sb[b]))
    want_q = np.zeros(H, np.uint8)
    for j, c in ex["q_nonzero"].items():
        want_q[int(j)] = int(c, 16)
    assert np.array_equal(q[0], want_q)
    q, wd, _ = oracle.dispatch(x, p2r, 1, oracle.QUANT_FP8_UE8M0, 1)
    ex = g["expected_ue8m0"]
    assert wd.shape == (1, 1) and wd[0, 0] == int(ex["word"], 16)
    want_q[:] = 0
    for j, c in ex["q_nonzero"].items():
        want_q[int(j)] = int(c, 16)
    assert np.array_equal(q[0], want_q)


def _quant_inputs(rng, T, H):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] *= 50.0                                  # outlier row
    x[1, :128] = 0.0                              # all-zero block
    x[2, 128:256] = rng.standard_normal(128) * 1e-39  # bf16 subnormals
    x[3, :128] = -0.0                             # negative zeros
    x[4] = rng.standard_normal(H) * 1e30          # huge magnitudes
    x[5] = rng.standard_normal(H) * 1e-30         # tiny magnitudes
    x[6] = rng.standard_normal(H) * 1e-8          # block maxima near the 1e-10 floor
    x[7] = rng.standard_normal(H) * 3e-11         # block maxima around the floor
    return W.f32_to_bf16_bits(x)


def test_dispatch_fp32_scales_vs_torch(oracle_lib):
    rng = np.random.default_rng(31)
    T, H, K = 40, 512, 2
    x = _quant_inputs(rng, T, H)
    p2r = np.arange(T * K, dtype=np.int32)
    q, s, _ = oracle.dispatch(x, p2r, K, oracle.QUANT_FP8_F32, T * K)
    xf = torch.from_numpy(_f32(x)).view(T, H // 128, 128)
    a = torch.clamp(xf.abs().amax(dim=2), min=1e-10)
    s_ref = a / 448.0                                 # binary32 division
    qv = torch.clamp(xf / s_ref[:, :, None], -448.0, 448.0).reshape(T, H)
    q_ref = qv.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for k in range(K):
        assert np.array_equal(s[k::K], s_ref.numpy())
        assert np.array_equal(q[k::K], q_ref)
    # the element reaching amax encodes to +-448
    amax_pos = xf.abs().argmax(dim=2)
    top = np.take_along_axis(q[::K].reshape(T, H // 128, 128), amax_pos.numpy()[:, :, None], 2)
    nz = a.numpy() > 1e-10
    assert np.all((top[:, :, 0][nz] & 0x7F) == 0x7E)
    # dequantisation error bound: within half an E4M3 ulp of x/s
    deq = _torch_e4m3_decode(q[::K]).reshape(T, H // 128, 128) * s_ref.numpy()[:, :, None]
    xd = xf.numpy().astype(np.float64)
    err = np.abs(deq - xd)
    sd = s_ref.numpy().astype(np.float64)[:, :, None]
    bound = np.maximum(np.abs(xd) * 2.0 ** -4, sd * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_dispatch_ue8m0_vs_torch(oracle_lib):
    rng = np.random.default_rng(32)
    T, H, K = 40, 640, 3   # 5 blocks: the second packed word has 1 used byte
    x = _quant_inputs(rng, T, H)
    p2r = np.arange(T * K, dtype=np.int32)
    q, w, _ = oracle.dispatch(x, p2r, K, oracle.QUANT_FP8_UE8M0, T * K)
    assert w.shape == (T * K, 2)
    by = w.view(np.uint8).reshape(T * K, 8)           # little-endian bytes
    assert np.all(by[:, 5:] == 0)                     # unused bytes are zero
    kexp = by[:, :5].astype(np.int64) - 127
    xf = _f32(x).reshape(T, H // 128, 128).astype(np.float64)
    a = np.maximum(np.abs(xf).max(axis=2), np.float32(1e-10))
    for k in range(K):
        kk = kexp[k::K]
        assert np.all(a <= np.ldexp(448.0, kk)) and np.all(a > np.ldexp(448.0, kk - 1))
        scaled = torch.from_numpy(np.ldexp(xf, -kk[:, :, None]).astype(np.float32))
        q_ref = scaled.reshape(T, H).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[k::K], q_ref)


def test_dispatch_bf16_rows_and_untouched(oracle_lib):
    rng = np.random.default_rng(33)
    T, H, E, K, C = 50, 64, 6, 3, 9
    idx = _random_ids(rng, T, K, E, allow_bad=True)
    h = oracle.dispatch_layout(idx, E, 3, oracle.MASKED, 1, C)
    rows = E * C
    x = _bf16(rng.standard_normal((T, H)))
    w = rng.random((T, K)).astype(np.float32)
    out_x = np.full((rows, H), 0xA5A5, np.uint16)
    rw = np.full(rows, np.nan, np.float32)
    oracle.dispatch(x, h["pair_to_row"], K, oracle.QUANT_NONE, rows, topk_w=w,
                    out_x=out_x, out_row_weight=rw)
    p2r = h["pair_to_row"]
    kept = np.nonzero(p2r >= 0)[0]
    assert h["status"][0] > 0  # the case exercises overflow
    assert np.array_equal(out_x[p2r[kept]], x[kept // K])
    assert np.array_equal(rw[p2r[kept]], w.reshape(-1)[kept])
    untouched = np.ones(rows, bool)
    untouched[p2r[kept]] = False
    assert np.all(out_x[untouched] == 0xA5A5) and np.all(np.isnan(rw[untouched]))


# ----------------------------------------------------------------------------
# Combine
# ----------------------------------------------------------------------------

def test_combine_vs_torch_float32_same_order(oracle_lib):
    """torch CPU float32 ops (separate multiply and add, ascending k) and its
    bfloat16 cast reproduce the definition exactly."""
    rng = np.random.default_rng(41)
    T, H, E, K = 64, 96, 16, 4
    idx = _random_ids(rng, T, K, E, allow_bad=True)
    h = oracle.dispatch_layout(idx, E, 4, oracle.MASKED, 1, 12)
    rows = E * 12
    y = _bf16(rng.standard_normal((rows, H)) * 3)
    w = rng.standard_normal((T, K)).astype(np.float32)
    out = oracle.combine(y, w, h["pair_to_row"])
    yt = torch.from_numpy(_f32(y))
    acc = torch.zeros((T, H), dtype=torch.float32)
    p2r = torch.from_numpy(h["pair_to_row"].reshape(T, K).astype(np.int64))
    wt = torch.from_numpy(w)
    for k in range(K):
        keep = p2r[:, k] >= 0
        prod = wt[:, k:k + 1] * yt[p2r[:, k].clamp(min=0)]
        acc = torch.where(keep[:, None], acc + prod, acc)
    ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_combine_closed_form_scaled_experts(oracle_lib):
    wl = W.WORKLOADS["tiny_T64"]
    inp = W.make_inputs(wl)
    h = oracle.dispatch_layout(inp.topk_idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity)
    y = W.expert_outputs(wl, inp, h["row_to_pair"])
    out = _f32(oracle.combine(y, inp.topk_w, h["pair_to_row"])).astype(np.float64)
    fac = (inp.topk_w.astype(np.float64) * (inp.topk_idx + 1) * 0.5).sum(axis=1)
    ref = _f32(inp.x).astype(np.float64) * fac[:, None]
    assert np.all(np.abs(out - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-30)


def test_combine_identity_experts_returns_x(oracle_lib):
    """Identity experts with weights summing to one give back x exactly."""
    rng = np.random.default_rng(42)
    T, H, E, K = 100, 256, 32, 8
    idx, w = W.route_softmax(rng, T, E, K)
    h = oracle.dispatch_layout(idx, E, 8, oracle.CONTIGUOUS, 4)
    x = _bf16(rng.standard_normal((T, H)))
    rows = oracle.rows_capacity(T, K, E, oracle.CONTIGUOUS, 4)
    y, _, _ = oracle.dispatch(x, h["pair_to_row"], K, oracle.QUANT_NONE, rows)
    out = oracle.combine(y, w, h["pair_to_row"])
    assert np.array_equal(out, x)


def test_combine_token_without_kept_pairs_is_positive_zero(oracle_lib):
    idx = np.array([[0, 1], [-1, -1], [1, 0]], np.int32)
    h = oracle.dispatch_layout(idx, 2, 1, oracle.MASKED, 1, 1)  # token 2 overflows
    y = _bf16(np.ones((2, 8)))
    out = oracle.combine(y, np.full((3, 2), -0.5, np.float32), h["pair_to_row"])
    assert np.all(out[1] == 0) and np.all(out[2] == 0)
    assert np.all(out[0] == _bf16([-1.0])[0])


# ----------------------------------------------------------------------------
# Input generators
# ----------------------------------------------------------------------------

def test_group_limited_router_properties():
    rng = np.random.default_rng(51)
    idx, w = W.route_group_limited(rng, 500, 256, 8, 8, 4)
    assert idx.dtype == np.int32 and w.dtype == np.float32
    assert all(len(set(r)) == 8 for r in idx.tolist())
    assert np.all(np.unique(idx // 32, axis=None).size <= 8)
    assert max(len(set((r // 32).tolist())) for r in idx) <= 4
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6) and np.all(w > 0)


def test_zipf_router_skew_and_distinct():
    rng = np.random.default_rng(52)
    idx, w = W.route_zipf(rng, 4000, 256, 8, 1.2)
    assert all(len(set(r)) == 8 for r in idx.tolist())
    cnt = np.bincount(idx.reshape(-1), minlength=256)
    assert cnt.max() > 5 * np.median(cnt)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_generators_are_deterministic():
    wl = W.WORKLOADS["qwen3moe_decode_T128"]
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    assert np.array_equal(a.topk_idx, b.topk_idx) and np.array_equal(a.x, b.x)
    assert np.array_equal(a.topk_w, b.topk_w)
    assert a.x.shape == (128, 2048) and a.topk_idx.shape == (128, 8)
