"""Pins for the oracle's grouped-GEMM adapters (no GPU needed): per-row
expert indices, masked <-> contiguous repack, MN-major scales.

Checked against a hand-worked fixture, brute force, the already pinned
dispatch layout and dispatch (a repacked masked dispatch must equal the
contiguous dispatch of the same kept pairs byte for byte), round trips,
combine under either layout, and numpy's transpose.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_topk_idx_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0xA5
QUANTS = [oracle.QUANT_NONE, oracle.QUANT_FP8_F32, oracle.QUANT_FP8_UE8M0, oracle.QUANT_MXFP8]


def _scale_buf(rows, H, quant):
    nb = H // 128
    if quant == oracle.QUANT_FP8_F32:
        return np.full((rows, nb * 4), SENT, np.uint8).view(np.float32)
    if quant == oracle.QUANT_FP8_UE8M0:
        return np.full((rows, (nb + 3) // 4 * 4), SENT, np.uint8).view(np.uint32)
    if quant == oracle.QUANT_MXFP8:
        return np.full((rows, H // 32), SENT, np.uint8)
    return None


def _x_buf(rows, H, quant):
    b = np.full((rows, H * (2 if quant == oracle.QUANT_NONE else 1)), SENT, np.uint8)
    return b.view(np.uint16) if quant == oracle.QUANT_NONE else b


def test_repack_golden(oracle_lib):
    g = json.load(open(os.path.join(GOLDEN, "repack_masked_E3_C4_A2.json")))
    E, C, A = g["E"], g["C"], g["align"]
    H = 8
    x = (np.arange(E * C)[:, None] * 16 + np.arange(H)[None, :]).astype(np.uint16)
    out = np.full((6, H), 0xFFFF, np.uint16)
    ox, _, off, rex = oracle.repack_masked_to_contiguous(x, None, np.array(g["recv_count"]), C, A,
                                                         oracle.QUANT_NONE, 6, out_x=out)
    assert off.tolist() == g["out_offset"]
    assert rex.tolist() == g["out_row_expert"]
    for r, src in enumerate(g["src_row_of_out_row"]):
        assert ox[r].tolist() == (x[src].tolist() if src >= 0 else [0xFFFF] * H)


def test_row_expert_matches_layout(oracle_lib):
    """For a contiguous dispatch layout, the row's expert is the id of the
    pair the layout put there (row_to_pair), -1 for padding and the tail."""
    rng = np.random.default_rng(41)
    for T, K, E, A in ((50, 4, 12, 4), (200, 8, 32, 16), (7, 2, 3, 1)):
        idx = rng.integers(-1, E, (T, K)).astype(np.int32)
        h = oracle.dispatch_layout(idx, E, 1, oracle.CONTIGUOUS, align=A)
        rows = h["row_to_pair"].size
        rex = oracle.row_expert(h["expert_offset"], h["recv_count"], rows)
        want = np.where(h["row_to_pair"] >= 0, idx.reshape(-1)[np.maximum(h["row_to_pair"], 0)], -1)
        assert np.array_equal(rex, want)
        hm = oracle.dispatch_layout(idx, E, 1, oracle.MASKED, capacity=3)
        rexm = oracle.row_expert(hm["expert_offset"], hm["recv_count"], E * 3)
        wantm = np.where(hm["row_to_pair"] >= 0, idx.reshape(-1)[np.maximum(hm["row_to_pair"], 0)], -1)
        assert np.array_equal(rexm, wantm)


@pytest.mark.parametrize("quant", QUANTS)
@pytest.mark.parametrize("cap", [6, 40])
def test_repacked_masked_dispatch_equals_contiguous_dispatch(oracle_lib, quant, cap):
    """Repacking a masked dispatch gives, byte for byte, the contiguous
    dispatch of the pairs the masked layout kept (dropped pairs removed),
    with the same offsets; untouched rows stay untouched."""
    rng = np.random.default_rng(42 + quant + cap)
    T, K, E, H, A = 60, 4, 10, 256, 4
    idx = rng.integers(-1, E, (T, K)).astype(np.int32)
    xf = rng.standard_normal((T, H)).astype(np.float32)
    xf[rng.random(T) < 0.1] *= 500
    x = W.f32_to_bf16_bits(xf)
    hm = oracle.dispatch_layout(idx, E, 1, oracle.MASKED, capacity=cap)
    mrows = E * cap
    mx, ms = _x_buf(mrows, H, quant), _scale_buf(mrows, H, quant)
    oracle.dispatch(x, hm["pair_to_row"], K, quant, mrows, out_x=mx, out_scale=ms)
    kept_idx = np.where(hm["pair_to_row"].reshape(T, K) >= 0, idx, -1)
    hc = oracle.dispatch_layout(kept_idx, E, 1, oracle.CONTIGUOUS, align=A)
    crows = hc["row_to_pair"].size
    cx, cs = _x_buf(crows, H, quant), _scale_buf(crows, H, quant)
    oracle.dispatch(x, hc["pair_to_row"], K, quant, crows, out_x=cx, out_scale=cs)
    rx, rs = _x_buf(crows, H, quant), _scale_buf(crows, H, quant)
    rx, rs, off, rex = oracle.repack_masked_to_contiguous(mx, ms, hm["recv_count"], cap, A, quant, crows,
                                                          out_x=rx, out_scale=rs)
    assert np.array_equal(off, hc["expert_offset"])
    assert np.array_equal(rx.view(np.uint8), cx.view(np.uint8))
    if rs is not None:
        assert np.array_equal(rs.view(np.uint8), cs.view(np.uint8))
    assert np.array_equal(rex, oracle.row_expert(hc["expert_offset"], hc["recv_count"], crows))
    if cap == 6:
        assert hm["status"][0] > 0   # drops exercised


def test_contiguous_to_masked_round_trip_and_combine(oracle_lib):
    """Expert outputs written in the repacked contiguous layout and moved
    back to the slab combine exactly as if written in the slab; slab rows
    holding no pair are not written."""
    rng = np.random.default_rng(43)
    T, K, E, H, C, A = 80, 6, 12, 64, 30, 8
    idx = rng.integers(-1, E, (T, K)).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    hm = oracle.dispatch_layout(idx, E, 1, oracle.MASKED, capacity=C)
    rc = hm["recv_count"]
    off = np.concatenate([[0], np.cumsum((rc + A - 1) // A * A)]).astype(np.int32)
    crows = int(off[-1])
    y_c = W.f32_to_bf16_bits(rng.standard_normal((crows, H)).astype(np.float32))
    y_m = np.full((E * C, H), 0x7FC1, np.uint16)
    oracle.repack_contiguous_to_masked(y_c, rc, off, C, out=y_m)
    for e in range(E):
        for s in range(C):
            if s < rc[e]:
                assert np.array_equal(y_m[e * C + s], y_c[off[e] + s])
            else:
                assert np.all(y_m[e * C + s] == 0x7FC1)
    # combine through the slab equals combine through the contiguous layout
    p2r_c = np.full(T * K, -1, np.int32)
    for p in range(T * K):
        r = hm["pair_to_row"][p]
        if r >= 0:
            e, s = divmod(int(r), C)
            p2r_c[p] = off[e] + s
    assert np.array_equal(oracle.combine(y_m, w, hm["pair_to_row"]), oracle.combine(y_c, w, p2r_c))


def test_scales_mn_major_vs_numpy(oracle_lib):
    rng = np.random.default_rng(44)
    for rows, S in ((1, 1), (3, 5), (10, 7), (5, 3), (98048, 14), (13, 56)):
        a = rng.integers(0, 2 ** 32, (rows, S), dtype=np.uint64).astype(np.uint32)
        out = oracle.scales_mn_major(a)
        ld = -(-rows // 4) * 4
        want = np.zeros((S, ld), np.uint32)
        want[:, :rows] = a.T
        assert out.shape == (S, ld) and np.array_equal(out, want)
