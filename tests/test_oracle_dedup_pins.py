"""Pins for the oracle's per-rank deduplicated exchange (no GPU needed).

The per-rank layout, the deduplicated dispatch, the receive-side expansion and
the two-level (partial + reduce) combine are checked against hand-worked
fixtures (tests/golden/), brute force on tiny inputs, the already pinned
one-level functions they must reduce to (dispatch, combine), closed forms and
invariants.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from combine_topk_idx_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SENT = 0xA5


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(a):
    return np.array([[int(v, 16) for v in row] for row in a], np.uint16)


def _random_ids(rng, T, K, E, bad=True):
    idx = rng.integers(0, E, (T, K)).astype(np.int32)
    if bad:
        m = rng.random((T, K))
        idx[m < 0.1] = -1
        idx[(m >= 0.1) & (m < 0.15)] = E + rng.integers(0, 5)
        idx[(m >= 0.15) & (m < 0.18)] = -7
    return idx


def _brute_rank_layout(idx, E, R):
    """Sets of ranks per token, then rows in (rank, token) order."""
    T, K = idx.shape
    L = E // R
    ranks = [sorted({int(e) // L for e in idx[t] if 0 <= e < E}) for t in range(T)]
    rows = {}
    nxt = 0
    count = []
    for r in range(R):
        c = 0
        for t in range(T):
            if r in ranks[t]:
                rows[(t, r)] = nxt
                nxt += 1
                c += 1
        count.append(c)
    return ranks, rows, count


# ----------------------------------------------------------------------------
# Per-rank layout
# ----------------------------------------------------------------------------

def test_rank_layout_golden(oracle_lib):
    g = _golden("rank_layout_T5_E8_K3_R4.json")
    h = oracle.rank_layout(np.array(g["topk_idx"], np.int32), g["E"], g["R"])
    assert h["rank_token_count"].tolist() == g["rank_token_count"]
    assert h["rank_token_offset"].tolist() == g["rank_token_offset"]
    assert h["token_rank_row"].reshape(-1, g["R"]).tolist() == g["token_rank_row"]
    assert h["rank_row_to_token"].tolist() == g["rank_row_to_token"]


def test_rank_layout_brute_force_tiny(oracle_lib):
    rng = np.random.default_rng(11)
    n = 0
    for T, K, E, R in itertools.product((0, 1, 3, 9), (1, 2, 5), (1, 4, 12), (1, 2, 4)):
        if E % R:
            continue
        for _ in range(6):
            idx = _random_ids(rng, T, K, E)
            h = oracle.rank_layout(idx, E, R)
            ranks, rows, count = _brute_rank_layout(idx, E, R)
            assert h["rank_token_count"].tolist() == count
            assert h["rank_token_offset"].tolist() == np.concatenate([[0], np.cumsum(count)]).tolist()
            trr = h["token_rank_row"].reshape(T, R)
            for t in range(T):
                for r in range(R):
                    assert trr[t, r] == rows.get((t, r), -1)
            inv = -np.ones(T * min(K, R), np.int32)
            for (t, r), q in rows.items():
                inv[q] = t
            assert np.array_equal(h["rank_row_to_token"], inv)
            n += 1
    assert n > 200


def test_rank_layout_relations_to_expert_layout(oracle_lib):
    """Against the (pinned) per-expert layout: a token's rank rows exist
    exactly where its kept-or-not valid pairs point, and a rank's token count
    is its pair count minus same-rank repeats within a token."""
    rng = np.random.default_rng(12)
    for T, K, E, R in ((64, 8, 32, 8), (50, 4, 16, 16), (33, 6, 24, 3), (20, 8, 8, 1)):
        idx = _random_ids(rng, T, K, E)
        L = E // R
        h = oracle.rank_layout(idx, E, R)
        e_lay = oracle.dispatch_layout(idx, E, R, oracle.CONTIGUOUS)
        trr = h["token_rank_row"].reshape(T, R)
        valid = (idx >= 0) & (idx < E)
        member = np.zeros((T, R), bool)
        for t in range(T):
            for k in range(K):
                if valid[t, k]:
                    member[t, idx[t, k] // L] = True
        assert np.array_equal(trr >= 0, member)
        pairs_per_rank = np.array([e_lay["expert_count"][r * L:(r + 1) * L].sum() for r in range(R)])
        repeats = np.zeros(R, np.int64)
        for t in range(T):
            rs = idx[t][valid[t]] // L
            for r in range(R):
                c = int((rs == r).sum())
                repeats[r] += max(c - 1, 0)
        assert np.array_equal(h["rank_token_count"], pairs_per_rank - repeats)
        # rows of each rank: consecutive, tokens ascending
        for r in range(R):
            rows = trr[:, r][trr[:, r] >= 0]
            assert np.array_equal(rows, np.arange(h["rank_token_offset"][r], h["rank_token_offset"][r + 1]))


def test_rank_layout_empty_and_overflow(oracle_lib):
    h = oracle.rank_layout(np.zeros((0, 4), np.int32), 8, 4)
    assert h["rank_token_count"].tolist() == [0] * 4
    assert h["rank_token_offset"].tolist() == [0] * 5
    with pytest.raises(ValueError):
        oracle.rank_layout(np.array([[0, 2, 4, 6]], np.int32), 8, 4, rows_cap=3)


# ----------------------------------------------------------------------------
# Deduplicated dispatch and receive-side expansion
# ----------------------------------------------------------------------------

def _x(rng, T, H):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[rng.random(T) < 0.1] *= 300.0
    x[:, :128][rng.random(T) < 0.1] = 0.0
    return W.f32_to_bf16_bits(x)


def _sentinel_bufs(rows, H, quant):
    NB = H // 128
    ox = np.full((rows, H * (2 if quant == oracle.QUANT_NONE else 1)), SENT, np.uint8)
    ox = ox.view(np.uint16) if quant == oracle.QUANT_NONE else ox
    if quant == oracle.QUANT_FP8_F32:
        sc = np.full((rows, NB * 4), SENT, np.uint8).view(np.float32)
    elif quant == oracle.QUANT_FP8_UE8M0:
        sc = np.full((rows, (NB + 3) // 4 * 4), SENT, np.uint8).view(np.uint32)
    elif quant == oracle.QUANT_MXFP8:
        sc = np.full((rows, H // 32), SENT, np.uint8)
    else:
        sc = None
    return ox, sc


@pytest.mark.parametrize("quant", [oracle.QUANT_NONE, oracle.QUANT_FP8_F32, oracle.QUANT_FP8_UE8M0,
                                   oracle.QUANT_MXFP8])
@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.MASKED])
def test_expand_of_dedup_equals_direct_dispatch(oracle_lib, quant, layout):
    """Sending each token once per rank and expanding on the receiver gives
    the per-expert rows of the direct dispatch byte for byte (quantization
    is per token, so the bytes cannot differ); untouched rows stay untouched."""
    rng = np.random.default_rng(13 + quant + 3 * layout)
    T, K, E, R, H = 40, 6, 16, 4, 384
    idx = _random_ids(rng, T, K, E)
    x = _x(rng, T, H)
    cap = 7
    lay = oracle.dispatch_layout(idx, E, R, layout, align=4, capacity=cap)
    rows = lay["row_to_pair"].size
    rk = oracle.rank_layout(idx, E, R)
    qrows = rk["rank_row_to_token"].size
    sx, ss = _sentinel_bufs(qrows, H, quant)
    sx, ss = oracle.dispatch_dedup(x, rk["token_rank_row"], R, quant, qrows, out_x=sx, out_scale=ss)
    ex, es = _sentinel_bufs(rows, H, quant)
    ex, es = oracle.expand(idx, E, R, quant, sx, ss, rk["token_rank_row"], lay["pair_to_row"], rows,
                           out_x=ex, out_scale=es)
    dx, ds = _sentinel_bufs(rows, H, quant)
    oracle.dispatch(x, lay["pair_to_row"], K, quant, rows, out_x=dx, out_scale=ds)
    assert np.array_equal(ex.view(np.uint8), dx.view(np.uint8))
    if ss is not None:
        assert np.array_equal(es.view(np.uint8), ds.view(np.uint8))
    if layout == oracle.MASKED:
        assert lay["status"][0] > 0  # drops exercised


def test_dispatch_dedup_bf16_rows_closed_form(oracle_lib):
    rng = np.random.default_rng(14)
    T, K, E, R, H = 30, 4, 12, 3, 40
    idx = _random_ids(rng, T, K, E)
    x = _x(rng, T, H)
    rk = oracle.rank_layout(idx, E, R)
    qrows = rk["rank_row_to_token"].size
    sx, _ = _sentinel_bufs(qrows, H, oracle.QUANT_NONE)
    oracle.dispatch_dedup(x, rk["token_rank_row"], R, oracle.QUANT_NONE, qrows, out_x=sx)
    r2t = rk["rank_row_to_token"]
    for q in range(qrows):
        if r2t[q] >= 0:
            assert np.array_equal(sx[q], x[r2t[q]])
        else:
            assert np.all(sx[q].view(np.uint8) == SENT)


# ----------------------------------------------------------------------------
# Two-level combine
# ----------------------------------------------------------------------------

def test_combine_two_level_golden(oracle_lib):
    g = _golden("combine_two_level_T1_K3_R2.json")
    idx = np.array(g["topk_idx"], np.int32)
    w = np.array(g["topk_w"], np.float32)
    p2r = np.array(g["pair_to_row"], np.int32)
    y = _bits(g["y_bf16_bits"])
    rk = oracle.rank_layout(idx, g["E"], g["R"])
    assert rk["token_rank_row"].reshape(-1, g["R"]).tolist() == g["token_rank_row"]
    lay = oracle.dispatch_layout(idx, g["E"], g["R"], oracle.CONTIGUOUS)
    assert lay["pair_to_row"].tolist() == g["pair_to_row"]
    part = oracle.combine_partial(idx, g["E"], g["R"], y, w, p2r, rk["token_rank_row"], 2)
    assert np.array_equal(part, _bits(g["partial_bf16_bits"]))
    out = oracle.combine_reduce(part, rk["token_rank_row"], g["R"])
    assert np.array_equal(out, _bits(g["out_two_level_bf16_bits"]))
    assert np.array_equal(oracle.combine(y, w, p2r), _bits(g["out_one_level_bf16_bits"]))


def _case(rng, T, K, E, R, H, layout=oracle.CONTIGUOUS, cap=4):
    idx = _random_ids(rng, T, K, E)
    w = rng.random((T, K)).astype(np.float32)
    lay = oracle.dispatch_layout(idx, E, R, layout, capacity=cap)
    rows = lay["row_to_pair"].size
    y = W.f32_to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    rk = oracle.rank_layout(idx, E, R)
    return idx, w, lay, y, rk


def test_two_level_with_one_rank_is_one_level(oracle_lib):
    """R = 1: the single partial is the one-level combine, and reducing one
    bf16 value returns it unchanged."""
    rng = np.random.default_rng(15)
    idx, w, lay, y, rk = _case(rng, 37, 6, 10, 1, 24)
    part = oracle.combine_partial(idx, 10, 1, y, w, lay["pair_to_row"], rk["token_rank_row"],
                                  rk["rank_row_to_token"].size)
    one = oracle.combine(y, w, lay["pair_to_row"])
    trr = rk["token_rank_row"]
    for t in range(37):
        if trr[t] >= 0:
            assert np.array_equal(part[trr[t]], one[t])
        else:
            assert not np.any(one[t])
    assert np.array_equal(oracle.combine_reduce(part, trr, 1), one)


def test_partial_single_pair_closed_form(oracle_lib):
    """One expert per rank and distinct experts per token: each partial is
    one product rounded to bf16 (torch's float32 product and bf16 cast)."""
    rng = np.random.default_rng(16)
    T, K, E, H = 25, 4, 8, 16
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, K)).astype(np.float32)
    lay = oracle.dispatch_layout(idx, E, E, oracle.CONTIGUOUS)
    y = W.f32_to_bf16_bits(rng.standard_normal((lay["row_to_pair"].size, H)).astype(np.float32))
    rk = oracle.rank_layout(idx, E, E)
    part = oracle.combine_partial(idx, E, E, y, w, lay["pair_to_row"], rk["token_rank_row"],
                                  rk["rank_row_to_token"].size)
    trr = rk["token_rank_row"].reshape(T, E)
    yt = torch.from_numpy(W.bf16_bits_to_f32(y))
    for t in range(T):
        for k in range(K):
            row = lay["pair_to_row"][t * K + k]
            prod = torch.tensor(w[t, k]) * yt[row]
            want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(part[trr[t, idx[t, k]]], want)


def test_reduce_vs_torch_float32_ascending_rank(oracle_lib):
    """combine_reduce is the fp32 sum of the partials in ascending rank,
    rounded once to bf16 (torch float32 adds, same order)."""
    rng = np.random.default_rng(17)
    idx, w, lay, y, rk = _case(rng, 31, 8, 16, 4, 40)
    part = oracle.combine_partial(idx, 16, 4, y, w, lay["pair_to_row"], rk["token_rank_row"],
                                  rk["rank_row_to_token"].size)
    out = oracle.combine_reduce(part, rk["token_rank_row"], 4)
    pf = torch.from_numpy(W.bf16_bits_to_f32(part))
    trr = rk["token_rank_row"].reshape(31, 4)
    for t in range(31):
        acc = torch.zeros(40, dtype=torch.float32)
        for r in range(4):
            if trr[t, r] >= 0:
                acc = acc + pf[trr[t, r]]
        want = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(out[t], want)


@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.MASKED])
def test_two_level_close_to_exact_sum(oracle_lib, layout):
    """Against the float64 sum of the kept products: two bf16 roundings and
    fp32 accumulation bound the error by 2^-7 S + 2^-8 |exact| per element,
    S = sum of |w y| over kept pairs; dropped pairs contribute nothing."""
    rng = np.random.default_rng(18 + layout)
    T, K, E, R, H = 60, 8, 32, 8, 48
    idx, w, lay, y, rk = _case(rng, T, K, E, R, H, layout=layout, cap=5)
    part = oracle.combine_partial(idx, E, R, y, w, lay["pair_to_row"], rk["token_rank_row"],
                                  rk["rank_row_to_token"].size)
    out = W.bf16_bits_to_f32(oracle.combine_reduce(part, rk["token_rank_row"], R)).astype(np.float64)
    yf = W.bf16_bits_to_f32(y).astype(np.float64)
    exact = np.zeros((T, H))
    S = np.zeros((T, H))
    p2r = lay["pair_to_row"].reshape(T, K)
    for t in range(T):
        for k in range(K):
            if p2r[t, k] >= 0:
                term = float(w[t, k]) * yf[p2r[t, k]]
                exact[t] += term
                S[t] += np.abs(term)
    assert np.all(np.abs(out - exact) <= 2.0 ** -7 * S + 2.0 ** -8 * np.abs(exact) + 1e-30)
    if layout == oracle.MASKED:
        assert lay["status"][0] > 0


def test_partial_of_fully_dropped_rank_is_positive_zero(oracle_lib):
    """A token in a rank whose pairs were all dropped by the masked capacity
    still has a partial row, and it is +0."""
    idx = np.array([[0, 1], [0, 1], [0, 3]], np.int32)   # E=4, R=2: experts 0,1 -> rank 0
    w = np.ones((3, 2), np.float32)
    lay = oracle.dispatch_layout(idx, 4, 2, oracle.MASKED, capacity=1)
    assert lay["pair_to_row"].tolist() == [0, 1, -1, -1, -1, 3]
    rk = oracle.rank_layout(idx, 4, 2)
    y = W.f32_to_bf16_bits(np.full((lay["row_to_pair"].size, 8), 2.0, np.float32))
    part = np.full((rk["rank_row_to_token"].size, 8), 0xFFFF, np.uint16)
    oracle.combine_partial(idx, 4, 2, y, w, lay["pair_to_row"], rk["token_rank_row"],
                           part.shape[0], out=part)
    trr = rk["token_rank_row"].reshape(3, 2)
    assert np.all(part[trr[1, 0]] == 0) and np.all(part[trr[2, 0]] == 0)
    assert np.all(W.bf16_bits_to_f32(part[trr[0, 0]]) == 4.0)
    assert np.all(W.bf16_bits_to_f32(part[trr[2, 1]]) == 2.0)


def test_expand_takes_the_row_of_the_pairs_rank(oracle_lib):
    """With a distinct byte pattern in every per-rank row, each expanded row
    is the row of its own (token, rank), which the direct-dispatch check
    cannot tell apart (there all rank rows of a token hold the same bytes)."""
    rng = np.random.default_rng(19)
    T, K, E, R, H = 24, 5, 12, 4, 256
    idx = _random_ids(rng, T, K, E)
    lay = oracle.dispatch_layout(idx, E, R, oracle.CONTIGUOUS, align=2)
    rows = lay["row_to_pair"].size
    rk = oracle.rank_layout(idx, E, R)
    qrows = rk["rank_row_to_token"].size
    for quant in (oracle.QUANT_NONE, oracle.QUANT_FP8_UE8M0):
        sx, ss = _sentinel_bufs(qrows, H, quant)
        sx.view(np.uint8)[:] = rng.integers(0, 256, sx.view(np.uint8).shape, dtype=np.uint8)
        if ss is not None:
            ss.view(np.uint8)[:] = rng.integers(0, 256, ss.view(np.uint8).shape, dtype=np.uint8)
        ex, es = _sentinel_bufs(rows, H, quant)
        oracle.expand(idx, E, R, quant, sx, ss, rk["token_rank_row"], lay["pair_to_row"], rows,
                      out_x=ex, out_scale=es)
        trr = rk["token_rank_row"].reshape(T, R)
        written = np.zeros(rows, bool)
        for t in range(T):
            for k in range(K):
                row = lay["pair_to_row"][t * K + k]
                if row < 0:
                    continue
                src = trr[t, idx[t, k] // (E // R)]
                assert np.array_equal(ex[row].view(np.uint8), sx[src].view(np.uint8))
                if ss is not None:
                    assert np.array_equal(es[row].view(np.uint8), ss[src].view(np.uint8))
                written[row] = True
        assert np.all(ex[~written].view(np.uint8) == SENT)


def test_partial_and_reduce_orders(oracle_lib):
    """2^30, -2^30 and 1 sum to 1 only in the order given (any other order
    loses the 1 to fp32 rounding): partial sums go in ascending k, the
    reduction in ascending rank, whatever order the rows are stored in."""
    big = [2.0 ** 30, -(2.0 ** 30), 1.0]
    # partial: one rank holding all three pairs of the token
    idx = np.array([[0, 1, 2]], np.int32)   # E=3, R=1
    w = np.ones((1, 3), np.float32)
    p2r = np.array([2, 0, 1], np.int32)     # rows out of pair order on purpose
    y = np.zeros((3, 2), np.uint16)
    for k in range(3):
        y[p2r[k]] = W.f32_to_bf16_bits(np.full(2, big[k], np.float32))
    part = oracle.combine_partial(idx, 3, 1, y, w, p2r, np.array([0], np.int32), 1)
    assert np.all(W.bf16_bits_to_f32(part) == 1.0)
    # reduce: token in three ranks whose rows are stored out of rank order
    trr = np.array([[2, 0, 1]], np.int32)
    partial = np.zeros((3, 2), np.uint16)
    for r in range(3):
        partial[trr[0, r]] = W.f32_to_bf16_bits(np.full(2, big[r], np.float32))
    out = oracle.combine_reduce(partial, trr, 3)
    assert np.all(W.bf16_bits_to_f32(out) == 1.0)
