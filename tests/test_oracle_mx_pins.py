"""Pins for the oracle's MXFP8 (1x32, OCP MX) dispatch (no GPU needed).

Checked against a hand-worked fixture, an exhaustive sweep of the shared
exponent over every positive finite bf16 value (against numpy's frexp and the
defining inequality), torch's float8_e4m3fn / float8_e8m0fnu casts of the
same formulas on random rows with outliers, zero blocks and subnormals, and
the element error bound.
"""
import json
import os

import numpy as np
import torch

import oracle
from combine_topk_idx_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_mx_golden_blocks(oracle_lib):
    with open(os.path.join(GOLDEN, "mxfp8_blocks_H128.json")) as f:
        g = json.load(f)
    x = np.array([[int(v, 16) for v in g["x_bf16_bits"]]], np.uint16)
    out_x, out_s, _ = oracle.dispatch(x, np.array([0], np.int32), 1, oracle.QUANT_MXFP8, 1)
    assert out_x[0].tolist() == [int(v, 16) for v in g["q_e4m3"]]
    assert out_s[0].tolist() == [int(v, 16) for v in g["scale_e8m0"]]


def test_mx_exponent_exhaustive_over_bf16(oracle_lib):
    bits = np.arange(1, 0x7F80, dtype=np.uint32)           # every positive finite bf16
    a = (bits << 16).view(np.float32)
    a = np.concatenate([a, np.float32([1e-10])])
    s = oracle.mx_exponent(a)
    _, e = np.frexp(a.astype(np.float64))                    # a = m 2^e, m in [0.5, 1)
    assert np.array_equal(s, e - 1 - 8)
    lo = np.ldexp(1.0, s + 8)
    assert np.all(lo <= a) and np.all(a < 2 * lo)


def _torch_mx(x_bits, floor=1e-10):
    """The MX conversion written with torch ops: float32 block maxima, the
    exponent from torch.frexp, power-of-two scaling, clamp, e4m3fn cast."""
    x = torch.from_numpy(W.bf16_bits_to_f32(x_bits))
    T, H = x.shape
    xb = x.view(T, H // 32, 32)
    a = xb.abs().amax(dim=2).clamp_min(floor)
    _, e = torch.frexp(a)
    s = (e - 1 - 8).to(torch.int32)
    scaled = xb * torch.pow(2.0, -s.to(torch.float32)).unsqueeze(2)
    q = scaled.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).view(T, H).numpy()
    scale = torch.pow(2.0, s.to(torch.float32)).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    return q, scale, s.numpy()


def _mx_rows(rng, T, H):
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[rng.random(T) < 0.1] *= 1e4                          # outlier rows
    x[:, 32:64][rng.random(T) < 0.2] = 0.0                 # zero blocks
    x[rng.random((T, H)) < 0.01] *= 1e-38                  # subnormal-range values
    x[rng.random(T) < 0.05, 5] = 3.0e38                    # near the top of the range
    x[rng.random(T) < 0.05] *= 1e-9                        # blocks near the amax floor
    return W.f32_to_bf16_bits(x)


def test_mx_dispatch_vs_torch(oracle_lib):
    rng = np.random.default_rng(31)
    T, H = 300, 512
    x = _mx_rows(rng, T, H)
    p2r = np.arange(T, dtype=np.int32)
    out_x, out_s, _ = oracle.dispatch(x, p2r, 1, oracle.QUANT_MXFP8, T)
    q, scale, _ = _torch_mx(x)
    assert np.array_equal(out_x, q)
    assert np.array_equal(out_s, scale)


def test_mx_saturation_and_error_bound(oracle_lib):
    """Per block 256 <= a 2^-s < 512; elements whose |x| 2^-s exceeds 448
    decode to +-448 2^s, and every other element is within half an E4M3 step
    of x (relative 2^-4 for normal results, absolute 2^-10 2^s below)."""
    rng = np.random.default_rng(32)
    T, H = 200, 256
    x = _mx_rows(rng, T, H)
    out_x, out_s, _ = oracle.dispatch(x, np.arange(T, dtype=np.int32), 1, oracle.QUANT_MXFP8, T)
    xf = W.bf16_bits_to_f32(x).astype(np.float64).reshape(T, H // 32, 32)
    s = out_s.astype(np.int64) - 127
    a = np.maximum(np.abs(xf).max(axis=2), 1e-10)
    r = a * np.ldexp(1.0, -s)
    assert np.all((256 <= r) & (r < 512))
    table = np.array([np.nan if c & 0x7F == 0x7F else (-1 if c & 0x80 else 1) * oracle.e4m3_value(c & 0x7F)
                      for c in range(256)])
    dq = table[out_x].reshape(T, H // 32, 32)
    dq = dq * np.ldexp(1.0, s)[:, :, None]
    scaled = np.abs(xf) * np.ldexp(1.0, -s)[:, :, None]
    sat = scaled > 448
    assert np.all(np.abs(dq[sat]) == 448 * np.ldexp(1.0, s)[:, :, None].repeat(32, 2)[sat])
    err = np.abs(dq - xf)[~sat]
    bound = np.maximum(2.0 ** -4 * np.abs(xf), 2.0 ** -10 * np.ldexp(1.0, s)[:, :, None].repeat(32, 2))[~sat]
    assert np.all(err <= bound)
    assert sat.any()


def test_mx_rows_copied_to_every_kept_row(oracle_lib):
    rng = np.random.default_rng(33)
    T, K, H = 20, 3, 128
    x = _mx_rows(rng, T, H)
    p2r = rng.permutation(T * K).astype(np.int32)
    p2r[rng.random(T * K) < 0.2] = -1
    rows = T * K
    ox = np.full((rows, H), 0xA5, np.uint8)
    osc = np.full((rows, H // 32), 0xA5, np.uint8)
    oracle.dispatch(x, p2r, K, oracle.QUANT_MXFP8, rows, out_x=ox, out_scale=osc)
    q, scale, _ = _torch_mx(x)
    for p in range(T * K):
        r = p2r[p]
        if r >= 0:
            assert np.array_equal(ox[r], q[p // K]) and np.array_equal(osc[r], scale[p // K])
    untouched = np.setdiff1d(np.arange(rows), p2r[p2r >= 0])
    assert np.all(ox[untouched] == 0xA5) and np.all(osc[untouched] == 0xA5)
