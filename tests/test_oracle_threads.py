"""The OpenMP form of the oracle's dispatch and combine (the all-cores CPU
baseline of the benchmark) gives the same bytes as one thread.

Tokens are independent in both functions, so splitting the token loop over
threads must not change any output bit; the layout stays serial.
"""
import numpy as np
import pytest

import oracle
from combine_topk_idx_amd import workloads as W


@pytest.mark.parametrize("quant", [oracle.QUANT_NONE, oracle.QUANT_FP8_F32, oracle.QUANT_FP8_UE8M0,
                                   oracle.QUANT_MXFP8])
@pytest.mark.parametrize("layout", [oracle.CONTIGUOUS, oracle.MASKED])
def test_threads_do_not_change_outputs(quant, layout):
    rng = np.random.default_rng(1000 + 10 * quant + layout)
    T, H, E, K, R = 301, 640, 24, 6, 4
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    idx[rng.random((T, K)) < 0.03] = -1  # some unrouted pairs
    w = rng.random((T, K)).astype(np.float32)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32) * 3)
    align, cap = (4, 1) if layout == oracle.CONTIGUOUS else (1, 60)  # the masked slab drops pairs
    h = oracle.dispatch_layout(idx, E, R, layout, align, cap)
    rows = h["row_to_pair"].size
    y = W.f32_to_bf16_bits(rng.standard_normal((rows, H)).astype(np.float32))
    outs = []
    try:
        for n in (1, 4, 7):
            assert oracle.set_threads(n) == n
            ox, osc, orw = oracle.dispatch(x, h["pair_to_row"], K, quant, rows, topk_w=w,
                                           out_row_weight=np.zeros(rows, np.float32))
            outs.append((ox, osc, orw, oracle.combine(y, w, h["pair_to_row"])))
    finally:
        oracle.set_threads(1)
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert (a is None and b is None) or np.array_equal(a.view(np.uint8), b.view(np.uint8))
