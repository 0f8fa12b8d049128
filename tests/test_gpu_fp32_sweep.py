"""Reachable-input sweep of the fp32-scale quantizer on the GPU.

With fp32 scales the hardware E4M3 conversion sees fl32(x / s), s =
fl32(max(a, 1e-10) / 448), for a block maximum a and any x with |x| <= a:
fp32 values with mantissa bits beyond bf16, rounding ties included.  This
sweep covers every such input the method can produce from bf16 data: every
positive finite bf16 block maximum a (subnormals included), each with every
bf16 magnitude 0..a in both signs in its blocks (element 0 of each block is
a, the other 127 carry the sweep), about 8.4M blocks in chunks.  E4M3 bytes
and scales must equal the oracle's bit for bit.

Every test prints the case it runs before touching the GPU.
"""
import os

import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M
import oracle
from combine_topk_idx_amd import workloads as W

pytestmark = pytest.mark.gpu

H = 7168                 # 56 blocks per token row
PER = 127                # swept values per block (element 0 holds the maximum)
CHUNK_BLOCKS = 1 << 19   # blocks per call


def sweep_chunks(max_blocks=CHUNK_BLOCKS):
    """uint16 blocks [n, 128]: for each positive finite bf16 a (bits 1..0x7F7F,
    increasing in value), element 0 = a and then the bf16 values of
    magnitude 0..a in both signs (value j of a's list: magnitude bits j >> 1,
    sign j & 1), the last block of each a padded with a."""
    A = np.arange(1, 0x7F80, dtype=np.int64)
    m = 2 * (A + 1)
    nb = -(-m // PER)
    cum = np.concatenate([[0], np.cumsum(nb)])
    start = 0
    while start < A.size:
        end = int(np.searchsorted(cum, cum[start] + max_blocks, side="right")) - 1
        end = max(end, start + 1)
        a = A[start:end].astype(np.int32)
        nba = nb[start:end]
        blk_a = np.repeat(a, nba)
        first = np.repeat((cum[start:end] - cum[start]).astype(np.int32), nba)
        bi = np.arange(blk_a.size, dtype=np.int32) - first
        j = bi[:, None] * PER + np.arange(PER, dtype=np.int32)[None, :]
        v = np.where(j < (2 * (blk_a + 1))[:, None], (j >> 1) | ((j & 1) << 15), blk_a[:, None])
        block = np.empty((blk_a.size, 128), np.uint16)
        block[:, 0] = blk_a
        block[:, 1:] = v
        yield block
        start = end


def _threads():
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = int(env) if env.strip().isdigit() and int(env) > 0 else len(os.sched_getaffinity(0))
    return min(n, 16)


def test_fp32_scale_reachable_inputs():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()
    oracle._load()
    oracle.set_threads(_threads())
    total = 0
    try:
        for ci, blocks in enumerate(sweep_chunks()):
            n = blocks.shape[0]
            T = -(-n * 128 // H)
            x = np.zeros(T * H, np.uint16)
            x[:n * 128] = blocks.reshape(-1)
            x = x.reshape(T, H)
            print(f"\n[case] fp32-scale reachable-input sweep chunk {ci}: {n} blocks, T={T}, "
                  f"maxima {int(blocks[0, 0]):#06x}..{int(blocks[-1, 0]):#06x}", flush=True)
            cfg = M.MoeConfig(max_tokens=T, hidden=H, num_experts=1, num_topk=1, num_ranks=1,
                              layout=M.LAYOUT_CONTIGUOUS, align=1, quant=M.QUANT_FP8_F32)
            bufs = M.DispatchBuffers(cfg)
            bufs.out_x.fill_(0xA5)
            bufs.out_scale.view(torch.uint8).fill_(0xA5)
            d_idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
            d_x = torch.from_numpy(x.view(np.int16)).cuda()
            M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace)
            M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale)
            torch.cuda.synchronize()
            gx = bufs.out_x.cpu().numpy()
            gs = bufs.out_scale.cpu().numpy().view(np.uint32)
            ox, osc, _ = oracle.dispatch(x, np.arange(T, dtype=np.int32), 1, oracle.QUANT_FP8_F32, T)
            if not np.array_equal(gx, ox):
                bad = np.nonzero(gx.reshape(-1) != ox.reshape(-1))[0]
                t, c = bad[0] // H, bad[0] % H
                raise AssertionError(f"chunk {ci}: {bad.size} E4M3 bytes differ; first at token {t} channel {c}: "
                                     f"x {int(x[t, c]):#06x} block max {int(x[t, c - c % 128]):#06x} "
                                     f"gpu {int(gx[t, c]):#04x} oracle {int(ox[t, c]):#04x}")
            assert np.array_equal(gs, osc.view(np.uint32)), f"chunk {ci}: scales differ"
            total += n
            del bufs, d_x, d_idx
    finally:
        oracle.set_threads(1)
    assert total == int(sum(-(-2 * (a + 1) // PER) for a in range(1, 0x7F80)))
    print(f"[ok] fp32-scale reachable-input sweep: {total} blocks bit-exact", flush=True)
