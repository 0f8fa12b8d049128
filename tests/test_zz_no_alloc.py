"""moe_dispatch_layout_noalloc (the layout with the library's static per-GPU
workspace) against moe_dispatch_layout with a caller workspace, through the
C ABI: every handle array bit for bit, on consecutive calls that share the
static array (the second and third with fewer tokens), in the schedules that
use the workspace (more than 65,536 pairs, or more than 512 experts) and in
the one-launch schedule that does not.

Every test prints the case it runs before touching the GPU.
"""
import numpy as np
import pytest
import torch

import combine_topk_idx_amd as M

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    M.library()


def _ids(rng, T, E, K):
    """Distinct experts per token (base + k * stride mod E, stride coprime to
    E), a few unrouted (-1) and invalid ids."""
    strides = np.array([s for s in range(1, E) if np.gcd(s, E) == 1])
    base = rng.integers(0, E, T)
    step = rng.choice(strides, T)
    idx = ((base[:, None] + np.arange(K)[None, :] * step[:, None]) % E).astype(np.int32)
    idx[rng.random((T, K)) < 0.01] = -1
    idx[rng.random((T, K)) < 0.001] = E + 3
    return idx


def _fresh_handle(cfg):
    h = M.Handle(cfg, "cuda")
    for t in h.tensors().values():
        t.view(torch.uint8).fill_(0xA5)
    return h


@pytest.mark.parametrize("E,K,layout,align,cap,Ts", [
    (256, 8, M.LAYOUT_CONTIGUOUS, 128, 1, (40000, 15000, 700)),   # 320,000 pairs, then 120,000, then one launch
    (600, 4, M.LAYOUT_MASKED, 1, 96, (9000, 5000, 20)),           # > 512 experts: workspace at any size
    (2048, 2, M.LAYOUT_CONTIGUOUS, 1, 1, (983008, 300000, 70000)),  # the largest call the array holds
])
def test_noalloc_matches_workspace_layout(E, K, layout, align, cap, Ts):
    cfg = M.MoeConfig(max_tokens=max(Ts), hidden=128, num_experts=E, num_topk=K, num_ranks=8 if E % 8 == 0 else 4,
                      layout=layout, align=align, capacity=cap)
    ws = torch.empty(max(M.moe_workspace_bytes(cfg), 4), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(E * 31 + K)
    for i, T in enumerate(Ts):
        print(f"\n[case] noalloc layout E={E} K={K} layout={layout} T={T} (call {i + 1} of {len(Ts)})", flush=True)
        d_idx = torch.from_numpy(_ids(rng, T, E, K)).cuda()
        ref, got = _fresh_handle(cfg), _fresh_handle(cfg)
        M.moe_dispatch_layout(cfg, T, d_idx, ref, ws)
        M.moe_dispatch_layout_noalloc(cfg, T, d_idx, got)
        torch.cuda.synchronize()
        for name, a in ref.tensors().items():
            b = got.tensors()[name]
            assert torch.equal(a, b), f"{name} differs (call {i + 1}, T={T})"


def test_noalloc_rejects_too_many_pairs():
    cfg = M.MoeConfig(max_tokens=1 << 20, hidden=128, num_experts=2048, num_topk=2, num_ranks=8)
    print("\n[case] noalloc layout: 983,009 tokens x 2 exceed the static workspace", flush=True)
    h = M.Handle(cfg, "cuda")
    d_idx = torch.zeros((983009, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(M.MoeError) as e:
        M.moe_dispatch_layout_noalloc(cfg, 983009, d_idx, h)
    assert e.value.code == M.MOE_ERR_CAPACITY
