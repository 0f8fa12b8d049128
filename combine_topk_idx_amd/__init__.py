"""MI355X (gfx950) MoE token dispatch / combine.

A thin ctypes binding over ``libmoe_dispatch.so`` (HIP kernels behind the C
ABI declared in ``include/moe_dispatch.h``).  The Python functions carry the
same names as the C entry points and only marshal arguments: torch tensors
supply device memory and the current HIP stream, and every step of the path
runs in the library's kernels.  There is no fallback: if the library is not
built, or the process has no GPU, the calls raise.

Typical use (prefill, FP8 with UE8M0 scales)::

    cfg = MoeConfig(max_tokens=8192, hidden=7168, num_experts=256, num_topk=8,
                    num_ranks=8, layout=LAYOUT_CONTIGUOUS, align=128,
                    quant=QUANT_FP8_UE8M0)
    bufs = DispatchBuffers(cfg, device="cuda")
    moe_dispatch_layout(cfg, T, topk_idx, bufs.handle, bufs.workspace)
    moe_dispatch(cfg, T, x, None, bufs.handle, bufs.out_x, bufs.out_scale)
    ...  # experts write y in the dispatched layout
    moe_combine(cfg, T, y, topk_w, bufs.handle, out)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_dispatch.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_CAPACITY = 2
MOE_ERR_UNSUPPORTED = 3
MOE_ERR_HIP = 4

LAYOUT_CONTIGUOUS = 0
LAYOUT_MASKED = 1
QUANT_NONE = 0
QUANT_FP8_F32 = 1
QUANT_FP8_UE8M0 = 2
QUANT_MXFP8 = 3


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {moe_status_str(code)} ({code})")
        self.code = code


class MoeConfig(ctypes.Structure):
    """moe_config_t."""

    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_tokens", "hidden", "num_experts", "num_topk", "num_ranks",
        "layout", "align", "capacity", "quant", "num_cus")]

    def __init__(self, max_tokens, hidden, num_experts, num_topk, num_ranks,
                 layout=LAYOUT_CONTIGUOUS, align=1, capacity=1, quant=QUANT_NONE, num_cus=0):
        super().__init__(max_tokens, hidden, num_experts, num_topk, num_ranks,
                         layout, align, capacity, quant, num_cus)


class MoeHandle(ctypes.Structure):
    """moe_handle_t: device pointers of the handle arrays."""

    _fields_ = [(n, ctypes.c_void_p) for n in (
        "expert_count", "recv_count", "expert_offset", "rank_offset",
        "pair_to_row", "row_to_pair", "status")]


class MoeRankHandle(ctypes.Structure):
    """moe_rank_handle_t: device pointers of the per-rank layout arrays."""

    _fields_ = [(n, ctypes.c_void_p) for n in (
        "rank_token_count", "rank_token_offset", "token_rank_row", "rank_row_to_token")]


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m combine_topk_idx_amd.build` "
            "(hipcc, gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp, hp = ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeHandle)
    lib.moe_rows_capacity.argtypes = [cfgp]
    lib.moe_rows_capacity.restype = sz
    lib.moe_workspace_bytes.argtypes = [cfgp]
    lib.moe_workspace_bytes.restype = sz
    lib.moe_config_check.argtypes = [cfgp]
    lib.moe_config_check.restype = ctypes.c_int
    lib.moe_dispatch_layout.argtypes = [cfgp, i32, P, hp, P, sz, P]
    lib.moe_dispatch_layout.restype = ctypes.c_int
    lib.moe_dispatch_layout_noalloc.argtypes = [cfgp, i32, P, hp, P]
    lib.moe_dispatch_layout_noalloc.restype = ctypes.c_int
    lib.moe_dispatch.argtypes = [cfgp, i32, P, P, hp, P, P, P, P]
    lib.moe_dispatch.restype = ctypes.c_int
    lib.moe_dispatch_fused.argtypes = [cfgp, i32, P, P, P, hp, P, sz, P, P, P, P]
    lib.moe_dispatch_fused.restype = ctypes.c_int
    lib.moe_combine.argtypes = [cfgp, i32, P, P, hp, P, P]
    lib.moe_combine.restype = ctypes.c_int
    rhp = ctypes.POINTER(MoeRankHandle)
    lib.moe_rank_rows_capacity.argtypes = [cfgp]
    lib.moe_rank_rows_capacity.restype = sz
    lib.moe_rank_layout.argtypes = [cfgp, i32, P, rhp, P]
    lib.moe_rank_layout.restype = ctypes.c_int
    lib.moe_dispatch_dedup.argtypes = [cfgp, i32, P, rhp, P, P, P]
    lib.moe_dispatch_dedup.restype = ctypes.c_int
    lib.moe_expand.argtypes = [cfgp, i32, P, P, P, rhp, hp, P, P, P]
    lib.moe_expand.restype = ctypes.c_int
    lib.moe_combine_partial.argtypes = [cfgp, i32, P, P, P, hp, rhp, P, P]
    lib.moe_combine_partial.restype = ctypes.c_int
    lib.moe_combine_reduce.argtypes = [cfgp, i32, P, rhp, P, P]
    lib.moe_combine_reduce.restype = ctypes.c_int
    lib.moe_row_expert.argtypes = [cfgp, hp, P, P]
    lib.moe_row_expert.restype = ctypes.c_int
    lib.moe_repack_rows_capacity.argtypes = [cfgp, i32]
    lib.moe_repack_rows_capacity.restype = sz
    lib.moe_repack_masked_to_contiguous.argtypes = [cfgp, i32, hp, P, P, P, P, P, P, P]
    lib.moe_repack_masked_to_contiguous.restype = ctypes.c_int
    lib.moe_repack_contiguous_to_masked.argtypes = [cfgp, hp, P, P, P, P]
    lib.moe_repack_contiguous_to_masked.restype = ctypes.c_int
    lib.moe_scale_words.argtypes = [cfgp]
    lib.moe_scale_words.restype = sz
    lib.moe_scales_mn_major.argtypes = [cfgp, i32, P, P, P]
    lib.moe_scales_mn_major.restype = ctypes.c_int
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library() -> ctypes.CDLL:
    """The loaded libmoe_dispatch.so (raises if it is not built)."""
    return _load()


def moe_status_str(code: int) -> str:
    return _load().moe_status_str(code).decode()


# Size queries depend on the config's values only; per-call marshalling asks
# for them on every call, so they are remembered per config value.
_size_cache: dict = {}


def _cached_size(fn: str, cfg: MoeConfig, *extra) -> int:
    key = (fn, bytes(cfg)) + extra
    v = _size_cache.get(key)
    if v is None:
        if len(_size_cache) > 4096:
            _size_cache.clear()
        v = int(getattr(_load(), fn)(ctypes.byref(cfg), *extra))
        _size_cache[key] = v
    return v


def moe_rows_capacity(cfg: MoeConfig) -> int:
    return _cached_size("moe_rows_capacity", cfg)


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    return int(_load().moe_workspace_bytes(ctypes.byref(cfg)))


def moe_config_check(cfg: MoeConfig) -> int:
    return int(_load().moe_config_check(ctypes.byref(cfg)))


def moe_rank_rows_capacity(cfg: MoeConfig) -> int:
    return _cached_size("moe_rank_rows_capacity", cfg)


# ---- marshalling helpers ----------------------------------------------------

def _ptr(t: Optional[torch.Tensor], dtype_bytes: Optional[int] = None,
         min_elems: int = 0, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dtype_bytes is not None and t.element_size() != dtype_bytes:
        raise ValueError(f"{name}: expected {dtype_bytes}-byte elements, got {t.dtype}")
    if t.numel() < min_elems:
        raise ValueError(f"{name}: {t.numel()} elements < required {min_elems}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, code: int):
    if code != MOE_OK:
        raise MoeError(fn, code)


class Handle:
    """Device arrays of one dispatch handle (moe_handle_t), allocated by torch."""

    def __init__(self, cfg: MoeConfig, device="cuda"):
        E, R = cfg.num_experts, cfg.num_ranks
        rows = moe_rows_capacity(cfg)
        if rows == 0 and moe_config_check(cfg) != MOE_OK:
            raise MoeError("moe_rows_capacity", moe_config_check(cfg))
        z = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=device)
        self.expert_count = z(E)
        self.recv_count = z(E)
        self.expert_offset = z(E + 1)
        self.rank_offset = z(R + 1)
        self.pair_to_row = z(cfg.max_tokens * cfg.num_topk)
        self.row_to_pair = z(rows)
        self.status = z(2)
        self.c = MoeHandle(*(t.data_ptr() for t in (
            self.expert_count, self.recv_count, self.expert_offset, self.rank_offset,
            self.pair_to_row, self.row_to_pair, self.status)))

    def tensors(self) -> dict:
        return {k: getattr(self, k) for k in (
            "expert_count", "recv_count", "expert_offset", "rank_offset",
            "pair_to_row", "row_to_pair", "status")}


class DispatchBuffers:
    """Handle, workspace and dispatched-activation buffers sized for a config."""

    def __init__(self, cfg: MoeConfig, device="cuda", row_weight: bool = False):
        self.cfg = cfg
        self.rows = moe_rows_capacity(cfg)
        self.handle = Handle(cfg, device)
        self.workspace = torch.empty(max(moe_workspace_bytes(cfg), 4), dtype=torch.uint8, device=device)
        H = cfg.hidden
        if cfg.quant == QUANT_NONE:
            self.out_x = torch.empty((self.rows, H), dtype=torch.int16, device=device)
            self.out_scale = None
        else:
            self.out_x = torch.empty((self.rows, H), dtype=torch.uint8, device=device)
            self.out_scale = _scale_buffer(cfg, self.rows, device)
        self.out_row_weight = (torch.empty(self.rows, dtype=torch.float32, device=device)
                               if row_weight else None)


# ---- entry points -----------------------------------------------------------

def moe_dispatch_layout(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, handle: Handle,
                        workspace: torch.Tensor, stream=None) -> None:
    """Counts, offsets, stable slots and both maps from int32 topk_idx [T, K]."""
    lib = _load()
    K = cfg.num_topk
    idx = _ptr(topk_idx, 4, num_tokens * K, "topk_idx") if num_tokens > 0 else None
    ws = _ptr(workspace, None, 0, "workspace")
    _check("moe_dispatch_layout", lib.moe_dispatch_layout(
        ctypes.byref(cfg), int(num_tokens), idx, ctypes.byref(handle.c), ws,
        workspace.numel() * workspace.element_size(), _stream(stream)))


def moe_dispatch_layout_noalloc(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, handle: Handle,
                                stream=None) -> None:
    """moe_dispatch_layout with the library's static per-GPU workspace (no
    allocation; calls that overlap on one GPU race)."""
    lib = _load()
    K = cfg.num_topk
    idx = _ptr(topk_idx, 4, num_tokens * K, "topk_idx") if num_tokens > 0 else None
    _check("moe_dispatch_layout_noalloc", lib.moe_dispatch_layout_noalloc(
        ctypes.byref(cfg), int(num_tokens), idx, ctypes.byref(handle.c), _stream(stream)))


def _dispatch_ptrs(cfg, num_tokens, x, topk_w, out_x, out_scale, out_row_weight):
    rows = moe_rows_capacity(cfg)
    H, K = cfg.hidden, cfg.num_topk
    xp = _ptr(x, 2, num_tokens * H, "x") if num_tokens > 0 else None
    wp = _ptr(topk_w, 4, num_tokens * K if out_row_weight is not None else 0, "topk_w")
    ob = 2 if cfg.quant == QUANT_NONE else 1
    op = _ptr(out_x, None, rows * H * ob // out_x.element_size(), "out_x")
    sp = _scale_ptr(cfg, out_scale, rows, "out_scale")
    rp = _ptr(out_row_weight, 4, rows, "out_row_weight")
    return xp, wp, op, sp, rp


def moe_dispatch(cfg: MoeConfig, num_tokens: int, x: torch.Tensor, topk_w: Optional[torch.Tensor],
                 handle: Handle, out_x: torch.Tensor, out_scale: Optional[torch.Tensor] = None,
                 out_row_weight: Optional[torch.Tensor] = None, stream=None) -> None:
    """Permute (and FP8-quantize when cfg.quant says so) bf16 rows x [T, H]."""
    lib = _load()
    xp, wp, op, sp, rp = _dispatch_ptrs(cfg, num_tokens, x, topk_w, out_x, out_scale, out_row_weight)
    _check("moe_dispatch", lib.moe_dispatch(
        ctypes.byref(cfg), int(num_tokens), xp, wp, ctypes.byref(handle.c), op, sp, rp,
        _stream(stream)))


def moe_dispatch_fused(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, x: torch.Tensor,
                       topk_w: Optional[torch.Tensor], handle: Handle, workspace: torch.Tensor,
                       out_x: torch.Tensor, out_scale: Optional[torch.Tensor] = None,
                       out_row_weight: Optional[torch.Tensor] = None, stream=None) -> None:
    """Layout + dispatch in one call (one launch for small batches)."""
    lib = _load()
    idx = _ptr(topk_idx, 4, num_tokens * cfg.num_topk, "topk_idx") if num_tokens > 0 else None
    ws = _ptr(workspace, None, 0, "workspace")
    xp, wp, op, sp, rp = _dispatch_ptrs(cfg, num_tokens, x, topk_w, out_x, out_scale, out_row_weight)
    _check("moe_dispatch_fused", lib.moe_dispatch_fused(
        ctypes.byref(cfg), int(num_tokens), idx, xp, wp, ctypes.byref(handle.c), ws,
        workspace.numel() * workspace.element_size(), op, sp, rp, _stream(stream)))


def moe_combine(cfg: MoeConfig, num_tokens: int, y: torch.Tensor, topk_w: torch.Tensor,
                handle: Handle, out: torch.Tensor, stream=None) -> None:
    """out[t] = bf16(sum_k w[t,k] * y[row(t,k)]) with fp32 accumulation."""
    lib = _load()
    rows = moe_rows_capacity(cfg)
    H, K = cfg.hidden, cfg.num_topk
    if num_tokens == 0:
        yp = wp = op = None
    else:
        yp = _ptr(y, 2, rows * H, "y")
        wp = _ptr(topk_w, 4, num_tokens * K, "topk_w")
        op = _ptr(out, 2, num_tokens * H, "out")
    _check("moe_combine", lib.moe_combine(
        ctypes.byref(cfg), int(num_tokens), yp, wp, ctypes.byref(handle.c), op, _stream(stream)))


# ---- per-rank deduplicated exchange -------------------------------------------

class RankHandle:
    """Device arrays of one per-rank layout (moe_rank_handle_t), allocated by torch."""

    def __init__(self, cfg: MoeConfig, device="cuda"):
        R = cfg.num_ranks
        rows = moe_rank_rows_capacity(cfg)
        if rows == 0 and cfg.max_tokens > 0:
            code = moe_config_check(cfg)
            raise MoeError("moe_rank_rows_capacity", code if code != MOE_OK else MOE_ERR_UNSUPPORTED)
        z = lambda n: torch.empty(max(int(n), 1), dtype=torch.int32, device=device)
        self.rank_token_count = z(R)
        self.rank_token_offset = z(R + 1)
        self.token_rank_row = z(cfg.max_tokens * R)
        self.rank_row_to_token = z(rows)
        self.c = MoeRankHandle(*(t.data_ptr() for t in (
            self.rank_token_count, self.rank_token_offset, self.token_rank_row,
            self.rank_row_to_token)))

    def tensors(self) -> dict:
        return {k: getattr(self, k) for k in (
            "rank_token_count", "rank_token_offset", "token_rank_row", "rank_row_to_token")}


class DedupBuffers:
    """Per-rank layout and the per-rank row buffers (send rows, their scales,
    and bf16 partial sums) sized for a config."""

    def __init__(self, cfg: MoeConfig, device="cuda", partial: bool = True):
        self.cfg = cfg
        self.rows = moe_rank_rows_capacity(cfg)
        self.handle = RankHandle(cfg, device)
        H = cfg.hidden
        nb = H // 128
        n = max(self.rows, 1)
        if cfg.quant == QUANT_NONE:
            self.send_x = torch.empty((n, H), dtype=torch.int16, device=device)
            self.send_scale = None
        else:
            self.send_x = torch.empty((n, H), dtype=torch.uint8, device=device)
            self.send_scale = _scale_buffer(cfg, n, device)
        self.partial = torch.empty((n, H), dtype=torch.int16, device=device) if partial else None


_ELEM_BYTES = {torch.float32: 4, torch.int32: 4, torch.uint8: 1}


def _scale_layout(cfg):
    """(dtype, columns) of a row's scales: fp32 per 128 channels, packed UE8M0
    words (4 blocks each), or MX E8M0 bytes per 32 channels; None for bf16."""
    nb = cfg.hidden // 128
    return {QUANT_FP8_F32: (torch.float32, nb), QUANT_FP8_UE8M0: (torch.int32, (nb + 3) // 4),
            QUANT_MXFP8: (torch.uint8, cfg.hidden // 32)}.get(cfg.quant)


def _scale_buffer(cfg, rows, device):
    dt, cols = _scale_layout(cfg)
    return torch.empty((rows, cols), dtype=dt, device=device)


def _scale_ptr(cfg, t, rows, name):
    lay = _scale_layout(cfg)
    if lay is None:
        if t is not None:
            raise ValueError(f"{name} must be None without FP8 quantization")
        return None
    dt, cols = lay
    return _ptr(t, _ELEM_BYTES[dt], rows * cols, name)


def moe_rank_layout(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, rank_handle: RankHandle,
                    stream=None) -> None:
    """Tokens per rank and the (token, rank) <-> row maps from topk_idx [T, K]."""
    lib = _load()
    idx = _ptr(topk_idx, 4, num_tokens * cfg.num_topk, "topk_idx") if num_tokens > 0 else None
    _check("moe_rank_layout", lib.moe_rank_layout(
        ctypes.byref(cfg), int(num_tokens), idx, ctypes.byref(rank_handle.c), _stream(stream)))


def moe_dispatch_dedup(cfg: MoeConfig, num_tokens: int, x: torch.Tensor, rank_handle: RankHandle,
                       send_x: torch.Tensor, send_scale: Optional[torch.Tensor] = None,
                       stream=None) -> None:
    """Each token row (quantized as by moe_dispatch) once per rank it is in."""
    lib = _load()
    rows = moe_rank_rows_capacity(cfg)
    H = cfg.hidden
    xp = _ptr(x, 2, num_tokens * H, "x") if num_tokens > 0 else None
    ob = 2 if cfg.quant == QUANT_NONE else 1
    op = _ptr(send_x, None, rows * H * ob // send_x.element_size(), "send_x")
    sp = _scale_ptr(cfg, send_scale, rows, "send_scale")
    _check("moe_dispatch_dedup", lib.moe_dispatch_dedup(
        ctypes.byref(cfg), int(num_tokens), xp, ctypes.byref(rank_handle.c), op, sp, _stream(stream)))


def moe_expand(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, send_x: torch.Tensor,
               send_scale: Optional[torch.Tensor], rank_handle: RankHandle, handle: Handle,
               out_x: torch.Tensor, out_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    """Receive-side expansion of per-rank rows into the per-expert layout."""
    lib = _load()
    rows, qrows = moe_rows_capacity(cfg), moe_rank_rows_capacity(cfg)
    H = cfg.hidden
    ob = 2 if cfg.quant == QUANT_NONE else 1
    if num_tokens > 0:
        idx = _ptr(topk_idx, 4, num_tokens * cfg.num_topk, "topk_idx")
        sx = _ptr(send_x, None, qrows * H * ob // send_x.element_size(), "send_x")
        ss = _scale_ptr(cfg, send_scale, qrows, "send_scale")
    else:
        idx = sx = ss = None
    op = _ptr(out_x, None, rows * H * ob // out_x.element_size(), "out_x")
    sp = _scale_ptr(cfg, out_scale, rows, "out_scale")
    _check("moe_expand", lib.moe_expand(
        ctypes.byref(cfg), int(num_tokens), idx, sx, ss, ctypes.byref(rank_handle.c),
        ctypes.byref(handle.c), op, sp, _stream(stream)))


def moe_combine_partial(cfg: MoeConfig, num_tokens: int, topk_idx: torch.Tensor, y: torch.Tensor,
                        topk_w: torch.Tensor, handle: Handle, rank_handle: RankHandle,
                        partial: torch.Tensor, stream=None) -> None:
    """bf16 partial sums per (token, rank) of the weighted expert outputs."""
    lib = _load()
    rows, qrows = moe_rows_capacity(cfg), moe_rank_rows_capacity(cfg)
    H, K = cfg.hidden, cfg.num_topk
    if num_tokens == 0:
        idx = yp = wp = pp = None
    else:
        idx = _ptr(topk_idx, 4, num_tokens * K, "topk_idx")
        yp = _ptr(y, 2, rows * H, "y")
        wp = _ptr(topk_w, 4, num_tokens * K, "topk_w")
        pp = _ptr(partial, 2, qrows * H, "partial")
    _check("moe_combine_partial", lib.moe_combine_partial(
        ctypes.byref(cfg), int(num_tokens), idx, yp, wp, ctypes.byref(handle.c),
        ctypes.byref(rank_handle.c), pp, _stream(stream)))


def moe_combine_reduce(cfg: MoeConfig, num_tokens: int, partial: torch.Tensor,
                       rank_handle: RankHandle, out: torch.Tensor, stream=None) -> None:
    """out[t] = bf16(sum over ranks ascending of the token's partial rows)."""
    lib = _load()
    qrows = moe_rank_rows_capacity(cfg)
    H = cfg.hidden
    if num_tokens == 0:
        pp = op = None
    else:
        pp = _ptr(partial, 2, qrows * H, "partial")
        op = _ptr(out, 2, num_tokens * H, "out")
    _check("moe_combine_reduce", lib.moe_combine_reduce(
        ctypes.byref(cfg), int(num_tokens), pp, ctypes.byref(rank_handle.c), op, _stream(stream)))


# ---- adapters for grouped-GEMM consumers --------------------------------------

def moe_repack_rows_capacity(cfg: MoeConfig, align: int) -> int:
    return int(_load().moe_repack_rows_capacity(ctypes.byref(cfg), int(align)))


def moe_scale_words(cfg: MoeConfig) -> int:
    return int(_load().moe_scale_words(ctypes.byref(cfg)))


def moe_row_expert(cfg: MoeConfig, handle: Handle, row_expert: torch.Tensor, stream=None) -> None:
    """Expert index of every dispatched row (-1 for rows holding no pair)."""
    lib = _load()
    rp = _ptr(row_expert, 4, moe_rows_capacity(cfg), "row_expert")
    _check("moe_row_expert", lib.moe_row_expert(ctypes.byref(cfg), ctypes.byref(handle.c), rp, _stream(stream)))


def moe_repack_masked_to_contiguous(cfg: MoeConfig, align: int, handle: Handle, x: torch.Tensor,
                                    scale: Optional[torch.Tensor], out_x: torch.Tensor,
                                    out_scale: Optional[torch.Tensor], out_expert_offset: torch.Tensor,
                                    out_row_expert: torch.Tensor, stream=None) -> None:
    """Masked slab rows (+ scales) -> contiguous segments padded to `align`."""
    lib = _load()
    rows, crows = moe_rows_capacity(cfg), moe_repack_rows_capacity(cfg, align)
    H = cfg.hidden
    ob = 2 if cfg.quant == QUANT_NONE else 1
    xp = _ptr(x, None, rows * H * ob // x.element_size(), "x")
    sp = _scale_ptr(cfg, scale, rows, "scale")
    op = _ptr(out_x, None, crows * H * ob // out_x.element_size(), "out_x")
    osp = _scale_ptr(cfg, out_scale, crows, "out_scale")
    offp = _ptr(out_expert_offset, 4, cfg.num_experts + 1, "out_expert_offset")
    rep = _ptr(out_row_expert, 4, crows, "out_row_expert")
    _check("moe_repack_masked_to_contiguous", lib.moe_repack_masked_to_contiguous(
        ctypes.byref(cfg), int(align), ctypes.byref(handle.c), xp, sp, op, osp, offp, rep, _stream(stream)))


def moe_repack_contiguous_to_masked(cfg: MoeConfig, handle: Handle, expert_offset: torch.Tensor,
                                    y: torch.Tensor, y_masked: torch.Tensor, stream=None) -> None:
    """Contiguous bf16 expert outputs -> the masked slab."""
    lib = _load()
    rows = moe_rows_capacity(cfg)
    H = cfg.hidden
    offp = _ptr(expert_offset, 4, cfg.num_experts + 1, "expert_offset")
    yp = _ptr(y, 2, 0, "y")
    mp = _ptr(y_masked, 2, rows * H, "y_masked")
    _check("moe_repack_contiguous_to_masked", lib.moe_repack_contiguous_to_masked(
        ctypes.byref(cfg), ctypes.byref(handle.c), offp, yp, mp, _stream(stream)))


def moe_scales_mn_major(cfg: MoeConfig, rows: int, scale: torch.Tensor, scale_mn: torch.Tensor,
                        stream=None) -> None:
    """Row-major scale words [rows, S] -> MN-major [S, ld], ld = rows rounded up to 4."""
    lib = _load()
    S = moe_scale_words(cfg)
    ld = (int(rows) + 3) // 4 * 4
    sp = _ptr(scale, None, 0, "scale")
    if scale.numel() * scale.element_size() < rows * S * 4:
        raise ValueError("scale: fewer than rows * S words")
    op = _ptr(scale_mn, None, 0, "scale_mn")
    if scale_mn.numel() * scale_mn.element_size() < S * ld * 4:
        raise ValueError("scale_mn: fewer than S * ld words")
    _check("moe_scales_mn_major", lib.moe_scales_mn_major(ctypes.byref(cfg), int(rows), sp, op, _stream(stream)))
