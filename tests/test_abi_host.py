"""Host-side tests of the C ABI (no GPU needed).

The library is loaded with ctypes and called only in ways that are decided
on the host before any HIP call: every argument error, the size queries, and
zero-token dispatch/combine (valid no-ops).  Pointers here are fake aligned
addresses; the library must reject or accept them without touching them.
"""
import ctypes
import os
import re
import subprocess

import pytest

import combine_topk_idx_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_dispatch.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmoe_dispatch.so is not built (python -m combine_topk_idx_amd.build)")
    return M.library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == {"moe_rows_capacity", "moe_workspace_bytes", "moe_config_check",
                          "moe_dispatch_layout", "moe_dispatch_layout_noalloc", "moe_dispatch", "moe_dispatch_fused",
                          "moe_combine",
                          "moe_status_str", "moe_rank_rows_capacity", "moe_rank_layout",
                          "moe_dispatch_dedup", "moe_expand", "moe_combine_partial",
                          "moe_combine_reduce", "moe_row_expert", "moe_repack_rows_capacity",
                          "moe_repack_masked_to_contiguous", "moe_repack_contiguous_to_masked",
                          "moe_scale_words", "moe_scales_mn_major"}
    out = subprocess.run(["nm", "-D", "--defined-only", M.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moe_[a-z_]+)\b", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(lib, n)


def _cfg(**kw):
    base = dict(max_tokens=64, hidden=256, num_experts=8, num_topk=2, num_ranks=2,
                layout=M.LAYOUT_CONTIGUOUS, align=1, capacity=1, quant=M.QUANT_NONE, num_cus=0)
    base.update(kw)
    return M.MoeConfig(**base)


FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def _handle(**override):
    vals = {n: FAKE + 0x1000 * i for i, (n, _) in enumerate(M.MoeHandle._fields_)}
    vals.update(override)
    return M.MoeHandle(**vals)


def test_status_strings(lib):
    assert M.moe_status_str(0) == "MOE_OK"
    assert M.moe_status_str(2) == "MOE_ERR_CAPACITY"
    assert M.moe_status_str(4) == "MOE_ERR_HIP"
    assert M.moe_status_str(99) == "MOE_ERR_UNKNOWN"
    assert M.moe_status_str(-1) == "MOE_ERR_UNKNOWN"   # any int from C, read without an enum load


def test_size_queries(lib):
    c = _cfg(max_tokens=8192, hidden=7168, num_experts=256, num_topk=8, num_ranks=8, align=128,
             quant=M.QUANT_FP8_UE8M0)
    assert M.moe_rows_capacity(c) == 8192 * 8 + 256 * 127
    ws = M.moe_workspace_bytes(c)
    assert ws >= 257 * 4 and ws % 256 == 0
    c = _cfg(layout=M.LAYOUT_MASKED, capacity=256, num_experts=256, num_topk=8, num_ranks=8)
    assert M.moe_rows_capacity(c) == 256 * 256
    assert M.moe_rows_capacity(_cfg(num_topk=0)) == 0
    assert M.moe_workspace_bytes(_cfg(num_ranks=3)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(num_topk=0), M.MOE_ERR_INVALID_ARG),
    (dict(num_topk=33), M.MOE_ERR_INVALID_ARG),
    (dict(num_topk=32), M.MOE_OK),
    (dict(num_ranks=3), M.MOE_ERR_INVALID_ARG),          # E % R != 0
    (dict(num_ranks=0), M.MOE_ERR_INVALID_ARG),
    (dict(num_experts=0), M.MOE_ERR_INVALID_ARG),
    (dict(hidden=100), M.MOE_ERR_INVALID_ARG),            # H % 8 != 0
    (dict(hidden=0), M.MOE_ERR_INVALID_ARG),
    (dict(hidden=264, quant=M.QUANT_FP8_F32), M.MOE_ERR_INVALID_ARG),  # H % 128 != 0
    (dict(hidden=264), M.MOE_OK),
    (dict(align=0), M.MOE_ERR_INVALID_ARG),
    (dict(layout=M.LAYOUT_MASKED, capacity=0), M.MOE_ERR_INVALID_ARG),
    (dict(layout=M.LAYOUT_MASKED, capacity=0, align=0), M.MOE_ERR_INVALID_ARG),
    (dict(layout=M.LAYOUT_MASKED, capacity=5, align=0), M.MOE_OK),  # align unused
    (dict(layout=2), M.MOE_ERR_INVALID_ARG),
    (dict(quant=4), M.MOE_ERR_INVALID_ARG),
    (dict(quant=M.QUANT_MXFP8), M.MOE_OK),
    (dict(hidden=264, quant=M.QUANT_MXFP8), M.MOE_ERR_INVALID_ARG),       # MX needs H % 128 too
    (dict(num_cus=-1), M.MOE_ERR_INVALID_ARG),
    (dict(max_tokens=-1), M.MOE_ERR_INVALID_ARG),
    (dict(num_experts=4096, num_ranks=1), M.MOE_ERR_UNSUPPORTED),
    (dict(max_tokens=1 << 28, num_topk=16), M.MOE_ERR_UNSUPPORTED),  # rows overflow int32
])
def test_config_validation(lib, kw, code):
    assert M.moe_config_check(_cfg(**kw)) == code


def test_null_config(lib):
    assert lib.moe_config_check(None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_rows_capacity(None) == 0


def _layout(lib, cfg, T, idx=FAKE, h=None, ws=FAKE, ws_bytes=1 << 20):
    h = _handle() if h is None else h
    return lib.moe_dispatch_layout(ctypes.byref(cfg), T, idx, ctypes.byref(h), ws, ws_bytes, None)


def test_layout_argument_errors(lib):
    c = _cfg()
    assert _layout(lib, c, 65) == M.MOE_ERR_CAPACITY           # num_tokens > max_tokens
    assert _layout(lib, c, -1) == M.MOE_ERR_INVALID_ARG
    assert _layout(lib, c, 4, idx=None) == M.MOE_ERR_INVALID_ARG
    assert _layout(lib, c, 4, idx=FAKE + 2) == M.MOE_ERR_INVALID_ARG   # misaligned
    assert _layout(lib, c, 4, ws=None) == M.MOE_ERR_INVALID_ARG
    assert _layout(lib, c, 4, ws=FAKE + 8) == M.MOE_ERR_INVALID_ARG   # table rows are 16-byte vectors
    assert _layout(lib, c, 4, ws_bytes=16) == M.MOE_ERR_CAPACITY
    for f, _ in M.MoeHandle._fields_:
        assert _layout(lib, c, 4, h=_handle(**{f: None})) == M.MOE_ERR_INVALID_ARG, f
        assert _layout(lib, c, 4, h=_handle(**{f: FAKE + 1})) == M.MOE_ERR_INVALID_ARG, f
    assert lib.moe_dispatch_layout(ctypes.byref(c), 4, FAKE, None, FAKE, 1 << 20, None) \
        == M.MOE_ERR_INVALID_ARG
    assert _layout(lib, _cfg(num_topk=40), 4) == M.MOE_ERR_INVALID_ARG


def test_noalloc_layout_argument_errors(lib):
    # every error below is found before the library touches a device
    def call(cfg, T, idx=FAKE, h=None):
        h = _handle() if h is None else h
        return lib.moe_dispatch_layout_noalloc(ctypes.byref(cfg), T, idx, ctypes.byref(h), None)
    c = _cfg()
    assert call(c, 65) == M.MOE_ERR_CAPACITY           # num_tokens > max_tokens
    assert call(c, -1) == M.MOE_ERR_INVALID_ARG
    assert call(c, 4, idx=None) == M.MOE_ERR_INVALID_ARG
    assert call(c, 4, idx=FAKE + 2) == M.MOE_ERR_INVALID_ARG
    for f, _ in M.MoeHandle._fields_:
        assert call(c, 4, h=_handle(**{f: None})) == M.MOE_ERR_INVALID_ARG, f
    assert lib.moe_dispatch_layout_noalloc(ctypes.byref(c), 4, FAKE, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_layout_noalloc(None, 4, FAKE, ctypes.byref(_handle()), None) == M.MOE_ERR_INVALID_ARG
    # the static workspace holds the 2048-expert table and 1,966,016 pair slots
    big = _cfg(max_tokens=1 << 20, num_experts=2048, num_topk=2, num_ranks=2)
    assert call(big, 1 << 20) == M.MOE_ERR_CAPACITY     # 2,097,152 pairs
    assert call(big, 983009) == M.MOE_ERR_CAPACITY      # 1,966,018 pairs


def _dispatch(lib, cfg, T, x=FAKE, w=None, out=FAKE, scale=None, rw=None, h=None):
    h = _handle() if h is None else h
    return lib.moe_dispatch(ctypes.byref(cfg), T, x, w, ctypes.byref(h), out, scale, rw, None)


def test_dispatch_argument_errors(lib):
    c = _cfg()
    f8 = _cfg(quant=M.QUANT_FP8_F32)
    assert _dispatch(lib, c, 65) == M.MOE_ERR_CAPACITY
    assert _dispatch(lib, c, -3) == M.MOE_ERR_INVALID_ARG
    assert _dispatch(lib, c, 4, x=None) == M.MOE_ERR_INVALID_ARG
    assert _dispatch(lib, c, 4, x=FAKE + 8) == M.MOE_ERR_INVALID_ARG      # needs 16-byte alignment
    assert _dispatch(lib, c, 4, out=None) == M.MOE_ERR_INVALID_ARG
    assert _dispatch(lib, c, 4, out=FAKE + 4) == M.MOE_ERR_INVALID_ARG
    assert _dispatch(lib, c, 4, scale=FAKE) == M.MOE_ERR_INVALID_ARG      # no scales without FP8
    assert _dispatch(lib, f8, 4) == M.MOE_ERR_INVALID_ARG                 # FP8 needs scales
    assert _dispatch(lib, c, 4, rw=FAKE) == M.MOE_ERR_INVALID_ARG         # row weights need topk_w
    assert _dispatch(lib, c, 4, h=_handle(pair_to_row=None)) == M.MOE_ERR_INVALID_ARG
    # zero tokens: valid, nothing enqueued
    assert _dispatch(lib, c, 0, x=None) == M.MOE_OK
    assert _dispatch(lib, f8, 0, x=None, scale=FAKE) == M.MOE_OK


def _combine(lib, cfg, T, y=FAKE, w=FAKE, out=FAKE, h=None):
    h = _handle() if h is None else h
    return lib.moe_combine(ctypes.byref(cfg), T, y, w, ctypes.byref(h), out, None)


def test_combine_argument_errors(lib):
    c = _cfg()
    assert _combine(lib, c, 65) == M.MOE_ERR_CAPACITY
    assert _combine(lib, c, -1) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 3, y=None) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 3, w=None) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 3, out=None) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 3, out=FAKE + 2) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, _cfg(hidden=12), 3) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 3, h=_handle(status=None)) == M.MOE_ERR_INVALID_ARG
    assert _combine(lib, c, 0, y=None, w=None, out=None) == M.MOE_OK


def test_binding_refuses_host_tensors(lib):
    import torch
    c = _cfg()
    with pytest.raises(ValueError):
        M._ptr(torch.zeros(4), 4, 0, "t")


def _fused(lib, cfg, T, idx=FAKE, x=FAKE, w=None, h=None, ws=FAKE, ws_bytes=1 << 20, out=FAKE, scale=None,
           rw=None):
    h = _handle() if h is None else h
    return lib.moe_dispatch_fused(ctypes.byref(cfg), T, idx, x, w, ctypes.byref(h), ws, ws_bytes, out, scale,
                                  rw, None)


def test_fused_dispatch_argument_errors(lib):
    """The fused call rejects everything either separate call rejects."""
    c = _cfg()
    f8 = _cfg(quant=M.QUANT_FP8_UE8M0)
    assert _fused(lib, c, 65) == M.MOE_ERR_CAPACITY
    assert _fused(lib, c, -1) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, idx=None) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, ws=None) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, ws=FAKE + 4) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, ws_bytes=8) == M.MOE_ERR_CAPACITY
    assert _fused(lib, c, 4, x=None) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, x=FAKE + 8) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, out=None) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, scale=FAKE) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, f8, 4) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, rw=FAKE) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, c, 4, h=_handle(row_to_pair=None)) == M.MOE_ERR_INVALID_ARG
    assert _fused(lib, _cfg(num_ranks=3), 4) == M.MOE_ERR_INVALID_ARG


# ---- per-rank deduplicated exchange -------------------------------------------

def _rank_handle(**override):
    vals = {n: FAKE + 0x100000 + 0x1000 * i for i, (n, _) in enumerate(M.MoeRankHandle._fields_)}
    vals.update(override)
    return M.MoeRankHandle(**vals)


def test_rank_rows_capacity(lib):
    c = _cfg(max_tokens=8192, hidden=7168, num_experts=256, num_topk=8, num_ranks=8)
    assert M.moe_rank_rows_capacity(c) == 8192 * 8
    assert M.moe_rank_rows_capacity(_cfg(num_topk=6, num_ranks=4, num_experts=8)) == 64 * 4
    assert M.moe_rank_rows_capacity(_cfg(num_experts=64, num_ranks=64)) == 0   # R > 32
    assert M.moe_rank_rows_capacity(_cfg(num_ranks=3)) == 0
    assert lib.moe_rank_rows_capacity(None) == 0


def _call(lib, name, cfg, T, **kw):
    """One per-rank entry point with FAKE arguments, overridable by name.
    Every use below passes at least one argument the host check rejects (or
    T == 0 where the call enqueues nothing), so no kernel is ever launched."""
    a = dict(idx=FAKE, x=FAKE, y=FAKE, w=FAKE, send=FAKE, send_scale=None, out=FAKE, out_scale=None,
             partial=FAKE, rh=_rank_handle(), h=_handle())
    a.update(kw)
    c = ctypes.byref(cfg)
    rh = None if a["rh"] is None else ctypes.byref(a["rh"])
    h = ctypes.byref(a["h"])
    if name == "dispatch_dedup":
        return lib.moe_dispatch_dedup(c, T, a["x"], rh, a["send"], a["send_scale"], None)
    if name == "expand":
        return lib.moe_expand(c, T, a["idx"], a["send"], a["send_scale"], rh, h, a["out"], a["out_scale"], None)
    if name == "combine_partial":
        return lib.moe_combine_partial(c, T, a["idx"], a["y"], a["w"], h, rh, a["partial"], None)
    if name == "combine_reduce":
        return lib.moe_combine_reduce(c, T, a["partial"], rh, a["out"], None)
    if name == "rank_layout":
        return lib.moe_rank_layout(c, T, a["idx"], rh, None)
    raise KeyError(name)


DEDUP = ("dispatch_dedup", "expand", "combine_partial", "combine_reduce", "rank_layout")


def test_dedup_argument_errors(lib):
    c = _cfg()
    wide = _cfg(num_experts=64, num_ranks=64)
    for name in DEDUP:
        assert _call(lib, name, c, 65) == M.MOE_ERR_CAPACITY, name
        assert _call(lib, name, c, -1) == M.MOE_ERR_INVALID_ARG, name
        assert _call(lib, name, wide, 4) == M.MOE_ERR_UNSUPPORTED, name
        assert _call(lib, name, _cfg(num_ranks=3), 4) == M.MOE_ERR_INVALID_ARG, name
        assert _call(lib, name, c, 4, rh=None) == M.MOE_ERR_INVALID_ARG, name
        for f, _ in M.MoeRankHandle._fields_:
            for bad in (None, FAKE + 2):
                assert _call(lib, name, c, 4, rh=_rank_handle(**{f: bad})) == M.MOE_ERR_INVALID_ARG, (f, name)
    assert _call(lib, "rank_layout", c, 4, idx=None) == M.MOE_ERR_INVALID_ARG
    assert _call(lib, "rank_layout", c, 4, idx=FAKE + 2) == M.MOE_ERR_INVALID_ARG
    # the calls that read the per-expert handle check it too
    for name in ("expand", "combine_partial"):
        assert _call(lib, name, c, 4, h=_handle(pair_to_row=None)) == M.MOE_ERR_INVALID_ARG, name


def test_dedup_pointer_errors(lib):
    c = _cfg()
    f8 = _cfg(quant=M.QUANT_FP8_UE8M0)
    bad = M.MOE_ERR_INVALID_ARG
    assert _call(lib, "dispatch_dedup", c, 4, x=None) == bad
    assert _call(lib, "dispatch_dedup", c, 4, x=FAKE + 8) == bad
    assert _call(lib, "dispatch_dedup", c, 4, send=FAKE + 8) == bad
    assert _call(lib, "dispatch_dedup", c, 4, send_scale=FAKE) == bad     # scales without FP8
    assert _call(lib, "dispatch_dedup", f8, 4) == bad                     # FP8 needs scales
    assert _call(lib, "expand", c, 4, idx=None) == bad
    assert _call(lib, "expand", c, 4, send=FAKE + 8) == bad
    assert _call(lib, "expand", c, 4, out=None) == bad
    assert _call(lib, "expand", c, 4, out_scale=FAKE) == bad              # scales without FP8
    assert _call(lib, "expand", f8, 4, out_scale=FAKE) == bad             # FP8 needs send scales
    assert _call(lib, "expand", f8, 4, send_scale=FAKE) == bad            # ... and out scales
    assert _call(lib, "combine_partial", c, 4, idx=None) == bad
    assert _call(lib, "combine_partial", c, 4, y=FAKE + 2) == bad
    assert _call(lib, "combine_partial", c, 4, w=None) == bad
    assert _call(lib, "combine_partial", c, 4, partial=FAKE + 2) == bad
    assert _call(lib, "combine_reduce", c, 4, partial=None) == bad
    assert _call(lib, "combine_reduce", c, 4, out=FAKE + 2) == bad
    # zero tokens: valid no-ops that enqueue nothing (the layout call is left
    # out: with zero tokens it still writes the empty layout on the device)
    assert _call(lib, "dispatch_dedup", c, 0, x=None) == M.MOE_OK
    assert _call(lib, "expand", c, 0, idx=None, send=None) == M.MOE_OK
    assert _call(lib, "combine_partial", c, 0, idx=None, y=None, w=None, partial=None) == M.MOE_OK
    assert _call(lib, "combine_reduce", c, 0, partial=None, out=None) == M.MOE_OK


# ---- grouped-GEMM adapters ----------------------------------------------------

def test_adapter_size_queries(lib):
    m = _cfg(max_tokens=256, hidden=7168, num_experts=256, num_topk=8, num_ranks=8,
             layout=M.LAYOUT_MASKED, capacity=256, quant=M.QUANT_FP8_F32)
    assert M.moe_repack_rows_capacity(m, 1) == 2048
    assert M.moe_repack_rows_capacity(m, 128) == 2048 + 256 * 127
    small = _cfg(layout=M.LAYOUT_MASKED, capacity=3)            # E*C = 24 < T*K = 128
    assert M.moe_repack_rows_capacity(small, 2) == 24 + 8
    assert M.moe_repack_rows_capacity(_cfg(), 4) == 0           # contiguous cfg
    assert M.moe_repack_rows_capacity(small, 0) == 0
    assert M.moe_scale_words(m) == 56
    assert M.moe_scale_words(_cfg(hidden=7168, quant=M.QUANT_FP8_UE8M0)) == 14
    assert M.moe_scale_words(_cfg(hidden=640, quant=M.QUANT_FP8_UE8M0)) == 2
    assert M.moe_scale_words(_cfg(hidden=7168, quant=M.QUANT_MXFP8)) == 56
    assert M.moe_scale_words(_cfg()) == 0
    assert lib.moe_scale_words(None) == 0


def test_adapter_argument_errors(lib):
    """Every call has at least one argument the host check rejects, so no
    kernel is launched."""
    bad = M.MOE_ERR_INVALID_ARG
    c = _cfg()
    m = _cfg(layout=M.LAYOUT_MASKED, capacity=4)
    mf = _cfg(layout=M.LAYOUT_MASKED, capacity=4, quant=M.QUANT_FP8_F32)
    h = ctypes.byref(_handle())
    assert lib.moe_row_expert(ctypes.byref(c), h, None, None) == bad
    assert lib.moe_row_expert(ctypes.byref(c), h, FAKE + 2, None) == bad
    assert lib.moe_row_expert(ctypes.byref(c), None, FAKE, None) == bad
    assert lib.moe_row_expert(ctypes.byref(_cfg(num_topk=0)), h, FAKE, None) == bad
    hb = ctypes.byref(_handle(recv_count=None))
    assert lib.moe_row_expert(ctypes.byref(c), hb, FAKE, None) == bad

    def m2c(cfg, align=4, h=h, x=FAKE, s=None, ox=FAKE, os_=None, off=FAKE, rex=FAKE):
        return lib.moe_repack_masked_to_contiguous(ctypes.byref(cfg), align, h, x, s, ox, os_, off, rex, None)
    assert m2c(c) == bad                       # contiguous cfg
    assert m2c(m, align=0) == bad
    assert m2c(m, h=hb) == bad
    assert m2c(m, x=None) == bad
    assert m2c(m, ox=FAKE + 8) == bad
    assert m2c(m, s=FAKE) == bad               # scales without FP8
    assert m2c(mf) == bad                      # FP8 needs both scale pointers
    assert m2c(mf, s=FAKE) == bad
    assert m2c(m, off=None) == bad
    assert m2c(m, rex=FAKE + 1) == bad

    def c2m(cfg, h=h, off=FAKE, y=FAKE, ym=FAKE):
        return lib.moe_repack_contiguous_to_masked(ctypes.byref(cfg), h, off, y, ym, None)
    assert c2m(c) == bad
    assert c2m(m, h=hb) == bad
    assert c2m(m, off=None) == bad
    assert c2m(m, y=FAKE + 2) == bad
    assert c2m(m, ym=None) == bad

    def mn(cfg, rows=8, s=FAKE, o=FAKE):
        return lib.moe_scales_mn_major(ctypes.byref(cfg), rows, s, o, None)
    assert mn(c) == bad                        # bf16: no scales
    assert mn(mf, rows=-1) == bad
    assert mn(mf, s=None) == bad
    assert mn(mf, o=FAKE + 4) == bad
    assert mn(mf, rows=0) == M.MOE_OK          # nothing to do, nothing enqueued
