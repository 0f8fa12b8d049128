"""CPU checks of bench.py's byte models and JSON helpers (no GPU needed).

The algorithmic bytes per call are what the roofline fractions divide by, so
they are pinned to hand counts of the DeepSeek-V3 prefill batch: 65,536
kept pairs, H = 7168, 56 quantization blocks, 14 packed UE8M0 words per row.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

bench = pytest.importorskip("bench")
from combine_topk_idx_amd import workloads as W  # noqa: E402


def test_direct_path_bytes_deepseek_prefill():
    wl = W.WORKLOADS["deepseekv3_prefill_T8192"]
    ab = bench.algorithmic_bytes(wl, 65536)
    T, K, H, N = 8192, 8, 7168, 65536
    assert ab["layout"] == 4 * T * K + 4 * T * K + 4 * N == 786_432
    assert ab["dispatch"] == 2 * T * H + 4 * T * K + N * (H + 56) == 591_134_720
    assert ab["combine"] == 2 * N * H + 8 * T * K + 2 * T * H == 1_057_488_896
    assert sum(ab.values()) == 1_649_410_048


def test_bytes_per_format():
    base = W.WORKLOADS["deepseekv3_prefill_T8192"]
    T, K, H, N = 8192, 8, 7168, 65536
    rows = {W.QUANT_NONE: 2 * H, W.QUANT_FP8_F32: H + 4 * 56, W.QUANT_FP8_UE8M0: H + 56,
            W.QUANT_MXFP8: H + 224}
    for q, row in rows.items():
        ab = bench.algorithmic_bytes(base.replace(quant=q), N)
        assert ab["dispatch"] == 2 * T * H + 4 * T * K + N * row
        assert bench.row_and_scale_bytes(base.replace(quant=q))[0] + \
            bench.row_and_scale_bytes(base.replace(quant=q))[1] == row


def test_dedup_bytes_deepseek_prefill():
    wl = W.WORKLOADS["deepseekv3_prefill_T8192"]
    T, K, H, R, N, Q = 8192, 8, 7168, 8, 65536, 32477
    ab = bench.dedup_bytes(wl, N, Q)
    row = H + 56
    assert ab["dispatch_dedup"] == 2 * T * H + 4 * T * R + Q * row
    assert ab["expand"] == 12 * T * K + Q * row + N * row
    assert ab["combine_partial"] == 2 * N * H + 16 * T * K + 2 * Q * H
    assert ab["combine_reduce"] == 4 * T * R + 2 * Q * H + 2 * T * H


def test_short_kernel_names():
    assert bench.short_kernel("void moe::(anonymous namespace)::dispatch_rows<2>(moe::DispatchArgs)") \
        == "dispatch_rows_fp8_ue8m0"
    for nt in ("false", "true"):
        assert bench.short_kernel(f"void moe::(anonymous namespace)::combine_kernel<false, {nt}>(moe::CombineArgs)") \
            == "combine_kernel"
        assert bench.short_kernel(f"void moe::(anonymous namespace)::combine_kernel<true, {nt}>(moe::CombineArgs)") \
            == "combine_kernel_partial"
    assert bench.short_kernel("moe::(anonymous namespace)::layout_single(moe::LayoutArgs)") == "layout_single"
    assert bench.short_kernel("void moe::(anonymous namespace)::rank_layout_kernel<2>(moe::RankLayoutArgs)") \
        == "rank_layout_kernel"
    assert bench.short_kernel("void moe::(anonymous namespace)::repack_kernel<true>(moe::RepackArgs)") \
        == "repack_to_contiguous"
    assert bench.short_kernel("void moe::(anonymous namespace)::dispatch_rows<3>(moe::DispatchArgs)") \
        == "dispatch_rows_mxfp8"


def test_kernel_bytes_cover_every_dispatch_kernel():
    ab = {"layout": 10, "dispatch": 100, "combine": 1000}
    algo = bench.kernel_bytes({"path": {"algorithmic_bytes": ab, "calls": "moe_dispatch_fused + moe_combine"}})
    for q in bench.QUANT_TEMPLATE.values():
        assert algo[f"dispatch_rows_{q}"] == 100
        assert algo[f"dispatch_fused_{q}"] == 110
    assert algo["combine_kernel"] == 1000 and algo["layout_single"] == 10


def test_library_hash_is_stable():
    assert bench.library_hash() == bench.library_hash()
    assert len(bench.library_hash()) == 64


def test_code_text_ignores_comments_not_code():
    src = 'int a = 1; // note\n/* block\n comment */ int b = 2;\nconst char *s = "// kept";\nchar c = \'\\\'\';\n'
    edited_comment = src.replace("note", "another note").replace("block", "other")
    relaid = src.replace("int b = 2;", "int   b =\n 2;")
    changed_code = src.replace("int b = 2;", "int b = 3;")
    assert bench.code_text(src) == bench.code_text(edited_comment) == bench.code_text(relaid)
    assert bench.code_text(src) != bench.code_text(changed_code)
    assert '"// kept"' in bench.code_text(src)
    assert "note" not in bench.code_text(src) and "comment" not in bench.code_text(src)


def test_bench_refuses_more_than_one_gpu(tmp_path):
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "one GPU" in r.stderr
