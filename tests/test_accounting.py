"""The bench's work accounting (expert_ffn_layer_gemm_amd/accounting.py), host
logic only: pinned to the numbers the pages print (tests/golden/
pages_worked_numbers.json, each entry citing its page and section) and to
small cases counted by hand."""
import json
import os

import numpy as np
import pytest

from expert_ffn_layer_gemm_amd import accounting as acc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_numbers.json")))


def test_tokens_per_expert_prefill_page_number():
    g = GOLDEN["tokens_per_expert_prefill"]
    assert acc.tokens_per_expert(g["T"], g["k"], g["E"]) == g["value"]


def test_groupgemm_m_at_ep128_page_number():
    g = GOLDEN["groupgemm_tokens_per_expert_ep128"]
    assert acc.ep_tokens_per_expert(g["batch"], g["qlen"], g["k"], g["ep"], g["E"]) == g["value"]


def test_groupgemm_cost_formulas():
    # 2*g*m*k*n FLOPs and g*(m*k + n*k + m*n) elements, written out for g=3, m=5, k=7, n=11
    assert acc.groupgemm_flops(3, 5, 7, 11) == 2 * 3 * 5 * 7 * 11 == 2310
    assert acc.groupgemm_io_elements(3, 5, 7, 11) == 3 * (35 + 77 + 55) == 501


def test_fp8_scale_shapes():
    # (M, K) x (K, N): activation scales [M, ceil(K/128)], weight scales [ceil(K/128), ceil(N/128)]
    assert acc.fp8_scale_shapes(4096, 7168, 2048) == ((4096, 56), (56, 16))
    assert acc.fp8_scale_shapes(3, 129, 1) == ((3, 2), (2, 1))


def test_kernel_work_by_hand():
    counts = np.array([0, 3, 70, 64, 65, 0])       # skinny: 3, 64; tiled: 70, 65
    H, I = 256, 128
    w = acc.kernel_work("skinny_gateup_bf16", counts, H, I, "bf16")
    assert w.groups == 2
    assert w.bytes == 2 * (2 * I * H * 2) + 67 * H * 2 + 67 * I * 2
    assert w.flops == 4.0 * 67 * I * H
    w = acc.kernel_work("tiled_down_bf16", counts, H, I, "bf16")
    assert w.groups == 2 and w.bytes == 2 * (H * I * 2) + 135 * I * 2 + 135 * H * 2
    # fp8: one byte per value, fp32 scale per 128x128 weight block and per 128 activation values
    w = acc.kernel_work("tiled_gateup_fp8", counts, H, I, "fp8")
    assert w.bytes == (2 * (2 * I * H) + 2 * 2 * (I // 128) * (H // 128) * 4
                       + 135 * H + 135 * (H // 128) * 4 + 135 * I + 135 * (I // 128) * 4)
    # mxfp8: one byte per value plus one E8M0 byte per 32 values of every row
    w = acc.kernel_work("skinny_down_mx", counts, H, I, "mxfp8")
    assert w.bytes == 2 * (H * I + H * (I // 32)) + 67 * (I + I // 32) + 67 * H * 2
    with pytest.raises(ValueError):
        acc.kernel_work("combine", counts, H, I, "bf16")


def test_skinny_split_follows_the_batch():
    # T <= 64: no group can exceed 64 rows, all of them stream; larger batches
    # send groups above 48 rows to the tiled kernels
    assert acc.skinny_max_rows(1) == acc.skinny_max_rows(64) == 64
    assert acc.skinny_max_rows(65) == acc.skinny_max_rows(8192) == 48
    counts = np.array([48, 49, 64, 3])
    assert list(acc.kernel_groups("skinny_down_bf16", counts, acc.skinny_max_rows(1000))) == [48, 3]
    assert list(acc.kernel_groups("tiled_down_bf16", counts, acc.skinny_max_rows(1000))) == [49, 64]
    assert list(acc.kernel_groups("skinny_down_bf16", counts, acc.skinny_max_rows(64))) == [48, 49, 64, 3]


def test_layer_work_by_hand():
    T, H, E, k, I = 10, 256, 4, 2, 128
    counts = np.array([7, 0, 13, 0, 10])            # routed (7+13 = 20 = T*k), then a shared expert
    w = acc.layer_work(T, H, E, k, I, 1, "bf16", counts)
    assert w.groups == 3
    assert w.bytes == 3 * 3 * H * I * 2 + 4 * H * E + 2 * T * H * 2
    assert w.flops == 2 * T * H * E + 2 * 30 * 3 * H * I


def test_roofline_picks_the_binding_roof():
    # ridge bf16 = 2500e12 / 8000e9 = 312.5 FLOP/B
    hbm = acc.roofline(acc.Work(bytes=1e9, flops=1e11, groups=1), 1e-3, "bf16")
    assert hbm["bound"] == "hbm" and abs(hbm["achieved"] - 1000.0) < 1e-9 and abs(hbm["frac"] - 0.125) < 1e-12
    mfma = acc.roofline(acc.Work(bytes=1e9, flops=1e12, groups=1), 1e-3, "bf16")
    assert mfma["bound"] == "mfma" and abs(mfma["achieved"] - 1000.0) < 1e-9 and abs(mfma["frac"] - 0.4) < 1e-12
    assert acc.PEAK_TFLOPS["fp8"] == acc.PEAK_TFLOPS["mxfp8"] == 2 * acc.PEAK_TFLOPS["bf16"]
