"""The FLOP accounting used for the MFMA roofline reproduces the expert-GEMM
figures the pages print (tests/golden/pages_expert_gemm_flops.json)."""
import json
import os

import pytest

from measure import accounting

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_expert_gemm_flops.json")))


@pytest.mark.parametrize("case", GOLD["cases"], ids=lambda c: c["what"])
def test_expert_gemm_gflops_match_pages(case):
    f = accounting.gate_up_flops if case["part"] == "gate_up" else accounting.down_flops
    got = case["G"] * f(case["m"], case["H"], case["I"]) / 1e9
    assert abs(got - case["gflop"]) <= case["rel"] * case["gflop"]


@pytest.mark.parametrize("case", GOLD["rows_per_group"], ids=lambda c: c["what"])
def test_rows_per_group_match_pages(case):
    m = case["tokens"] * case["k"] * case["gpus"] // case["experts_total"]
    assert m == case["m"]


def test_per_row_expert_work():
    # 6 H I per (row, expert) at the DeepSeek-V3 shape: 88.08 MFLOP
    assert accounting.ffn_flops(1, 7168, 2048) == 6 * 7168 * 2048
    assert accounting.weight_bytes_per_expert(7168, 2048, "bf16") == 88080384
