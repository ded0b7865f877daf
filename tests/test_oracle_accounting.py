"""KV-cache accounting closed forms against the numbers the pages print (tests/golden/kv_accounting.json)."""
import json
import os
from fractions import Fraction

import pytest

from oracle import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kv_accounting.json")))


def test_llama3_headline_cards():
    p, g = GOLD["llama3_8b_preset"], GOLD["gqa_headline"]
    assert acc.savings_vs_mha(p["q_heads"], p["kv_groups"]) == g["savings"]
    assert acc.kv_bytes_per_token(p["kv_groups"], p["head_dim"], p["bits"], p["layers"]) == g["kv_bytes_per_token"]
    assert acc.kv_buffer_bytes(p["kv_groups"], p["head_dim"], p["bits"], p["layers"], p["context"]) == g["buffer_bytes_8192"]
    assert acc.kv_buffer_bytes(p["q_heads"], p["head_dim"], p["bits"], p["layers"], p["context"]) == g["mha_buffer_bytes_8192"]
    assert acc.kv_buffer_bytes(1, p["head_dim"], p["bits"], p["layers"], p["context"]) == g["mqa_buffer_bytes_8192"]
    # binary units: 128 KiB, 1 GiB, 4 GiB, 128 MiB
    assert g["kv_bytes_per_token"] == 128 * 2**10 and g["buffer_bytes_8192"] == 2**30
    assert g["mha_buffer_bytes_8192"] == 4 * 2**30 and g["mqa_buffer_bytes_8192"] == 128 * 2**20


@pytest.mark.parametrize("row", GOLD["mode_table"]["rows"], ids=lambda r: r["mode"])
def test_mode_table_rows(row):
    p = GOLD["llama3_8b_preset"]
    got = acc.mode_row(p["q_heads"], row["kv_groups"], p["layers"], p["head_dim"], p["context"], p["bits"])
    for key in ("mode", "kv_groups", "q_per_group", "kv_bytes_per_token", "buffer_bytes", "savings",
                "kv_proj_params", "all4_proj_params"):
        want = row[key if key != "savings" else "savings"]
        have = got[key if key != "savings" else "savings_vs_mha"]
        assert have == want, key
    # Q and O projections do not depend on the grouping: about 1.07 billion in every row
    assert round(got["qo_proj_params"] / 1e9, 2) == GOLD["mode_table"]["qo_proj_params_rounded_billions"]


def test_savings_is_linear_in_groups_and_independent_of_context_and_dtype():
    p = GOLD["llama3_8b_preset"]
    for groups in acc.valid_group_counts(p["q_heads"]):
        mha = acc.kv_buffer_bytes(p["q_heads"], p["head_dim"], p["bits"], p["layers"], p["context"])
        this = acc.kv_buffer_bytes(groups, p["head_dim"], p["bits"], p["layers"], p["context"])
        assert mha / this == acc.savings_vs_mha(p["q_heads"], groups) == Fraction(p["q_heads"], groups)
        for ctx in (0, 512, 131072):
            for bits in GOLD["head_dim_choices"]["bits"].values():
                a = acc.kv_buffer_bytes(p["q_heads"], p["head_dim"], bits, p["layers"], ctx)
                b = acc.kv_buffer_bytes(groups, p["head_dim"], bits, p["layers"], ctx)
                if ctx:
                    assert a / b == Fraction(p["q_heads"], groups)


def test_fp8_halves_and_int4_quarters():
    p = GOLD["llama3_8b_preset"]
    bf16 = acc.kv_bytes_per_token(p["kv_groups"], p["head_dim"], 16, p["layers"])
    fp8 = acc.kv_bytes_per_token(p["kv_groups"], p["head_dim"], 8, p["layers"])
    int4 = acc.kv_bytes_per_token(p["kv_groups"], p["head_dim"], 4, p["layers"])
    assert fp8 * 2 == bf16 and int4 * 4 == bf16
    # one int4 element is half a byte; results stay exact Fractions
    assert acc.kv_bytes_per_token(1, 1, 4, 1) == Fraction(2 * 4, 8)
    assert isinstance(int4, Fraction)


def test_invalid_group_counts_are_errors_not_rounded():
    g = GOLD["invalid_groups"]
    assert acc.valid_group_counts(g["q_heads"]) == g["valid"]
    for bad in g["bad_groups"]:
        with pytest.raises(acc.GroupCountError) as ei:
            acc.check_groups(g["q_heads"], bad)
        assert ei.value.valid == g["valid"]
    with pytest.raises(acc.GroupCountError) as ei:
        acc.mode_row(g["q_heads"], 3, 32, 128, 8192, 16)
    assert ei.value.remainder == g["remainder_for_3"]


def test_quiz():
    q = GOLD["quiz"]
    assert acc.savings_vs_mha(64, 8) == q["q64_kv8_savings"]
    p = GOLD["llama3_8b_preset"]
    mha = acc.mode_row(p["q_heads"], p["q_heads"], p["layers"], p["head_dim"], p["context"], p["bits"])
    gqa = acc.mode_row(p["q_heads"], p["kv_groups"], p["layers"], p["head_dim"], p["context"], p["bits"])
    assert round(mha["all4_proj_params"] / gqa["all4_proj_params"], 1) == q["all4_ratio_rounded"]
    assert mha["kv_proj_params"] / gqa["kv_proj_params"] == 4


def test_minimind_gqa_vs_mla_elements():
    m = GOLD["minimind"]
    gqa = acc.kv_elems_per_token_layer(m["gqa_kv_groups"], m["gqa_head_dim"])
    mla = acc.mla_elems_per_token_layer(m["mla_kv_lora_rank"], m["mla_rope_dim"])
    assert gqa == m["gqa_elems"] and mla == m["mla_elems"]
    assert round(gqa / mla, 1) == m["compression_rounded"]
    assert Fraction(gqa, mla) == Fraction(48, 11)


def test_endpoints_of_the_ladder():
    # groups == query heads reproduces the MHA row; groups == 1 reproduces the MQA row
    assert acc.mode_name(32, 32) == "MHA" and acc.mode_name(32, 1) == "MQA" and acc.mode_name(32, 8) == "GQA"
