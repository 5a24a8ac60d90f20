"""Byte accounting against the figures the GSI pages print (tests/golden)."""
import json
import os

from rank_gated_memory_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_weight_read_speedups_match_printed():
    for row in load()["weight_read_speedup"]:
        s = acc.weight_read_speedup(row["d"], row["k"], 1.0 - row["fast_share"])
        assert abs(s - row["printed"]) <= row["abs_tol"], (row["model"], s)


def test_effective_parameters_match_printed():
    for row in load()["effective_parameters"]:
        p = acc.effective_parameters(row["total"], row["d"], row["k"])
        assert abs(p - row["printed"]) <= row["rel_tol"] * row["printed"]


def test_storage_overhead_below_printed_bound():
    for row in load()["storage_overhead"]:
        assert row["overhead_bytes"] / row["model_bytes"] < row["printed_bound"]


def test_token_bytes_by_hand():
    # QKV map of the GPT-J shape, bf16: fast = 2*(4096*256 + 12288*256 + 4096 + 12288)
    assert acc.token_bytes(4096, 12288, 256, 2, False) == 2 * (4096 * 256 + 12288 * 256 + 4096 + 12288)
    assert acc.token_bytes(4096, 12288, 256, 2, True) == 2 * (4096 * 256 + 4096 * 12288 + 4096 + 12288)
    assert (acc.project_bytes(4096, 256, 2) + acc.apply_bytes(4096, 12288, 256, 2, False)
            == acc.token_bytes(4096, 12288, 256, 2, False))
    assert (acc.project_bytes(4096, 256, 2) + acc.apply_bytes(4096, 12288, 256, 2, True)
            == acc.token_bytes(4096, 12288, 256, 2, True) + 2 * 4096)
    # dense / fast ratios of the GPT-J shapes
    assert round(acc.dense_bytes(4096, 12288, 2) / acc.token_bytes(4096, 12288, 256, 2, False), 1) == 12.0
