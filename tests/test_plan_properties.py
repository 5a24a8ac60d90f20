"""Properties of stack plans over random call arrays (host only: gsi_stack_plan
is pure host work, so no device is touched).

For any valid array of calls (random shapes within the documented limits,
either dtype, non-decreasing wave numbers) the plan must cover every row of
every map exactly once with its units, keep the workspace regions it hands
out disjoint and inside the workspace, and keep its tables consistent: the
projection units of a wave are contiguous, each call's units are contiguous
and point back to it, and the output order is wave-major.  These are the
facts the single-launch kernel relies on without checking them.
"""
import os

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from rank_gated_memory_amd import gsi
from tests.test_abi import GSI_OK, build_plan, plan_tables

pytestmark = pytest.mark.skipif(not os.path.exists(gsi.LIB_PATH), reason="libgsi.so not built")

KMAX, ROW_BYTES, TILE = 1024, 32768, 64
GROUP_UNITS, GROUP_UNITS2 = 16, 64   # two-level sums above 64 units, groups of 16
CTL_HEADER, CTL_PER_WAVE = 96, 1088   # control words: header, one block per wave, two per call


@st.composite
def call_arrays(draw):
    dtype = draw(st.sampled_from([0, 1]))  # fp32, bf16
    es = 4 if dtype == 0 else 2
    n = draw(st.integers(1, 24))
    specs = []
    for _ in range(n):
        d = 8 * draw(st.integers(1, ROW_BYTES // es // 8))
        k = 8 * draw(st.integers(1, min(d, KMAX) // 8))
        d_out = 8 * draw(st.integers(1, 4096))
        specs.append((d, d_out, k, dtype))
    steps = draw(st.lists(st.integers(0, 2), min_size=n, max_size=n))
    waves = list(np.cumsum(steps) - steps[0])  # non-decreasing, may skip numbers
    return specs, [int(w) for w in waves]


def align_up(v, a):
    return (v + a - 1) // a * a


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(call_arrays())
def test_plan_covers_every_row_and_keeps_regions_apart(arg):
    specs, waves = arg
    st_, plan, nb = build_plan(specs, waves)
    assert st_ == GSI_OK
    h, desc, unit_call, order, p_begin, o_begin = plan_tables(plan)
    n = len(specs)
    assert h["n"] == n and h["total_bytes"] == nb
    # waves renumbered densely in order of appearance
    dense = np.cumsum([0] + [int(waves[i] != waves[i - 1]) for i in range(1, n)])
    assert list(desc["wave"]) == list(dense) and h["n_waves"] == dense[-1] + 1
    W = int(h["n_waves"])
    for i, (d, d_out, k, _) in enumerate(specs):
        c = desc[i]
        assert (c["d"], c["d_out"], c["k"]) == (d, d_out, k) and c["gate_off"] == i
        # projection units: rows of V_k, every row once
        rows, au = int(c["a_rows"]), int(c["a_units"])
        assert rows == d or (rows % 16 == 0 and rows <= 2048)
        assert (au - 1) * rows < d <= au * rows
        assert c["groups"] == (1 if au <= GROUP_UNITS2 else -(-au // GROUP_UNITS))
        # fast units: 64-row tiles of M; slow units: rows of W
        tiles, ft, fu = -(-d_out // TILE), int(c["fast_tiles"]), int(c["fast_units"])
        assert 1 <= ft <= 32 and (fu - 1) * ft < tiles <= fu * ft
        sr, su = int(c["slow_rows"]), int(c["slow_units"])
        assert sr % 4 == 0 and 4 <= sr <= 256 and (su - 1) * sr < d_out <= su * sr
        # coherent x after the first wave, coherent y before the last
        assert bool(c["flags"] & 1) == (c["wave"] > 0) and bool(c["flags"] & 2) == (c["wave"] + 1 < W)
        # each call's projection units are contiguous and point back to it
        assert list(unit_call[c["a_begin"]:c["a_begin"] + au]) == [i] * au
    assert h["units_a"] == desc["a_units"].sum() == len(unit_call)
    ub = np.maximum(desc["fast_units"], desc["slow_units"])
    assert h["units_b"] == ub.sum() and h["units_max"] == ub.max()
    assert h["max_k"] == max(8, max(s[2] for s in specs)) and h["max_d"] == max(8, max(s[0] for s in specs))
    # output order: a wave-major permutation, projection units laid out in it,
    # calls with more units first within a wave
    assert sorted(order) == list(range(n))
    assert [desc["wave"][c] for c in order] == sorted(desc["wave"])
    assert list(desc["a_begin"][order]) == list(np.cumsum([0] + list(desc["a_units"][order]))[:-1])
    for w in range(W):
        ow = order[o_begin[w]:o_begin[w + 1]]
        assert all(desc["wave"][c] == w for c in ow) and len(ow) == (desc["wave"] == w).sum()
        assert list(desc["a_units"][ow]) == sorted(desc["a_units"][ow], reverse=True)
        assert p_begin[w] == (desc["a_begin"][ow[0]] if len(ow) else p_begin[w + 1])
    assert p_begin[0] == 0 and p_begin[W] == h["units_a"] and o_begin[W] == n
    # float region: g slots, then the partial rows of each call, all disjoint
    spans = []
    for i, (d, d_out, k, _) in enumerate(specs):
        c = desc[i]
        spans.append((int(c["g_off"]), int(c["g_off"]) + align_up(k, 4), "g"))
        extra = int(c["groups"]) if c["groups"] > 1 else 0
        spans.append((int(c["part_off"]), int(c["part_off"]) + (int(c["a_units"]) + extra) * (k + 4), "p"))
    spans.sort()
    for (a0, a1, _), (b0, _, _) in zip(spans, spans[1:]):
        assert a1 <= b0, "workspace regions overlap"
    assert max(s[1] for s in spans if s[2] == "g") <= min(s[0] for s in spans if s[2] == "p")
    floats_end = int(h["ws_float_off"]) + 4 * max(s[1] for s in spans)
    assert int(h["ws_gate_off"]) < int(h["ws_need_off"]) < int(h["ws_pref_off"]) < int(h["ws_float_off"])
    assert floats_end <= int(h["ws_ctl_off"])
    # control words, then the group counters of two-level sums, inside the workspace
    assert h["ctl_words"] == CTL_HEADER + CTL_PER_WAVE * W + 2 * n
    gcnt = align_up(int(h["ws_ctl_off"]) + 4 * int(h["ctl_words"]), 256)
    assert gcnt + 4 * int(h["units_a"]) <= int(h["ws_bytes"])
    assert gsi.lib().gsi_stack_workspace(plan.ctypes.data) == h["ws_bytes"]
    assert gsi.lib().gsi_stack_status_offset(plan.ctypes.data) == h["ws_ctl_off"]
