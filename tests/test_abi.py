"""C ABI of libgsi without a GPU: symbols, status codes, host-side checks, plans.

Every call here returns before any kernel launch (argument errors or pure
host work), so no device is touched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from rank_gated_memory_amd import gsi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsi.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gsi.LIB_PATH), reason="libgsi.so not built")

GSI_OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_HIP, E_ARG = range(8)
FAKE = 0x7f0000000000  # 256-byte aligned fake device address (never dereferenced)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gsi_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = gsi.lib()
    names = declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"libgsi.so does not export {n}"


TRACE_LIB = os.path.join(ROOT, "rank_gated_memory_amd", "libgsi_trace.so")


@pytest.mark.skipif(not os.path.exists(TRACE_LIB), reason="instrumented build not built")
def test_trace_build_exports_only_there():
    """The per-job trace entry points live in the instrumented build only,
    which also exports every declared symbol; the product library does not
    have them."""
    tr = ctypes.CDLL(TRACE_LIB)
    assert hasattr(tr, "gsi_trace_read") and hasattr(tr, "gsi_trace_reset")
    for n in declared_functions():
        assert hasattr(tr, n), f"libgsi_trace.so does not export {n}"
    L = gsi.lib()
    assert not hasattr(L, "gsi_trace_read") and not hasattr(L, "gsi_trace_reset")


def test_version_and_status_strings():
    assert gsi.gsi_abi_version() == 3
    m = re.search(r"#define GSI_ABI_VERSION (\d+)", open(HEADER).read())
    assert int(m.group(1)) == gsi.gsi_abi_version()
    assert gsi.status_str(0) == "GSI_OK"
    assert gsi.status_str(5) == "GSI_E_WORKSPACE"
    assert gsi.status_str(99) == "GSI_E_UNKNOWN"


def test_image_bytes():
    assert gsi.gsi_image_bytes(512, 16, 0) == 512 * 16 * 4
    assert gsi.gsi_image_bytes(100, 8, 1) == 128 * 8 * 2      # padded to two 64-row tiles
    assert gsi.gsi_image_bytes(12288, 256, 1) == 12288 * 256 * 2
    assert gsi.gsi_image_bytes(0, 8, 1) == 0
    assert gsi.gsi_image_bytes(64, 8, 7) == 0


def mk_map(d=256, d_out=512, k=16, dtype=1, W=FAKE, V=FAKE + 0x100000, M=FAKE + 0x200000):
    return gsi.GsiMapStruct(d, d_out, k, dtype, W, V, M)


def prep(m):
    return gsi.lib().gsi_prepare(ctypes.byref(m), None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=12), E_SHAPE), (dict(d=250), E_SHAPE), (dict(d_out=0), E_SHAPE),
    (dict(k=512, d=256), E_SHAPE), (dict(k=2048, d=4096), E_SHAPE),
    (dict(d=32768, dtype=1), E_SHAPE), (dict(d=16384, dtype=0, k=16), E_SHAPE),
    (dict(dtype=3), E_DTYPE), (dict(W=0), E_NULL), (dict(M=0), E_NULL),
    (dict(V=FAKE + 8), E_ALIGN),
])
def test_prepare_rejects_before_launch(kw, status):
    assert prep(mk_map(**kw)) == status


def test_prepare_null_map():
    assert gsi.lib().gsi_prepare(None, None) == E_NULL


def linear(m, T=1, x=FAKE + 0x300000, y=FAKE + 0x400000, mode=0, ws=FAKE + 0x500000,
           ws_bytes=1 << 30, rho=0, slow=0, eps=0.05):
    return gsi.lib().gsi_linear(ctypes.byref(m), x, y, T, eps, mode, rho, slow, ws, ws_bytes, None)


def test_linear_rejects_before_launch():
    m = mk_map()
    assert linear(m, T=0) == GSI_OK                    # empty batch: nothing to do
    assert linear(m, T=-1) == E_SHAPE
    assert linear(m, mode=3) == E_ARG
    assert linear(m, x=0) == E_NULL
    assert linear(m, ws=0) == E_NULL
    assert linear(m, y=FAKE + 2) == E_ALIGN
    assert linear(m, ws=FAKE + 16) == E_ALIGN
    assert linear(m, rho=FAKE + 1) == E_ALIGN
    need = gsi.lib().gsi_linear_workspace(ctypes.byref(m), 1)
    assert need > 0
    assert linear(m, ws_bytes=need - 1) == E_WS


def test_linear_workspace_grows_with_tokens():
    m = mk_map(d=4096, d_out=12288, k=256)
    L = gsi.lib()
    w1 = L.gsi_linear_workspace(ctypes.byref(m), 1)
    w256 = L.gsi_linear_workspace(ctypes.byref(m), 256)
    w5000 = L.gsi_linear_workspace(ctypes.byref(m), 5000)
    assert 0 < w1 < w256 <= w5000
    assert L.gsi_linear_workspace(ctypes.byref(m), 0) == 0


def calls_array(specs, waves=None, xy=None):
    """specs: (d, d_out, k, dtype) per call; waves: wave per call; xy: (x, y) addresses per call."""
    arr = (gsi.GsiCallStruct * max(len(specs), 1))()
    base = FAKE
    for i, (d, d_out, k, dt) in enumerate(specs):
        mp = gsi.GsiMapStruct(d, d_out, k, dt, base, base + 0x1000000, base + 0x2000000)
        x, y = xy[i] if xy else (base + 0x3000000, base + 0x4000000)
        arr[i] = gsi.GsiCallStruct(mp, x, y, 0.05, waves[i] if waves else 0, 0, 0)
        base += 0x10000000
    return arr


PLAN_HDR = np.dtype([("magic", "<u4"), ("version", "<u4"), ("n", "<i4"), ("dtype", "<i4"),
                     ("units_a", "<i4"), ("units_b", "<i4"), ("max_k", "<i4"), ("max_d", "<i4"),
                     ("ws_bytes", "<u8"), ("desc_off", "<u8"), ("unit_off", "<u8"),
                     ("total_bytes", "<u8"), ("ws_gate_off", "<u8"), ("ws_need_off", "<u8"),
                     ("ws_pref_off", "<u8"), ("ws_float_off", "<u8"), ("ws_ctl_off", "<u8"),
                     ("order_off", "<u8"), ("n_waves", "<i4"), ("ctl_words", "<i4"),
                     ("units_max", "<i4"), ("pad", "<i4")])
DESC = np.dtype([("ptrs", "<u8", 7), ("d", "<i4"), ("d_out", "<i4"), ("k", "<i4"), ("eps", "<f4"),
                 ("a_begin", "<i4"), ("a_units", "<i4"), ("a_rows", "<i4"), ("fast_units", "<i4"),
                 ("slow_units", "<i4"), ("slow_rows", "<i4"), ("part_off", "<i8"), ("g_off", "<i8"),
                 ("gate_off", "<i4"), ("fast_tiles", "<i4"), ("flags", "<i4"), ("wave", "<i4"),
                 ("share_next", "<i4"), ("groups", "<i4"), ("G", "<u8")])


def header(plan):
    return np.frombuffer(plan[:PLAN_HDR.itemsize].tobytes(), dtype=PLAN_HDR)[0]


def build_plan(specs, waves=None, xy=None):
    L = gsi.lib()
    arr = calls_array(specs, waves, xy)
    nb = L.gsi_stack_plan_bytes(arr, len(specs))
    buf = np.zeros(nb + 64, dtype=np.uint8)
    off = (-buf.ctypes.data) % 16
    view = buf[off:off + nb]
    st = L.gsi_stack_plan(arr, len(specs), view.ctypes.data, nb)
    return st, view, nb


def test_stack_plan_layout():
    specs = [(4096, 12288, 256, 1), (4096, 4096, 256, 1), (4096, 16384, 256, 1),
             (16384, 4096, 512, 1)] * 3
    st, plan, nb = build_plan(specs)
    assert st == GSI_OK
    h = header(plan)
    assert PLAN_HDR.itemsize == 128 and DESC.itemsize == 144
    assert h["magic"] == 0x50495347 and h["version"] == 3 and h["n"] == 12 and h["dtype"] == 1
    assert h["n_waves"] == 1
    assert h["total_bytes"] == nb and h["max_k"] == 512 and h["max_d"] == 16384
    uo, ua = int(h["unit_off"]), int(h["units_a"])
    unit_call = np.frombuffer(plan[uo:uo + 4 * ua].tobytes(), "<i4")
    assert len(unit_call) == h["units_a"]
    # every call's units are contiguous; calls with more units (fc_out, d=16384, k=512) come first
    changes = np.flatnonzero(np.diff(unit_call)) + 1
    runs = np.split(unit_call, changes)
    assert sorted(int(r[0]) for r in runs) == list(range(12))
    sizes = [len(r) for r in runs]
    assert sizes == sorted(sizes, reverse=True)
    assert int(runs[0][0]) % 4 == 3
    assert gsi.lib().gsi_stack_workspace(plan.ctypes.data) == h["ws_bytes"] > 0


def test_stack_plan_rejects():
    L = gsi.lib()
    st, _, _ = build_plan([(4096, 4096, 256, 1), (4096, 4096, 256, 0)])
    assert st == E_DTYPE
    st, _, _ = build_plan([(4096, 4096, 12, 1)])
    assert st == E_SHAPE
    arr = calls_array([(256, 512, 16, 0)])
    assert L.gsi_stack_plan(arr, 1, None, 0) == E_NULL
    assert L.gsi_stack_plan_bytes(arr, 5000) == 0
    assert L.gsi_stack_plan(arr, -1, None, 0) == E_SHAPE


def test_stack_rejects_before_launch():
    L = gsi.lib()
    st, plan, nb = build_plan([(256, 512, 16, 0)])
    assert st == GSI_OK
    ws_need = L.gsi_stack_workspace(plan.ctypes.data)
    p = plan.ctypes.data
    assert L.gsi_stack(None, FAKE, 0, FAKE, ws_need, None) == E_NULL
    assert L.gsi_stack(p, FAKE, 4, FAKE, ws_need, None) == E_ARG
    assert L.gsi_stack(p, 0, 0, FAKE, ws_need, None) == E_NULL
    assert L.gsi_stack(p, FAKE, 0, FAKE, ws_need - 1, None) == E_WS
    bad = plan.copy()
    bad[0] ^= 0xFF
    assert L.gsi_stack(bad.ctypes.data, FAKE, 0, FAKE, ws_need, None) == E_ARG
    st0, plan0, _ = build_plan([])
    assert st0 == GSI_OK
    assert L.gsi_stack(plan0.ctypes.data, 0, 0, 0, 0, None) == GSI_OK


def plan_tables(plan):
    h = header(plan)
    n, W = int(h["n"]), int(h["n_waves"])
    desc = np.frombuffer(plan[int(h["desc_off"]):int(h["desc_off"]) + n * DESC.itemsize].tobytes(), DESC)
    uo, ua = int(h["unit_off"]), int(h["units_a"])
    unit_call = np.frombuffer(plan[uo:uo + 4 * ua].tobytes(), "<i4")
    oo = int(h["order_off"])
    tab = np.frombuffer(plan[oo:oo + 4 * (n + 2 * (W + 1))].tobytes(), "<i4")
    return h, desc, unit_call, tab[:n], tab[n:n + W + 1], tab[n + W + 1:]


def test_stack_plan_waves():
    # two GPT-J-shaped layers as four waves: (qkv, fc_in), (out, fc_out), ...
    specs = [(4096, 12288, 256, 1), (4096, 16384, 256, 1), (4096, 4096, 256, 1),
             (16384, 4096, 512, 1)] * 2
    waves = [0, 0, 1, 1, 2, 2, 3, 3]
    st, plan, _ = build_plan(specs, waves)
    assert st == GSI_OK
    h, desc, unit_call, order, p_begin, o_begin = plan_tables(plan)
    assert h["n_waves"] == 4
    assert list(desc["wave"]) == waves
    # agent-coherent x from wave 1 on, coherent y up to the last wave but one
    assert list(desc["flags"] & 1) == [0, 0, 1, 1, 1, 1, 1, 1]
    assert list(desc["flags"] & 2) == [2, 2, 2, 2, 2, 2, 0, 0]
    # output order is wave-major and holds every call once
    assert sorted(order) == list(range(8))
    assert [waves[c] for c in order] == sorted(waves)
    assert list(o_begin) == [0, 2, 4, 6, 8]
    # projection units are wave-major; each wave's range holds exactly its calls' units
    assert p_begin[0] == 0 and p_begin[-1] == h["units_a"]
    for w in range(4):
        calls = set(unit_call[p_begin[w]:p_begin[w + 1]].tolist())
        assert calls == {i for i in range(8) if waves[i] == w}
        assert p_begin[w + 1] - p_begin[w] == sum(desc["a_units"][i] for i in calls)
    for i in range(8):
        assert list(unit_call[desc["a_begin"][i]:desc["a_begin"][i] + desc["a_units"][i]]) == [i] * desc["a_units"][i]
    # control words: header, one block per wave, one open-list entry per call
    assert h["ctl_words"] == 96 + 1088 * 4 + 2 * 8
    assert h["ws_ctl_off"] + 4 * h["ctl_words"] <= h["ws_bytes"]
    assert gsi.lib().gsi_stack_status_offset(plan.ctypes.data) == h["ws_ctl_off"]


def test_stack_plan_wave_numbers_may_skip():
    st, plan, _ = build_plan([(256, 512, 16, 0)] * 3, waves=[0, 5, 5])
    assert st == GSI_OK
    h, desc, *_ = plan_tables(plan)
    assert h["n_waves"] == 2 and list(desc["wave"]) == [0, 1, 1]


def test_stack_plan_rejects_bad_waves_and_aliasing():
    spec = [(256, 512, 16, 0)] * 2
    assert build_plan(spec, waves=[1, 0])[0] == E_ARG       # decreasing
    assert build_plan(spec, waves=[-1, 0])[0] == E_ARG      # negative
    X, Y = FAKE + 0x3000000, FAKE + 0x4000000
    # same wave: y of one call overlaps y of another, or the x of another
    assert build_plan(spec, xy=[(X, Y), (X + 0x10000, Y + 1024)])[0] == E_ARG
    assert build_plan(spec, xy=[(X, Y), (Y + 2032, Y + 0x10000)])[0] == E_ARG
    # x ranges may overlap (reads only), and touching ranges do not overlap
    assert build_plan(spec, xy=[(X, Y), (X + 16, Y + 2048)])[0] == GSI_OK
    assert build_plan(spec, xy=[(X, Y), (Y + 2048, Y + 0x10000)])[0] == GSI_OK
    # across waves, x may be the y of an earlier call (a chain)
    assert build_plan(spec, waves=[0, 1], xy=[(X, Y), (Y, Y + 0x10000)])[0] == GSI_OK
    chain = [(256, 256, 16, 0)] * 3
    assert build_plan(chain, waves=[0, 1, 2], xy=[(X, Y), (Y, X), (X, Y)])[0] == GSI_OK
    assert build_plan(chain, waves=[0, 1, 1], xy=[(X, Y), (Y, X), (X, Y)])[0] == E_ARG


def test_stack_phase_rejects_multi_wave_plans():
    L = gsi.lib()
    st, plan, _ = build_plan([(256, 512, 16, 0)] * 2, waves=[0, 1])
    assert st == GSI_OK
    need = L.gsi_stack_workspace(plan.ctypes.data)
    assert L.gsi_stack_phase(plan.ctypes.data, FAKE, 0, 1, FAKE, need, None) == E_ARG


def test_stack_plan_shares_projections():
    """Calls of one wave with the same x, V_k, d and k share one projection:
    the first owns the units, the others link to it and read its g."""
    X, Y = FAKE + 0x3000000, FAKE + 0x4000000
    L = gsi.lib()
    arr = (gsi.GsiCallStruct * 6)()
    V = FAKE + 0x100000
    specs = [  # (d, d_out, k, V, x, wave)
        (4096, 12288, 256, V, X, 0), (4096, 16384, 256, V, X, 0), (4096, 4096, 256, V + 0x10000000, X, 0),
        (4096, 4096, 256, V, X + 0x100000, 0), (4096, 12288, 256, V, X, 0), (4096, 4096, 256, V, X, 1)]
    for i, (d, do, k, v, x, w) in enumerate(specs):
        mp = gsi.GsiMapStruct(d, do, k, 1, FAKE + 0x20000000 * (i + 1), v, FAKE + 0x20000000 * (i + 1) + 0x10000000)
        arr[i] = gsi.GsiCallStruct(mp, x, Y + 0x100000 * i, 0.05, w, 0, 0)
    nb = L.gsi_stack_plan_bytes(arr, 6)
    buf = np.zeros(nb + 64, dtype=np.uint8)
    off = (-buf.ctypes.data) % 16
    plan = buf[off:off + nb]
    assert L.gsi_stack_plan(arr, 6, plan.ctypes.data, nb) == GSI_OK
    h, desc, unit_call, *_ = plan_tables(plan)
    # calls 0, 1 and 4 share (same x, V, d, k, wave); 2 (other V), 3 (other x), 5 (other wave) do not
    assert list(desc["share_next"]) == [2, 5, 0, 0, 0, 0]
    assert desc["a_units"][1] == 0 and desc["a_units"][4] == 0
    assert all(desc["a_units"][i] > 0 for i in (0, 2, 3, 5))
    assert desc["g_off"][1] == desc["g_off"][0] == desc["g_off"][4]
    assert len(set(desc["g_off"][[0, 2, 3, 5]].tolist())) == 4
    assert set(unit_call.tolist()) == {0, 2, 3, 5}
    assert h["units_a"] == sum(desc["a_units"])


def test_stack_plan_many_projection_units():
    """Latency-bound waves split V_k into 16-row units (bf16, k = 512: 16 KiB
    each), up to 64 per call summed in one level; the last unit may be
    ragged.  A wide V_k that 64 units would cut into pieces above 64 KiB
    (fc_out, 16384 x 512: 256 KiB) gets up to 256 units of 64 KiB, summed in
    two levels (groups of 16).  Partial rows (unit rows plus one per group)
    do not overlap and fit the float region; the group counters fit after
    the control words."""
    specs = [(592, 200, 512, 1), (536, 72, 512, 1), (512, 64, 512, 1), (2048, 128, 512, 1),
             (16384, 4096, 512, 1)]
    st, plan, _ = build_plan(specs, waves=[0, 1, 2, 3, 4])
    assert st == GSI_OK
    h, desc, *_ = plan_tables(plan)
    assert list(desc["a_units"]) == [37, 34, 32, 64, 256]
    assert list(desc["a_rows"]) == [16, 16, 16, 32, 64]
    assert list(desc["groups"]) == [1, 1, 1, 1, 16]
    rows = [int(u) + (int(g) if g > 1 else 0) for u, g in zip(desc["a_units"], desc["groups"])]
    spans = sorted((int(o), int(o) + r * (int(k) + 4)) for o, r, k in zip(desc["part_off"], rows, desc["k"]))
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    assert h["ws_float_off"] + 4 * spans[-1][1] <= h["ws_ctl_off"]
    gcnt = (int(h["ws_ctl_off"]) + 4 * int(h["ctl_words"]) + 255) // 256 * 256
    assert gcnt + 4 * int(h["units_a"]) <= h["ws_bytes"]
    # the 112-map single-wave step keeps one level (fc_out: 43 units of 384 KiB)
    st, plan, _ = build_plan([(4096, 12288, 256, 1), (4096, 4096, 256, 1), (4096, 16384, 256, 1),
                              (16384, 4096, 512, 1)] * 28)
    assert st == GSI_OK
    _, desc, *_ = plan_tables(plan)
    assert set(desc["groups"].tolist()) == {1}


def test_gram_bytes_and_alignment():
    L = gsi.lib()
    assert L.gsi_gram_bytes(256, 1) == 256 * 256 * 2
    assert L.gsi_gram_bytes(16, 0) == 16 * 16 * 4
    assert L.gsi_gram_bytes(0, 1) == 0 and L.gsi_gram_bytes(8, 5) == 0
    m = mk_map()
    m.G = FAKE + 0x600008  # misaligned E
    assert prep(m) == E_ALIGN


def calib(n=512, d=256, k=16, dtype=1, A=FAKE, V0=FAKE + 0x1000000, V=FAKE + 0x2000000, iters=2):
    return gsi.GsiCalibStruct(n, d, k, dtype, A, V0, V, iters, 0)


def test_calibrate_rejects_before_launch():
    L = gsi.lib()
    good = calib()
    need = L.gsi_calibrate_workspace(ctypes.byref(good))
    assert need > 0
    ws = FAKE + 0x3000000
    def run(c, ws=ws, nb=need):
        return L.gsi_calibrate(ctypes.byref(c), ws, nb, None)
    assert L.gsi_calibrate(None, ws, need, None) == E_NULL
    assert run(calib(k=300)) == E_SHAPE        # k > d
    assert run(calib(n=8)) == E_SHAPE          # k > n
    assert run(calib(k=0)) == E_SHAPE
    assert run(calib(dtype=4)) == E_DTYPE
    assert run(calib(iters=-1)) == E_ARG
    assert run(calib(A=0)) == E_NULL
    assert run(calib(V=FAKE + 8)) == E_ALIGN
    assert run(good, ws=0) == E_NULL
    assert run(good, ws=FAKE + 64) == E_ALIGN
    assert run(good, nb=need - 1) == E_WS
    assert L.gsi_calibrate_status_offset() == 0
    # workspace grows with the block
    assert L.gsi_calibrate_workspace(ctypes.byref(calib(n=4096, d=4096, k=256))) > need


def test_static_entry_point_rejects_before_launch():
    """gsi_linear_static checks its arguments (map, sizes, mode, pointers,
    alignment) before it enqueues its clear of the scratch array."""
    L = gsi.lib()
    m = gsi.GsiMapStruct(256, 512, 16, gsi.GSI_FP32, 256, 512, 1024, 0)
    assert L.gsi_static_scratch_bytes() == 64 << 20
    st = lambda mm, x, y, T, mode=0, rho=0: L.gsi_linear_static(ctypes.byref(mm), x, y, T, ctypes.c_float(0.05),
                                                              mode, rho, 0, 0)  # noqa: E731
    assert st(m, 4096, 4096, 0) == 0                     # T = 0: nothing to do
    assert st(m, 4096, 4096, -1) == 2                    # GSI_E_SHAPE
    assert st(m, 4096, 4096, 4, mode=3) == 7             # GSI_E_ARG
    assert st(m, 0, 4096, 4) == 1                        # GSI_E_NULL
    assert st(m, 4104, 4096, 4) == 4                     # x not 16-byte aligned
    assert st(m, 4096, 4096, 4, rho=4098) == 4           # rho not 4-byte aligned
    bad = gsi.GsiMapStruct(255, 512, 16, gsi.GSI_FP32, 256, 512, 1024, 0)
    assert st(bad, 4096, 4096, 4) == 2                   # d not a multiple of 8
    big = gsi.GsiMapStruct(16384, 64, 1024, gsi.GSI_BF16, 256, 512, 1024, 0)
    assert st(big, 4096, 4096, 4096) == 5                # workspace beyond the array
