"""GPU parity of dependency-chained stacks (calls in waves, later waves
reading earlier outputs) against the oracle's chain evaluation.

The stacks follow the GPT-J parallel block made synthetic (GSI-TS §2.3, §3):
per layer, wave 2l runs qkv and fc_in on the layer input, wave 2l+1 runs out
on the value third of qkv's output and fc_out on fc_in's output, whose output
is the next layer's input.  Several independent token streams ("chains")
share the maps; some start with a large residual (slow path).  Calls go
through the C ABI (gsi_stack, one launch per stack).
"""
import os

import numpy as np
import pytest
import torch

from oracle import gsi_oracle as orc
from rank_gated_memory_amd import gsi, synth
from tests.parity import GATE_BAND, TOL, eps32, f64

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
STORE = {torch.float32: "fp32", torch.bfloat16: "bf16"}


def sync():
    torch.cuda.synchronize()


def build_chain(dtype, d=256, k=32, f=512, kf=64, layers=3, chains=4, slow_chains=(1, 3), eps=0.05,
                seed=0):
    """GPU stack plan, its output tensors and the matching oracle call list."""
    cfg, (vh0, uh0) = synth.chain_config(d, k, f, kf, layers, (96, seed), dtype=dtype)
    mask = torch.tensor([c in slow_chains for c in range(chains)])
    X0, _ = synth.tokens(vh0, uh0, mask, (96, seed, 99), rho_slow=(0.2, 0.5))
    X0 = X0.to(dtype)
    maps, host = {}, {}
    for l, layer in enumerate(cfg):
        for role, (W, V) in layer.maps.items():
            m = gsi.Map(W.to(DEV).contiguous(), V.to(DEV).contiguous())
            gsi.gsi_prepare(m)
            maps[(l, role)] = m
            Wf, Vf = f64(W), f64(V)
            host[(l, role)] = (Wf, Vf, orc.prepare(Wf, Vf))
    gpu_calls, orc_calls, outs = [], [], []

    def add(l, role, chain, wave, x_t, src):
        m = maps[(l, role)]
        y = torch.empty(m.d_out, dtype=dtype, device=DEV)
        r = torch.empty(1, dtype=torch.float32, device=DEV)
        s = torch.empty(1, dtype=torch.uint8, device=DEV)
        gpu_calls.append((m, x_t, y, eps, r, s, wave))
        W, V, M = host[(l, role)]
        c = {"W": W, "V": V, "M": M, "eps": eps32(eps)}
        if src is None:
            c["x"] = f64(x_t)
        else:
            c["src"] = src
        orc_calls.append(c)
        outs.append((l, role, chain, y, r, s))
        return len(gpu_calls) - 1, y

    h = [(None, X0[c].to(DEV)) for c in range(chains)]  # (producing call, tensor)
    for l in range(layers):
        qkv, fcin = [], []
        for c in range(chains):
            src = None if h[c][0] is None else (h[c][0], 0)
            qkv.append(add(l, "qkv", c, 2 * l, h[c][1], src))
            fcin.append(add(l, "fc_in", c, 2 * l, h[c][1], src))
        nh = []
        for c in range(chains):
            iq, yq = qkv[c]
            add(l, "out", c, 2 * l + 1, yq[2 * d:3 * d], (iq, 2 * d))
            nh.append(add(l, "fc_out", c, 2 * l + 1, fcin[c][1], (fcin[c][0], 0)))
        h = nh
    return gsi.Stack(gpu_calls), outs, orc_calls


def check_chain(outs, ref, dtype, what):
    tol = TOL[dtype]
    worst = 0.0
    for i, ((l, role, c, y, r, s), o) in enumerate(zip(outs, ref)):
        where = f"{what} call {i} (layer {l} {role} chain {c})"
        assert abs(o["rho"] - 0.05) >= GATE_BAND, f"{where}: test data too close to the threshold"
        assert bool(int(s.item())) == bool(o["slow"]), f"{where}: gate gpu={int(s.item())} oracle rho={o['rho']:.5f}"
        assert abs(float(r.item()) - o["rho"]) <= 2e-2, f"{where}: rho {float(r.item())} vs {o['rho']}"
        err = np.linalg.norm(f64(y) - o["y"]) / np.linalg.norm(o["y"])
        worst = max(worst, err)
        assert err <= tol, f"{where}: rel L2 {err:.3e} > {tol}"
    return worst


@pytest.mark.parametrize("chains,slow_chains", [(4, (1, 3)), (2, (1,))], ids=["8-call-waves", "4-call-waves"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_chained_stack_matches_oracle_chain(dtype, chains, slow_chains):
    """Waves of 8 calls hand out output units through the open list; waves of
    at most 4 calls number their output tickets statically (each call's tiles,
    then its further slow units) and publish each gate in a word of its own.
    Both with fast and slow calls in every wave."""
    st, outs, calls = build_chain(dtype, chains=chains, slow_chains=slow_chains)
    ws = st.run()
    sync()
    ref = orc.chain(calls, STORE[dtype])
    slow = [bool(o["slow"]) for o in ref]
    assert any(slow) and not all(slow)
    worst = check_chain(outs, ref, dtype, f"chain {STORE[dtype]}")
    assert st.status(ws) == 0
    # the same bits on a second run over the same workspace
    y0 = [o[3].clone() for o in outs]
    st.run(ws=ws)
    sync()
    assert all(torch.equal(o[3], a) for o, a in zip(outs, y0))
    print(f"{STORE[dtype]}: {len(outs)} calls in {2 * 3} waves of {2 * chains}, worst rel L2 {worst:.2e}")


def test_chained_stack_forced_modes():
    st, outs, calls = build_chain(torch.bfloat16, layers=2, chains=2, slow_chains=(1,))
    ws = gsi.workspace(st.ws_bytes, DEV)
    for mode in (gsi.FORCE_FAST, gsi.FORCE_SLOW):
        gsi.gsi_stack(st, mode, ws)
        sync()
        ref = orc.chain(calls, "bf16", mode)
        for i, ((l, role, c, y, r, s), o) in enumerate(zip(outs, ref)):
            assert int(s.item()) == (mode == gsi.FORCE_SLOW)
            err = np.linalg.norm(f64(y) - o["y"]) / np.linalg.norm(o["y"])
            assert err <= 2e-2, f"mode {mode} call {i}: rel L2 {err:.3e}"
    assert st.status(ws) == 0


def test_many_chains_max_calls():
    """4096 calls (the plan maximum): 1024 token streams through 4 chained maps."""
    d, k, n, waves = 64, 8, 1024, 4
    frames = [synth.orthonormal_frame(d, k, 32 if w == 0 else 0, (97, w, 0, 1)) for w in range(waves + 1)]
    mask = synth.pick_slow(n, n // 4, (97, 0, 0, 2))
    X0, _ = synth.tokens(frames[0][0], frames[0][1], mask, (97, 0, 0), rho_slow=(0.2, 0.5))
    X0 = X0.float().to(DEV)
    maps, host = [], []
    for w in range(waves):
        W = synth.subspace_map(frames[w][0], frames[w + 1][0], (97, w, 0, 3), dtype=torch.float32)
        V = frames[w][0].float()
        m = gsi.Map(W.to(DEV), V.to(DEV).contiguous())
        gsi.gsi_prepare(m)
        maps.append(m)
        host.append((f64(W), f64(V), orc.prepare(f64(W), f64(V))))
    Y = torch.empty((waves, n, d), dtype=torch.float32, device=DEV)
    R = torch.empty((waves, n), dtype=torch.float32, device=DEV)
    S = torch.empty((waves, n), dtype=torch.uint8, device=DEV)
    gpu_calls, orc_calls = [], []
    for w in range(waves):
        for t in range(n):
            x = X0[t] if w == 0 else Y[w - 1, t]
            gpu_calls.append((maps[w], x, Y[w, t], 0.05, R[w, t:t + 1], S[w, t:t + 1], w))
            c = {"W": host[w][0], "V": host[w][1], "M": host[w][2], "eps": eps32(0.05)}
            if w == 0:
                c["x"] = f64(X0[t])
            else:
                c["src"] = ((w - 1) * n + t, 0)
            orc_calls.append(c)
    st = gsi.Stack(gpu_calls)
    assert st.n == 4096
    ws = st.run()
    sync()
    ref = orc.chain(orc_calls, "fp32")
    Sg, Rg, Yg = S.cpu().numpy().reshape(-1), R.cpu().numpy().reshape(-1), f64(Y).reshape(waves * n, d)
    for i, o in enumerate(ref):
        assert abs(o["rho"] - 0.05) >= GATE_BAND
        assert bool(Sg[i]) == bool(o["slow"]), f"call {i}: gate"
        err = np.linalg.norm(Yg[i] - o["y"]) / np.linalg.norm(o["y"])
        assert err <= 1e-5, f"call {i}: rel L2 {err:.3e}"
    assert Sg.sum() > 0 and Sg.sum() < len(Sg)
    assert st.status(ws) == 0


def test_exhausted_wait_bound_drains_and_recovers(monkeypatch):
    """A device-side wait bound of zero makes waits give up: the launch still
    ends, the status word records it, and the next run (normal bound) on the
    same workspace is complete and correct."""
    st, outs, calls = build_chain(torch.float32, layers=3, chains=4)
    ws = gsi.workspace(st.ws_bytes, DEV)
    monkeypatch.setenv("GSI_SPIN_LIMIT", "0")
    with pytest.raises(gsi.StackIncomplete):
        gsi.gsi_stack(st, gsi.GATED, ws, check=True)
    assert st.status(ws) != 0, "no wait ran out with a zero bound"
    ws[st.status_offset:st.status_offset + 4] = 0
    monkeypatch.delenv("GSI_SPIN_LIMIT")
    for o in outs:
        o[3].fill_(float("nan"))
    gsi.gsi_stack(st, gsi.GATED, ws, check=True)
    assert st.status(ws) == 0
    check_chain(outs, orc.chain(calls, "fp32"), torch.float32, "after recovery")


def test_exhausted_wait_bound_recovers_two_level_sums(monkeypatch):
    """The same with a wide basis in the second wave (16384 x 512: 256
    projection units whose partials are summed in two levels, groups of 16):
    a launch whose bound ran out may leave a group of partials half counted,
    and the next runs on the same workspace still give the bits of a run that
    never failed."""
    bf = torch.bfloat16
    WA = synth.gaussian_weight(16384, 512, (98, 1, 0, 0), dtype=bf)
    vA, uA = synth.orthonormal_frame(512, 64, 16, (98, 1, 0, 1))
    WB = synth.gaussian_weight(4096, 16384, (98, 1, 1, 0), dtype=bf)
    vB, _ = synth.orthonormal_frame(16384, 512, 0, (98, 1, 1, 1))
    xA, _ = synth.tokens(vA, uA, torch.tensor([False]), (98, 1, 2))
    mA, mB = gsi.Map(WA.to(DEV), vA.to(bf).to(DEV)), gsi.Map(WB.to(DEV), vB.to(bf).to(DEV))
    gsi.gsi_prepare(mA)
    gsi.gsi_prepare(mB)
    x = xA[0].to(bf).to(DEV)
    yA = torch.empty(16384, dtype=bf, device=DEV)
    yB = torch.empty(4096, dtype=bf, device=DEV)
    st = gsi.Stack([(mA, x, yA, 0.05, None, None, 0), (mB, yA, yB, 0.05, None, None, 1)])
    ws = gsi.workspace(st.ws_bytes, DEV)
    gsi.gsi_stack(st, gsi.GATED, ws, check=True)
    sync()
    ref = (yA.clone(), yB.clone())
    monkeypatch.setenv("GSI_SPIN_LIMIT", "0")
    with pytest.raises(gsi.StackIncomplete):
        gsi.gsi_stack(st, gsi.GATED, ws, check=True)
    ws[st.status_offset:st.status_offset + 4] = 0
    monkeypatch.delenv("GSI_SPIN_LIMIT")
    for _ in range(3):
        yA.fill_(float("nan"))
        yB.fill_(float("nan"))
        gsi.gsi_stack(st, gsi.GATED, ws, check=True)
        sync()
        assert torch.equal(yA, ref[0]) and torch.equal(yB, ref[1])
    assert st.status(ws) == 0
