"""The library's calls captured in HIP graphs and replayed (GPU).

A decode loop captures its step once and replays it, so every call must leave
its workspace ready for the next run without a memset (the kernels clear
their own counters and control words) and a replay must give the eager
result bit for bit.  Each graph here is replayed several times with eager
work and host synchronisation between the replays; before each replay the
outputs are overwritten, so that a unit that did not run shows, and every
replay is compared with the eager run."""
import pytest
import torch

from rank_gated_memory_amd import gsi, synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 4


def new_map(W, V):
    m = gsi.Map(W.to(DEV).contiguous(), V.to(DEV).contiguous())
    gsi.gsi_prepare(m)
    return m


def map_and_tokens(d, d_out, k, n_tok, slow_every, dtype, seed):
    W = synth.gaussian_weight(d_out, d, (98, seed, 0, 0), dtype=dtype)
    v, u = synth.orthonormal_frame(d, k, 16, (98, seed, 0, 1))
    mask = torch.tensor([t % slow_every == slow_every - 1 for t in range(n_tok)])
    X, _ = synth.tokens(v, u, mask, (98, seed, 0))
    return new_map(W, v.to(dtype)), X.to(dtype).to(DEV).contiguous()


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else (t.view(torch.int32) if t.element_size() == 4 else t)


def check_replays(issue, outs, status=None):
    """issue(): enqueue the calls on the current stream; outs: what they write;
    status(): the device status word to read after each run, if any."""
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        issue()
    stream.synchronize()
    ref = [o.clone() for o in outs]
    if status is not None:
        assert status() == 0
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        issue()
    torch.cuda.synchronize()
    junk = torch.ones(1 << 20, device=DEV)
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(7 if o.dtype == torch.uint8 else float("nan"))
        junk.mul_(1.5).add_(float(r))  # the program's own eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
        stream.synchronize()
        for i, (o, want) in enumerate(zip(outs, ref)):
            assert torch.equal(bits(o), bits(want)), f"replay {r}: output {i} differs from the eager run"
        if status is not None:
            assert status() == 0, f"replay {r}: status word set"
    del g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_stack_plans_replay_in_graphs(dtype):
    """A two-wave chained plan (wave 1 reads wave 0's outputs, latency-bound
    waves) and a one-wave plan of 24 calls (open-list tickets)."""
    ma, xa = map_and_tokens(512, 1024, 64, 4, 2, dtype, 1)
    mb, _ = map_and_tokens(1024, 512, 64, 1, 2, dtype, 2)
    ya = torch.empty(4, 1024, dtype=dtype, device=DEV)
    yb = torch.empty(4, 512, dtype=dtype, device=DEV)
    rho = torch.empty(8, dtype=torch.float32, device=DEV)
    sl = torch.empty(8, dtype=torch.uint8, device=DEV)
    calls = [(ma, xa[t], ya[t], 0.05, rho[t:t + 1], sl[t:t + 1], 0) for t in range(4)]
    calls += [(mb, ya[t], yb[t], 0.05, rho[4 + t:5 + t], sl[4 + t:5 + t], 1) for t in range(4)]
    st = gsi.Stack(calls)
    ws = gsi.workspace(st.ws_bytes, DEV)
    check_replays(lambda: gsi.gsi_stack(st, gsi.GATED, ws), [ya, yb, rho, sl], lambda: st.status(ws))
    assert int(sl[:4].sum()) == 2  # every other token of wave 0 takes the slow path

    mc, xc = map_and_tokens(768, 1536, 128, 24, 3, dtype, 3)
    yc = torch.empty(24, 1536, dtype=dtype, device=DEV)
    rc = torch.empty(24, dtype=torch.float32, device=DEV)
    sc = torch.empty(24, dtype=torch.uint8, device=DEV)
    st1 = gsi.Stack([(mc, xc[t], yc[t], 0.05, rc[t:t + 1], sc[t:t + 1]) for t in range(24)])
    ws1 = gsi.workspace(st1.ws_bytes, DEV)
    check_replays(lambda: gsi.gsi_stack(st1, gsi.GATED, ws1), [yc, rc, sc], lambda: st1.status(ws1))
    assert int(sc.sum()) == 8


def test_batched_linear_replays_in_graphs():
    """T = 64 bf16 tokens, a quarter slow (row streams for both paths), and
    T = 256 with a third slow (wide items and tiles)."""
    for n_tok, every, seed in ((64, 4, 4), (256, 3, 5)):
        m, X = map_and_tokens(1024, 2048, 128, n_tok, every, torch.bfloat16, seed)
        y = torch.empty(n_tok, 2048, dtype=torch.bfloat16, device=DEV)
        rho = torch.empty(n_tok, dtype=torch.float32, device=DEV)
        sl = torch.empty(n_tok, dtype=torch.uint8, device=DEV)
        ws = gsi.workspace(gsi.gsi_linear_workspace(m, n_tok), DEV)
        check_replays(lambda: gsi.gsi_linear(m, X, 0.05, y=y, rho=rho, slow=sl, ws=ws), [y, rho, sl])
        assert int(sl.sum()) == n_tok // every


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_single_token_calls_replay_in_graphs(dtype):
    """Eight T = 1 calls in one graph on one workspace, and the same through
    gsi_linear_static (the library's own device array as workspace)."""
    m, X = map_and_tokens(1024, 1536, 64, 8, 4, dtype, 6)
    y = torch.empty(8, 1536, dtype=dtype, device=DEV)
    rho = torch.empty(8, dtype=torch.float32, device=DEV)
    sl = torch.empty(8, dtype=torch.uint8, device=DEV)
    ws = gsi.workspace(gsi.gsi_linear_workspace(m, 1), DEV)

    def issue():
        for t in range(8):
            gsi.gsi_linear(m, X[t:t + 1], 0.05, y=y[t:t + 1], rho=rho[t:t + 1], slow=sl[t:t + 1], ws=ws)

    check_replays(issue, [y, rho, sl])
    assert int(sl.sum()) == 2
    y_ws = y.clone()

    def issue_static():
        for t in range(8):
            gsi.gsi_linear_static(m, X[t:t + 1], 0.05, y=y[t:t + 1], rho=rho[t:t + 1], slow=sl[t:t + 1])

    check_replays(issue_static, [y, rho, sl])
    assert torch.equal(bits(y), bits(y_ws))
