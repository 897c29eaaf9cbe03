"""The entry points enqueue kernels only (no allocation, memset or synchronisation),
so a caller can capture them in a HIP graph.  Each capture here is replayed several
times with eager work and synchronisations between the replays, and every replay
is checked bit for bit against the eager result; the two-call step, the loss form and
the one-call step (plain and reduced) are captured.  Two calls on two streams with
their own workspaces run concurrently and match sequential results (the library
keeps no state between calls), for the two calls and for the one call."""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def jsd_step(v, sh, shg, beta, part, stats, kl, loss, g):
    v.vjsd_forward(sh, beta, part, stats, kl, loss)
    v.vjsd_bwd(shg, stats, kl, beta, g, part)


@pytest.mark.parametrize("V,beta", [(16032, 0.5), (20000, 0.3), (4000, 0.0)])
def test_graph_replays_match_eager(V, beta):
    v = vj()
    N = 256
    b = synth.draw("full_vocab", device="cuda", N=N, V=V)
    part = v.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), device="cuda")
    loss = torch.empty(N, device="cuda")
    gs, gt = torch.empty_like(b.s), torch.empty_like(b.t)
    sh = v.ShardSet(b.s, b.t)
    shg = v.ShardSet(b.s, b.t, gs=gs, gt=gt)
    jsd_step(v, sh, shg, beta, part, stats, kl, loss, b.gout)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (stats, kl, loss, gs, gt)]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            jsd_step(v, sh, shg, beta, part, stats, kl, loss, b.gout)
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        for x in (stats, kl, loss, gs, gt):
            x.fill_(float("nan")) if x.dtype.is_floating_point else x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("stats", "kl", "loss", "gs", "gt"), (stats, kl, loss, gs, gt), ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs"
        # eager work between replays
        jsd_step(v, sh, shg, beta, part, stats, kl, loss, b.gout)
        torch.cuda.synchronize()


def test_graph_replays_of_the_loss_form():
    v = vj()
    N = 192
    b = synth.draw("full_vocab", device="cuda", N=N, V=12000)
    keep = (torch.arange(N, device="cuda") % 3 != 0).to(torch.uint8)
    opts = v.loss_opts(N, 2.0, True, keep, "mean")
    part = v.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), device="cuda")
    rows = torch.empty(N, device="cuda")
    out = torch.empty(1, device="cuda")
    g = torch.ones(1, device="cuda")
    gs = torch.empty_like(b.s)
    sh = v.ShardSet(b.s, b.t)
    shg = v.ShardSet(b.s, b.t, gs=gs)

    def step():
        v.vjsd_loss_forward(sh, 0.5, opts, part, stats, kl, rows, out)
        v.vjsd_loss_backward(shg, 0.5, opts, stats, kl, g, part)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (rows, out, gs)]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            step()
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        for x in (rows, out, gs):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("rows", "out", "gs"), (rows, out, gs), ref):
            assert torch.equal(x, r), f"replay {rep}: {name} differs"
        step()
        torch.cuda.synchronize()


def test_concurrent_streams_with_separate_workspaces():
    v = vj()
    N = 512
    a = synth.draw("full_vocab", device="cuda", N=N, V=20000, seed=1)
    c = synth.draw("full_vocab", device="cuda", N=N, V=16032, seed=2)

    def buffers(b):
        return dict(part=v.new_part(N, 1, "cuda"),
                    stats=torch.empty((N, 4), dtype=torch.float64, device="cuda"),
                    kl=torch.empty((N, 2), device="cuda"), loss=torch.empty(N, device="cuda"),
                    gs=torch.empty_like(b.s), gt=torch.empty_like(b.t))

    def run(b, x, stream=None):
        sh = v.ShardSet(b.s, b.t)
        shg = v.ShardSet(b.s, b.t, gs=x["gs"], gt=x["gt"])
        v.vjsd_forward(sh, 0.5, x["part"], x["stats"], x["kl"], x["loss"], stream)
        v.vjsd_bwd(shg, x["stats"], x["kl"], 0.5, b.gout, x["part"], stream)

    xa, xc = buffers(a), buffers(c)
    run(a, xa)
    run(c, xc)
    torch.cuda.synchronize()
    ref_a = {k: t.clone() for k, t in xa.items() if k != "part"}
    ref_c = {k: t.clone() for k, t in xc.items() if k != "part"}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        run(a, xa, s1)
        run(c, xc, s2)
    torch.cuda.synchronize()
    for k in ref_a:
        assert torch.equal(xa[k], ref_a[k]), k
        assert torch.equal(xc[k], ref_c[k]), k


@pytest.mark.parametrize("V,opts", [(16032, None), (50000, None),
                                    (12000, dict(temperature=2.0, scale_t2=True,
                                                 reduction="mean"))])
def test_graph_replays_of_the_one_call(V, opts):
    """vjsd_forward_backward (register-held and two-sweep rows) and the reduced loss form
    in one call (its kept-row count, the one launch, the reduction) captured and
    replayed, each replay bit for bit the eager result, with eager calls between."""
    v = vj()
    N = 256
    b = synth.draw("full_vocab", device="cuda", N=N, V=V)
    part = v.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), device="cuda")
    loss = torch.empty(N, device="cuda")
    out = torch.empty(1, device="cuda")
    gs, gt = torch.empty_like(b.s), torch.empty_like(b.t)
    shg = v.ShardSet(b.s, b.t, gs=gs, gt=gt)
    o = None if opts is None else v.loss_opts(N, **opts)
    g1 = torch.full((1,), 0.5, device="cuda")

    def step():
        if o is None:
            v.vjsd_forward_backward(shg, 0.4, b.gout, part, stats, kl, loss)
        else:
            v.vjsd_loss_forward_backward(shg, 0.4, o, g1, part, stats, kl, loss, out)

    outs = (stats, kl, loss, gs, gt) + (() if o is None else (out,))
    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(graph, stream=st):
            step()
    torch.cuda.current_stream().wait_stream(st)
    for rep in range(4):
        for x in outs:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (x, r) in enumerate(zip(outs, ref)):
            assert torch.equal(x, r), f"replay {rep}: output {i} differs"
        step()
        torch.cuda.synchronize()


def test_concurrent_streams_one_call():
    """Two one-call steps on two streams, each with its own workspace and outputs,
    match the sequential results."""
    v = vj()
    N = 512
    a = synth.draw("full_vocab", device="cuda", N=N, V=50000, seed=3)
    c = synth.draw("full_vocab", device="cuda", N=N, V=16032, seed=4)

    def buffers(b):
        return dict(part=v.new_part(N, 1, "cuda"),
                    stats=torch.empty((N, 4), dtype=torch.float64, device="cuda"),
                    kl=torch.empty((N, 2), device="cuda"), loss=torch.empty(N, device="cuda"),
                    gs=torch.empty_like(b.s), gt=torch.empty_like(b.t))

    def run(b, x, stream=None):
        shg = v.ShardSet(b.s, b.t, gs=x["gs"], gt=x["gt"])
        v.vjsd_forward_backward(shg, 0.5, b.gout, x["part"], x["stats"], x["kl"], x["loss"],
                                stream)

    xa, xc = buffers(a), buffers(c)
    run(a, xa)
    run(c, xc)
    torch.cuda.synchronize()
    ref_a = {k: t.clone() for k, t in xa.items() if k != "part"}
    ref_c = {k: t.clone() for k, t in xc.items() if k != "part"}
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        run(a, xa, s1)
        run(c, xc, s2)
    torch.cuda.synchronize()
    for k in ref_a:
        assert torch.equal(xa[k], ref_a[k]), k
        assert torch.equal(xc[k], ref_c[k]), k
