"""GPU parity of the sibling ops on the statistics engine -- single-pass KL, entropy,
per-id / top-k log-probabilities -- against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_stats, assert_values

pytestmark = pytest.mark.gpu

NINF = float("-inf")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def run_kl(s, t, reverse, widths=None, gout=None, want_t=False):
    v = vj()
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    part = v.new_part(N, S, s.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=s.device)
    kl = torch.empty((N, 2), dtype=torch.float32, device=s.device)
    loss = torch.empty((N,), dtype=torch.float32, device=s.device)
    v.vkl_fwd(sh, reverse, part, stats, kl, loss)
    gs = torch.full_like(s, float("nan"))
    gt = torch.full_like(t, float("nan")) if want_t else None
    gout = torch.ones(N, device=s.device) if gout is None else gout
    v.vkl_bwd(v.ShardSet(s, t, widths=widths, gs=gs, gt=gt), reverse, stats, kl, gout, part)
    torch.cuda.synchronize()
    return dict(stats=stats.cpu(), kl=kl.cpu(), loss=loss.cpu(), gs=gs.cpu(),
                gt=None if gt is None else gt.cpu())


def check_kl(s, t, reverse, widths=None, gout=None, want_t=False):
    dt = s.dtype
    g = run_kl(s, t, reverse, widths, gout, want_t)
    sc, tc = s.cpu().contiguous(), t.cpu().contiguous()
    ref = oracle.kl_div(sc, tc, reverse=reverse, widths=widths,
                        gout=None if gout is None else gout.cpu().double().numpy())
    assert_stats(g["stats"], *oracle.stats(sc, widths=widths), 0, "student stats")
    assert_stats(g["stats"], *oracle.stats(tc, widths=widths), 1, "teacher stats")
    assert_values(g["loss"], ref["loss"], dt, "KL")
    assert_values(g["kl"][:, 1 if reverse else 0], ref["loss"], dt, "saved KL")
    assert np.all(g["kl"][:, 0 if reverse else 1].numpy()[np.isfinite(ref["loss"])] == 0.0)
    fin = np.isfinite(ref["loss"])
    undefined = np.isnan(ref["loss"])
    # the student is the target side of reverse KL: compare it on finite rows only
    rows = fin | undefined if reverse else np.ones_like(fin)
    masked_s = ~np.isfinite(sc.double().numpy())
    assert_grads(g["gs"][rows], ref["gs"][rows], dt, "d/ds",
                 exact_zero=(ref["gs"][rows] == 0.0) & (masked_s[rows] | undefined[rows][:, None]))
    if want_t:
        rows_t = np.ones_like(fin) if reverse else (fin | undefined)
        assert_grads(g["gt"][rows_t], ref["gt"][rows_t], dt, "d/dt")
    return g, ref


@pytest.mark.parametrize("reverse", [False, True])
def test_kl_tiny_fp32(reverse):
    b = synth.draw("tiny", device="cuda")
    check_kl(b.s, b.t, reverse, gout=b.gout, want_t=True)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("reverse", [False, True])
def test_kl_siblings_recipe_teacher_detached(dtype, reverse):
    b = synth.draw("siblings", device="cuda", N=16, dtype=dtype)
    check_kl(b.s, b.t, reverse, gout=b.gout)


@pytest.mark.parametrize("reverse", [False, True])
def test_kl_masks_offsets_and_shards(reverse):
    w = list(synth.WORKLOADS["robust"].widths)
    b = synth.draw("robust", device="cuda", N=100)
    s, t = b.s.clone(), b.t.clone()
    s[5, 70000] = NINF  # forward KL of row 5 becomes +inf (teacher mass there unless masked)
    t[5, 70000] = 0.0
    g, ref = check_kl(s, t, reverse, widths=w, gout=b.gout, want_t=True)
    if not reverse:
        assert np.isinf(g["loss"].numpy()[5])
    g1 = run_kl(s, t, reverse, None, b.gout)
    fin = np.isfinite(g["loss"].numpy())
    np.testing.assert_allclose(g1["loss"].numpy()[fin], g["loss"].numpy()[fin], rtol=1e-5,
                               atol=1e-6)


def test_kl_matches_the_jsd_endpoint_branches():
    v = vj()
    b = synth.draw("siblings", device="cuda", N=24, V=5000)
    for reverse, beta in ((False, 0.0), (True, 1.0)):
        a = v.kl_div(b.s, b.t, reverse=reverse)
        c = v.jsd(b.s, b.t, beta)
        torch.testing.assert_close(a, c, rtol=2e-5, atol=2e-6)


# ---- entropy ---------------------------------------------------------------------------

def run_entropy(x, widths=None, gout=None):
    v = vj()
    sh = v.ShardSet(x, widths=widths)
    N, S = sh.N, sh.S
    part = v.new_part(N, S, x.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=x.device)
    ent = torch.empty((N,), dtype=torch.float32, device=x.device)
    v.ventropy_fwd(sh, part, stats, ent)
    gx = torch.full_like(x, float("nan"))
    gout = torch.ones(N, device=x.device) if gout is None else gout
    v.ventropy_bwd(v.ShardSet(x, widths=widths, gs=gx), stats, ent, gout, part)
    torch.cuda.synchronize()
    return dict(stats=stats.cpu(), ent=ent.cpu(), gx=gx.cpu())


@pytest.mark.parametrize("name,dtype,widths", [
    ("tiny", torch.float32, None),
    ("siblings", torch.float16, None),
    ("siblings", torch.bfloat16, [70000, 0, 58256]),
    ("robust", torch.float32, [60000, 0, 40000, 28256]),
])
def test_entropy(name, dtype, widths):
    b = synth.draw(name, device="cuda", N=40 if name != "tiny" else None, dtype=dtype)
    x = b.s.clone()
    x[3] = NINF  # an undefined row
    x[4, ::3] = NINF  # a partly masked row
    g = run_entropy(x, widths, b.gout)
    ref = oracle.entropy(x.cpu(), widths=widths, gout=b.gout.cpu().double().numpy())
    assert_stats(g["stats"], *oracle.stats(x.cpu(), widths=widths), 0, "stats")
    assert_values(g["ent"], ref["ent"], dtype, "entropy")
    masked = ~np.isfinite(x.cpu().double().numpy())
    assert_grads(g["gx"], ref["gx"], dtype, "d/dx", exact_zero=masked)


def test_entropy_closed_forms():
    v = vj()
    V = 4099
    x = torch.zeros(3, V, device="cuda")
    x[1] = NINF
    x[1, 17] = 2.0
    x[2, : V // 2] = NINF
    e = v.entropy(x).cpu().double().numpy()
    np.testing.assert_allclose(e, [np.log(V), 0.0, np.log(V - V // 2)], rtol=2e-6, atol=1e-6)


# ---- log-probabilities --------------------------------------------------------------------

def run_logprobs(x, ids, ignore=-100, widths=None, gout=None):
    v = vj()
    sh = v.ShardSet(x, widths=widths)
    N, S = sh.N, sh.S
    K = ids.shape[-1]
    part = v.new_part(N, S, x.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=x.device)
    out = torch.full((N, K), float("nan"), device=x.device)
    err = torch.zeros(1, dtype=torch.int32, device=x.device)
    v.vlogprobs_fwd(sh, sh.V, ids, ignore, part, stats, out, err)
    gx = torch.full_like(x, float("nan"))
    gout = torch.ones((N, K), device=x.device) if gout is None else gout
    v.vlogprobs_bwd(v.ShardSet(x, widths=widths, gs=gx), sh.V, stats, ids, ignore, gout, part)
    torch.cuda.synchronize()
    return dict(stats=stats.cpu(), out=out.cpu(), gx=gx.cpu(), err=int(err.item()))


@pytest.mark.parametrize("dtype,widths", [
    (torch.float16, None), (torch.bfloat16, None), (torch.bfloat16, [40000, 88256]),
    (torch.float32, [1, 128254, 1]),
])
def test_topk_logprobs(dtype, widths):
    b = synth.draw("siblings", device="cuda", N=24, dtype=dtype)
    ids = b.ids.clone()
    ids[0, 1] = ids[0, 0]  # a repeated id accumulates its gradient
    ids[1, :] = -100  # a row of ignored ids
    ids[2, 0] = 128255  # the last and first ids of the vocabulary
    ids[2, 1] = 0
    x = b.s.clone()
    x[3] = NINF  # undefined row: NaN for valid ids, 0 for ignored, zero gradient
    g = run_logprobs(x, ids, -100, widths, b.gids)
    assert g["err"] == 0
    ref = oracle.logprobs(x.cpu(), ids.cpu().numpy(), -100, widths=widths,
                          gout=b.gids.cpu().double().numpy())
    ign = ids.cpu().numpy() == -100
    assert np.all(g["out"].numpy()[ign] == 0.0)
    assert_values(g["out"], ref["out"], dtype, "logprobs")
    masked = ~np.isfinite(x.cpu().double().numpy())
    assert_grads(g["gx"], ref["gx"], dtype, "d/dx", exact_zero=masked)


def test_logprobs_single_id_and_autograd():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=30, V=1001, dtype=torch.bfloat16)
    x = b.s.clone().requires_grad_()
    idx = torch.arange(30, device="cuda") * 33
    idx[4] = -100
    lp = v.logprobs(x, idx, split=[500, 501])
    assert lp.shape == (30,) and lp[4].item() == 0.0
    lp.sum().backward()
    ref = oracle.logprobs(b.s.cpu(), idx.cpu().numpy()[:, None], -100)
    assert_values(lp.detach(), ref["out"][:, 0], torch.bfloat16, "logprob")
    assert_grads(x.grad, ref["gx"], torch.bfloat16, "d/dx")


def test_logprobs_out_of_range_ids_raise():
    v = vj()
    x = torch.randn(4, 50, device="cuda")
    for bad in (50, -1, 10**12):
        idx = torch.tensor([[0, 1], [2, bad], [3, 4], [5, 6]], device="cuda")
        with pytest.raises(ValueError):
            v.logprobs(x, idx)
    with pytest.raises(ValueError):
        v.logprobs(x, torch.zeros(4, 2, dtype=torch.long, device="cuda"), split=[25, 0, 25])
