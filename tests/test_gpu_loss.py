"""GPU parity of the distillation-loss entry points (vjsd_loss_forward / _backward and
the jsd_loss autograd op) against oracle.jsd_loss: temperature, T^2 scaling, token
masks and none / sum / mean reductions, over every forward route (rows held in
registers, two sweeps, several shards, the beta = 0 / 1 one-pass KL) and dtypes.
Also: T = 1 without a mask reproduces vjsd_forward / vjsd_bwd bit for bit, and a
dropped token's logits are never read (they are NaN here)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_values, temperature_grad_scale

pytestmark = pytest.mark.gpu

NAN = float("nan")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def run(s, t, beta, T=1.0, t2=False, mask=None, red="none", grad=None, widths=None,
        want_t=True):
    v = vj()
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    opts = v.loss_opts(N, T, t2, mask, red)
    part = v.new_part(N, S, s.device)
    stats = torch.full((N, 4), NAN, dtype=torch.float64, device=s.device)
    kl = torch.full((N, 2), NAN, device=s.device)
    rows = torch.full((N,), NAN, device=s.device)
    out = torch.full((1,), NAN, device=s.device) if red != "none" else None
    v.vjsd_loss_forward(sh, beta, opts, part, stats, kl, rows, out)
    gs = torch.full_like(s, NAN)
    gt = torch.full_like(t, NAN) if want_t else None
    v.vjsd_loss_backward(v.ShardSet(s, t, widths=widths, gs=gs, gt=gt), beta, opts, stats, kl,
                         grad, part)
    torch.cuda.synchronize()
    return dict(stats=stats.cpu(), kl=kl.cpu(), rows=rows.cpu(), out=None if out is None else out.cpu(),
                gs=gs.cpu(), gt=None if gt is None else gt.cpu())


def upstream(N, red, seed):
    g = torch.Generator().manual_seed(seed)
    if red == "none":
        return torch.rand(N, generator=g, dtype=torch.float64) + 0.5
    return torch.tensor([0.8], dtype=torch.float64)


def check(s, t, beta, T, t2, keep, red, widths=None, seed=0, nan_dropped=False):
    dt = s.dtype
    N = s.shape[0]
    if nan_dropped and keep is not None:  # dropped rows must never be read
        s, t = s.clone(), t.clone()
        s[torch.from_numpy(~keep.astype(bool)).to(s.device)] = NAN
        t[torch.from_numpy(~keep.astype(bool)).to(s.device)] = NAN
    grad = upstream(N, red, seed)
    mask = None if keep is None else torch.from_numpy(keep.astype(np.uint8)).to(s.device)
    g = run(s, t, beta, T, t2, mask, red, grad.to(torch.float32).to(s.device), widths)
    gnp = grad.numpy() if red == "none" else float(grad[0])
    ref = oracle.jsd_loss(s.cpu(), t.cpu(), beta, temperature=T, scale_t2=t2, mask=keep,
                          reduction=red, grad=gnp, widths=widths)
    assert_values(g["rows"], ref["rows"], dt, "per-token loss")
    assert_values(g["kl"][:, 0], ref["kt"], dt, "KL(p_t||M)")
    assert_values(g["kl"][:, 1], ref["ks"], dt, "KL(p_s||M)")
    if red != "none":
        assert_values(g["out"], np.array([ref["out"]]), dt, red)
    k = np.ones(N, bool) if keep is None else keep.astype(bool)
    sn, tn = s.cpu().double().numpy(), t.cpu().double().numpy()
    und = ~np.isfinite(ref["rows"]) & np.isnan(ref["rows"])
    for key, x in (("gs", sn), ("gt", tn)):
        zero = (ref[key] == 0) & (~k[:, None] | (x == -np.inf) | und[:, None])
        assert_grads(g[key], ref[key], dt, key, exact_zero=zero,
                     scale=temperature_grad_scale(dt, T))
    assert (g["gs"][torch.from_numpy(~k)] == 0).all()
    return g, ref


def keep_mask(N, frac, seed):
    rng = np.random.default_rng(seed)
    k = (rng.random(N) < frac).astype(np.uint8)
    k[0] = 1
    return k


# 4000 bf16 columns: row held in registers; 20000: two sweeps
@pytest.mark.parametrize("V", [4000, 20000])
@pytest.mark.parametrize("beta", [0.5, 0.0, 1.0])
@pytest.mark.parametrize("T", [0.5, 2.0])
@pytest.mark.parametrize("red", ["none", "sum", "mean"])
def test_loss_bf16_routes(V, beta, T, red):
    b = synth.draw("full_vocab", device="cuda", N=48, V=V, seed=7)
    keep = keep_mask(48, 0.7, V + int(10 * T))
    check(b.s, b.t, beta, T, red != "sum", keep, red, nan_dropped=True)


@pytest.mark.parametrize("beta", [0.3, 0.0, 1.0])
def test_loss_sharded_fp32(beta):
    b = synth.draw("robust", device="cuda", N=64, V=3000)
    keep = keep_mask(64, 0.6, 3)
    check(b.s, b.t, beta, 1.7, True, keep, "mean", widths=[1300, 0, 1700], nan_dropped=True)


@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_loss_other_dtypes(dtype):
    b = synth.draw("tiny", device="cuda", N=40, V=6000, dtype=dtype)
    check(b.s, b.t, 0.5, 3.0, True, keep_mask(40, 0.5, 5), "mean")
    check(b.s, b.t, 0.5, 0.25, False, None, "none")


def test_loss_masked_undefined_and_offset_rows():
    b = synth.draw("robust", device="cuda", N=120, V=5000)
    keep = keep_mask(120, 0.8, 9)
    check(b.s, b.t, 0.5, 1.5, True, keep, "mean")
    check(b.s, b.t, 0.0, 1.5, True, keep, "sum")


@pytest.mark.parametrize("beta", [0.5, 0.0])
@pytest.mark.parametrize("V", [4000, 20000])
def test_t1_without_mask_matches_per_token_calls_bitwise(beta, V):
    v = vj()
    b = synth.draw("full_vocab", device="cuda", N=32, V=V)
    N = 32
    g = b.gout
    got = run(b.s, b.t, beta, grad=g)
    sh = v.ShardSet(b.s, b.t)
    part = v.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), device="cuda")
    loss = torch.empty((N,), device="cuda")
    v.vjsd_forward(sh, beta, part, stats, kl, loss)
    gs, gt = torch.empty_like(b.s), torch.empty_like(b.t)
    v.vjsd_bwd(v.ShardSet(b.s, b.t, gs=gs, gt=gt), stats, kl, beta, g, part)
    torch.cuda.synchronize()
    assert torch.equal(got["rows"], loss.cpu())
    assert torch.equal(got["stats"], stats.cpu())
    assert torch.equal(got["gs"], gs.cpu()) and torch.equal(got["gt"], gt.cpu())


def test_no_kept_token():
    b = synth.draw("tiny", device="cuda", N=8, V=1000, dtype=torch.bfloat16)
    s, t = b.s.clone(), b.t.clone()
    s[:] = NAN  # never read
    keep = np.zeros(8, np.uint8)
    g = run(s, t, 0.5, 2.0, True, torch.from_numpy(keep).cuda(), "mean",
            torch.tensor([1.0], device="cuda"))
    assert g["out"].item() == 0.0
    assert (g["rows"] == 0).all() and (g["gs"] == 0).all() and (g["gt"] == 0).all()


def test_empty_batch_reduction_writes_zero():
    v = vj()
    s = torch.empty((0, 100), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1,), NAN, device="cuda")
    e = torch.empty(0, device="cuda")
    v.vjsd_loss_forward(v.ShardSet(s, s), 0.5, v.loss_opts(0, 2.0, True, None, "mean"),
                        e, e.double(), e, e, out)
    torch.cuda.synchronize()
    assert out.item() == 0.0


@pytest.mark.parametrize("name", ["tp8_shard", "full_vocab"])
def test_loss_full_size_sparse_mask(name):
    """The teacher-cache caller's shape of work: few response tokens among many."""
    v = vj()
    b = synth.draw(name, device="cuda")
    N = b.s.shape[0]
    keep = keep_mask(N, 0.03, 17)
    kept = np.flatnonzero(keep)
    T = 2.0
    g = run(b.s, b.t, 0.5, T, True, torch.from_numpy(keep).cuda(), "mean",
            torch.tensor([0.8], device="cuda"), want_t=True)
    rows = g["rows"].double().numpy()
    assert (rows[keep == 0] == 0).all()
    np.testing.assert_allclose(g["out"].item(), rows[kept].mean(), rtol=1e-6)
    samp = np.unique(np.concatenate([kept[:4], kept[-2:], np.flatnonzero(keep == 0)[:2]]))
    gup = np.full(samp.size, 0.8 / kept.size)
    ref = oracle.jsd_loss(b.s[samp].cpu(), b.t[samp].cpu(), 0.5, temperature=T, scale_t2=True,
                          mask=keep[samp], reduction="none", grad=gup)
    assert_values(g["rows"][samp], ref["rows"], b.s.dtype, "per-token loss")
    assert_grads(g["gs"][samp], ref["gs"], b.s.dtype, "d/ds")
    assert_grads(g["gt"][samp], ref["gt"], b.s.dtype, "d/dt")
    assert (g["gs"][torch.from_numpy(keep == 0)] == 0).all()


def test_autograd_jsd_loss():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=12, V=3000, dtype=torch.bfloat16)
    s = b.s.clone().view(3, 4, 3000).requires_grad_()
    t = b.t.clone().view(3, 4, 3000).requires_grad_()
    mask = torch.rand(3, 4, generator=torch.Generator().manual_seed(1)) < 0.6
    mask[0, 0] = True
    loss = v.jsd_loss(s, t, 0.4, temperature=1.8, scale_t2=True, mask=mask.cuda(), reduction="mean")
    (2.0 * loss).backward()
    keep = mask.reshape(-1).numpy().astype(np.uint8)
    ref = oracle.jsd_loss(b.s.cpu(), b.t.cpu(), 0.4, temperature=1.8, scale_t2=True, mask=keep,
                          reduction="mean", grad=2.0)
    assert_values(loss.detach().cpu().reshape(1), np.array([ref["out"]]), torch.bfloat16, "loss")
    assert_grads(s.grad.reshape(12, 3000).cpu(), ref["gs"], torch.bfloat16, "d/ds")
    assert_grads(t.grad.reshape(12, 3000).cpu(), ref["gt"], torch.bfloat16, "d/dt")
    per = v.jsd_loss(s.detach(), t.detach(), 0.4, temperature=1.8, mask=mask.cuda(), reduction="none")
    assert per.shape == (3, 4) and (per[~mask.cuda()] == 0).all()
