"""Full-size workloads on the GPU.

Each workload runs over every row through the route the benchmark times: the
one-call forward (``vjsd_forward``: one launch that holds the row in registers,
sweeps it twice, or merges its shards in the workgroup) followed by ``vjsd_bwd``.
The fp64 oracle checks a sample of rows element by element (always including the
first and last rows and the workload's special rows); every row is compared with
the three-launch route (``vjsd_stats``, ``vjsd_merge``, ``vjsd_fwd``), and
properties that hold at any size are checked on all rows.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_stats, assert_values, sample_rows

pytestmark = pytest.mark.gpu

NAN = float("nan")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def jsd_all(s, t, beta, widths=None, gout=None, want_t=True, timed=True):
    """Statistics, KL pair, loss and gradients of every row.  ``timed``: the one-call
    forward then the backward, as the benchmark's step runs them; else the three
    separate forward launches then the backward.  Outputs start as NaN, so a row or
    element left unwritten shows."""
    v = vj()
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    dev = s.device
    part = v.new_part(N, S, dev)
    stats = torch.full((N, 4), NAN, dtype=torch.float64, device=dev)
    kl = torch.full((N, 2), NAN, dtype=torch.float32, device=dev)
    loss = torch.full((N,), NAN, dtype=torch.float32, device=dev)
    if timed:
        v.vjsd_forward(sh, beta, part, stats, kl, loss)
    else:
        v.vjsd_stats(sh, 3, part)
        v.vjsd_merge(part, S, N, 3, stats)
        v.vjsd_fwd(sh, stats, beta, part, kl, loss)
    gs = torch.full_like(s, NAN)
    gt = torch.full_like(t, NAN) if want_t else None
    v.vjsd_bwd(v.ShardSet(s, t, widths=widths, gs=gs, gt=gt), stats, kl, beta, gout, part)
    torch.cuda.synchronize()
    return stats, kl, loss, gs, gt


def same_as_three_launch(out, ref, dtype):
    """Every row of the timed route against the three-launch route on the same data:
    row maxima bit-exact, ln sum exp and the per-token values within rounding, NaN
    and infinity patterns identical, gradients within one unit in the last place of
    the storage format (both routes feed the same backward kernel; their statistics
    differ only in summation order)."""
    st, kl, loss, gs, gt = out
    st3, kl3, loss3, gs3, gt3 = ref
    m, m3 = st[:, 0::2], st3[:, 0::2]
    assert torch.equal(torch.isnan(m), torch.isnan(m3))
    assert torch.equal(m.nan_to_num(), m3.nan_to_num()), "row maxima differ"
    lz, lz3 = st[:, 1::2], st3[:, 1::2]
    fin = torch.isfinite(lz3)
    assert torch.equal(torch.isfinite(lz), fin)
    assert (lz[fin] - lz3[fin]).abs().max().item() <= 4e-6
    # each route sums a row's V terms in fp32 in its own order: the two sums differ by
    # rounding of order sqrt(V) * 2^-24 relative; four times that, plus the fp32
    # value tolerance's absolute part
    V = gs.shape[-1]
    rtol = 4.0 * math.sqrt(V) * 2.0 ** -24
    for a, b in ((loss, loss3), (kl, kl3)):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(np.isnan(a), np.isnan(b))
        assert np.array_equal(np.isinf(a), np.isinf(b))
        f = np.isfinite(b)
        np.testing.assert_allclose(a[f], b[f], rtol=rtol, atol=1e-6)
    eps = 2.0 ** -7 if dtype == torch.bfloat16 else (2.0 ** -10 if dtype == torch.float16 else 1e-4)
    for a, b in ((gs, gs3), (gt, gt3)):
        if a is None:
            continue
        for r0 in range(0, a.shape[0], 1024):  # row blocks: bounded fp32 temporaries
            x, y = a[r0:r0 + 1024].float(), b[r0:r0 + 1024].float()
            assert not torch.isnan(x).any() and not torch.isnan(y).any()
            bound = eps * torch.maximum(x.abs(), y.abs()) + 1e-6
            assert ((x - y).abs() <= bound).all(), f"gradients differ in rows from {r0}"


def check_rows(rows, s, t, beta, widths, gout, stats, kl, loss, gs, gt):
    dt = s.dtype
    sc, tc = s[rows].cpu(), t[rows].cpu()
    g = gout[rows].cpu().double().numpy()
    ref = oracle.jsd(sc, tc, beta, widths=widths, gout=g)
    st = stats[rows].cpu()
    assert_stats(st, *oracle.stats(sc, widths=widths), 0, "student stats")
    assert_stats(st, *oracle.stats(tc, widths=widths), 1, "teacher stats")
    assert_values(loss[rows].cpu(), ref["loss"], dt, "loss")
    assert_values(kl[rows].cpu()[:, 0], ref["kt"], dt, "KL(p_t||M)")
    assert_values(kl[rows].cpu()[:, 1], ref["ks"], dt, "KL(p_s||M)")
    masked_s = ~np.isfinite(sc.double().numpy())
    masked_t = ~np.isfinite(tc.double().numpy())
    undefined = np.isnan(ref["loss"])[:, None]
    assert_grads(gs[rows].cpu(), ref["gs"], dt, "d/ds",
                 exact_zero=(ref["gs"] == 0) & (masked_s | undefined))
    if gt is not None:
        assert_grads(gt[rows].cpu(), ref["gt"], dt, "d/dt",
                     exact_zero=(ref["gt"] == 0) & (masked_t | undefined))


def H(beta):
    return -beta * math.log(beta) - (1 - beta) * math.log1p(-beta)


@pytest.mark.parametrize("detached", [False, True])
def test_tp8_shard_full(detached):
    """One tensor-parallel rank's width (8192 x 16032 bf16, beta 0.5): the one-call
    forward holds each row in registers."""
    b = synth.draw("tp8_shard", device="cuda")
    out = jsd_all(b.s, b.t, 0.5, None, b.gout, want_t=not detached)
    rows = sample_rows(b.s.shape[0], 24, 11)
    check_rows(rows, b.s, b.t, 0.5, None, b.gout, *out)
    loss = out[2]
    assert torch.isfinite(loss).all() and (loss >= -1e-5).all() and (loss <= H(0.5) + 1e-5).all()
    same_as_three_launch(out, jsd_all(b.s, b.t, 0.5, None, b.gout, want_t=not detached,
                                      timed=False), b.s.dtype)


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
def test_full_vocab_timed_step(beta):
    """The benchmark's step at its full size (8192 x 151936 bf16, both gradients) at
    each of its three betas: the two-sweep forward with held steps, then the
    backward."""
    b = synth.draw("full_vocab", device="cuda")
    assert beta in synth.WORKLOADS["full_vocab"].betas
    out = jsd_all(b.s, b.t, beta, None, b.gout)
    rows = sample_rows(b.s.shape[0], 10, 20 + int(beta * 10))
    check_rows(rows, b.s, b.t, beta, None, b.gout, *out)
    loss = out[2]
    assert torch.isfinite(loss).all()
    assert (loss >= -1e-5).all() and (loss <= H(beta) + 1e-5).all()
    same_as_three_launch(out, jsd_all(b.s, b.t, beta, None, b.gout, timed=False), b.s.dtype)


def test_robust_full_size_sharded_and_split_independent():
    w = synth.WORKLOADS["robust"]
    b = synth.draw("robust", device="cuda")
    out4 = jsd_all(b.s, b.t, 0.5, list(w.widths), b.gout)
    must = list(b.rows_masked[:3].cpu().numpy()) + list(b.rows_offset[:5].cpu().numpy())
    rows = sample_rows(b.s.shape[0], 12, 30, must)
    check_rows(rows, b.s, b.t, 0.5, list(w.widths), b.gout, *out4)
    loss4 = out4[2].cpu().numpy()
    masked = b.rows_masked.cpu().numpy()
    assert np.isnan(loss4[masked]).all()
    assert np.isfinite(np.delete(loss4, masked)).all()
    assert torch.all(out4[3][b.rows_masked] == 0) and torch.all(out4[4][b.rows_masked] == 0)
    same_as_three_launch(out4, jsd_all(b.s, b.t, 0.5, list(w.widths), b.gout, timed=False),
                         b.s.dtype)
    del out4
    loss1 = jsd_all(b.s, b.t, 0.5, None, b.gout)[2].cpu().numpy()
    fin = np.isfinite(loss4)
    np.testing.assert_allclose(loss1[fin], loss4[fin], rtol=5e-6, atol=5e-7)
    assert np.array_equal(np.isnan(loss1), np.isnan(loss4))


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
def test_siblings_full_size(dtype):
    v = vj()
    b = synth.draw("siblings", device="cuda", dtype=dtype)
    N = b.s.shape[0]
    rows = sample_rows(N, 8, 40)
    sc, tc = b.s[rows].cpu(), b.t[rows].cpu()
    g = b.gout[rows].cpu().double().numpy()
    for reverse in (False, True):
        sh = v.ShardSet(b.s, b.t)
        part = v.new_part(N, 1, "cuda")
        stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
        kl = torch.empty((N, 2), dtype=torch.float32, device="cuda")
        loss = torch.empty(N, device="cuda")
        v.vkl_fwd(sh, reverse, part, stats, kl, loss)
        gs = torch.empty_like(b.s)
        v.vkl_bwd(v.ShardSet(b.s, b.t, gs=gs), reverse, stats, kl, b.gout, part)
        torch.cuda.synchronize()
        ref = oracle.kl_div(sc, tc, reverse=reverse, gout=g)
        assert_values(loss[rows].cpu(), ref["loss"], dtype, "KL")
        assert_grads(gs[rows].cpu(), ref["gs"], dtype, "d/ds")
        assert torch.isfinite(loss).all() and (loss >= -1e-4).all()
        del gs
    # entropy of the student
    part = v.new_part(N, 1, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    ent = torch.empty(N, device="cuda")
    sh = v.ShardSet(b.s)
    v.ventropy_fwd(sh, part, stats, ent)
    gx = torch.empty_like(b.s)
    v.ventropy_bwd(v.ShardSet(b.s, gs=gx), stats, ent, b.gout, part)
    torch.cuda.synchronize()
    ref = oracle.entropy(sc, gout=g)
    assert_values(ent[rows].cpu(), ref["ent"], dtype, "entropy")
    assert_grads(gx[rows].cpu(), ref["gx"], dtype, "d/dx entropy")
    V = b.s.shape[1]
    assert (ent >= 0).all() and (ent <= math.log(V) + 1e-4).all()
    # top-k log-probabilities with ignore_index
    K = b.ids.shape[1]
    out = torch.empty((N, K), device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    v.vlogprobs_fwd(sh, V, b.ids, -100, part, stats, out, err)
    v.vlogprobs_bwd(v.ShardSet(b.s, gs=gx), V, stats, b.ids, -100, b.gids, part)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ids_r = b.ids[rows].cpu().numpy()
    ref = oracle.logprobs(sc, ids_r, -100, gout=b.gids[rows].cpu().double().numpy())
    assert_values(out[rows].cpu(), ref["out"], dtype, "logprobs")
    assert_grads(gx[rows].cpu(), ref["gx"], dtype, "d/dx logprobs")
    ign = b.ids == -100
    assert torch.all(out[ign] == 0) and (out[~ign] <= 0).all()
    assert abs(ign.float().mean().item() - 0.10) < 1e-3
