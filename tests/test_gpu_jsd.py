"""GPU parity of the JSD path (statistics, merge, divergence, backward) against the
fp64 oracle, element by element, through the C ABI.

Sizes span several row tiles (256 lanes x 4 vectors of 16 bytes) and a ragged
tail; shard splits include uneven and empty shards; views include unaligned and
causal-shift slices.  Tolerances are those of tests/parity.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_grads, assert_special_pattern, assert_stats, assert_values,
                    grad_ulp_report)

pytestmark = pytest.mark.gpu

NINF = float("-inf")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def run_jsd(s, t, beta, widths=None, gout=None, want_s=True, want_t=True):
    """stats -> merge -> fwd -> bwd through the ABI; returns dict of host tensors."""
    v = vj()
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    dev = s.device
    part = v.new_part(N, S, dev)
    stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
    kl = torch.empty((N, 2), dtype=torch.float32, device=dev)
    loss = torch.empty((N,), dtype=torch.float32, device=dev)
    v.vjsd_stats(sh, 3, part)
    v.vjsd_merge(part, S, N, 3, stats)
    v.vjsd_fwd(sh, stats, beta, part, kl, loss)
    gs = torch.full_like(s, float("nan")) if want_s else None
    gt = torch.full_like(t, float("nan")) if want_t else None
    if gout is None:
        gout = torch.ones(N, device=dev)
    shg = v.ShardSet(s, t, widths=widths, gs=gs, gt=gt)
    v.vjsd_bwd(shg, stats, kl, beta, gout, part)
    torch.cuda.synchronize()
    return dict(stats=stats.cpu(), kl=kl.cpu(), loss=loss.cpu(),
                gs=None if gs is None else gs.cpu(), gt=None if gt is None else gt.cpu())


def rows2d(x):
    return x.reshape(-1, x.shape[-1])


def check_against_oracle(s, t, beta, widths=None, gout=None, want_s=True, want_t=True,
                         inf_rows_target_side=True):
    dt = s.dtype
    g = run_jsd(s, t, beta, widths, gout, want_s, want_t)
    sc, tc = rows2d(s).cpu().contiguous(), rows2d(t).cpu().contiguous()
    go = None if gout is None else gout.cpu().double().numpy()
    ref = oracle.jsd(sc, tc, beta, widths=widths, gout=go)
    ms, lzs = oracle.stats(sc, widths=widths)
    mt, lzt = oracle.stats(tc, widths=widths)
    assert_stats(g["stats"], ms, lzs, 0, "student stats")
    assert_stats(g["stats"], mt, lzt, 1, "teacher stats")
    assert_values(g["loss"], ref["loss"], dt, "loss")
    assert_values(g["kl"][:, 0], ref["kt"], dt, "KL(p_t||M)")
    assert_values(g["kl"][:, 1], ref["ks"], dt, "KL(p_s||M)")
    infinite = np.isinf(ref["loss"])
    if want_s:
        gs = rows2d(g["gs"])
        side_ok = ~infinite if beta == 1.0 else np.ones_like(infinite)
        assert_grads(gs[side_ok], ref["gs"][side_ok], dt, "d/ds",
                     exact_zero=(ref["gs"][side_ok] == 0.0) & (~np.isfinite(sc.double().numpy()[side_ok]) |
                                                               np.isnan(ref["loss"][side_ok])[:, None]))
    if want_t:
        gt = rows2d(g["gt"])
        side_ok = ~infinite if beta == 0.0 else np.ones_like(infinite)
        assert_grads(gt[side_ok], ref["gt"][side_ok], dt, "d/dt",
                     exact_zero=(ref["gt"][side_ok] == 0.0) & (~np.isfinite(tc.double().numpy()[side_ok]) |
                                                               np.isnan(ref["loss"][side_ok])[:, None]))
    return g, ref


# ---- the tiny workload at full size ----------------------------------------------------

@pytest.mark.parametrize("beta", [0.5, 0.0, 0.1, 0.9, 1.0])
def test_tiny_fp32_all_betas(beta):
    b = synth.draw("tiny", device="cuda")
    check_against_oracle(b.s, b.t, beta, gout=b.gout)


# ---- reduced versions of the large workloads ------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("detached", [False, True])
def test_tp8_shard_recipe(dtype, detached):
    b = synth.draw("tp8_shard", device="cuda", N=48, dtype=dtype)
    g, _ = check_against_oracle(b.s, b.t, 0.5, gout=b.gout, want_t=not detached)
    if dtype != torch.float32:
        # beyond the tolerance: nearly every gradient is within one unit in the last place
        ref = oracle.jsd(b.s.cpu(), b.t.cpu(), 0.5, gout=b.gout.cpu().double().numpy())
        assert grad_ulp_report(g["gs"], ref["gs"], dtype, quantile=0.999) <= 1.0


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
def test_full_vocab_recipe_full_rows(beta):
    b = synth.draw("full_vocab", device="cuda", N=12)
    check_against_oracle(b.s, b.t, beta, gout=b.gout)


def test_robust_recipe_sharded_masked_offset_rows():
    w = synth.WORKLOADS["robust"]
    b = synth.draw("robust", device="cuda", N=100)
    assert b.rows_masked.numel() == 1 and b.rows_offset.numel() == 10
    g, ref = check_against_oracle(b.s, b.t, 0.5, widths=list(w.widths), gout=b.gout)
    assert np.isnan(ref["loss"][b.rows_masked.cpu().numpy()]).all()
    # the same data as one shard gives the same answer (split independence)
    g1 = run_jsd(b.s, b.t, 0.5, None, b.gout)
    fin = np.isfinite(g["loss"].numpy())
    np.testing.assert_allclose(g1["loss"].numpy()[fin], g["loss"].numpy()[fin], rtol=2e-6,
                               atol=2e-7)
    np.testing.assert_allclose(g1["gs"].numpy(), g["gs"].numpy(), rtol=1e-5, atol=1e-9)


@pytest.mark.parametrize("widths", [[51, 50], [1, 0, 100], [0, 101], [101, 0], [20] * 5 + [1]])
@pytest.mark.parametrize("beta", [0.0, 0.3, 1.0])
def test_uneven_and_empty_shards(widths, beta):
    b = synth.draw("tiny", device="cuda", N=37, V=101)
    check_against_oracle(b.s, b.t, beta, widths=widths, gout=b.gout)


def test_shards_given_as_separate_tensors():
    b = synth.draw("tiny", device="cuda", N=20, V=300, dtype=torch.bfloat16)
    ws = [120, 0, 180]
    s_parts = [b.s[:, :120].contiguous(), b.s[:, 120:120].contiguous(), b.s[:, 120:].contiguous()]
    t_parts = [b.t[:, :120].contiguous(), b.t[:, 120:120].contiguous(), b.t[:, 120:].contiguous()]
    v = vj()
    whole = v.jsd(b.s, b.t, 0.4, split=ws)
    parts = v.jsd(s_parts, t_parts, 0.4)
    # another memory layout changes the lane order of the reductions, nothing else
    torch.testing.assert_close(parts, whole, rtol=2e-6, atol=2e-7)


# ---- views -------------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_unaligned_and_mismatched_views(dtype):
    base = synth.draw("tiny", device="cuda", N=16, V=2003, dtype=dtype)
    s = base.s[:, 1:]  # starts 1 element past a 16-byte boundary: scalar head
    t = base.t[:, 1:]
    check_against_oracle(s, t, 0.5, gout=base.gout)
    # the same teacher values at another offset inside 16 bytes and another row stride
    pad = torch.zeros((16, 2), dtype=dtype, device="cuda")
    t2 = torch.cat([pad, base.t], dim=1)[:, 3:]
    assert torch.equal(t2, t) and t2.stride(0) != t.stride(0)
    check_against_oracle(s, t2, 0.25, gout=base.gout)


def test_causal_shift_views():
    """[B, T-1, V] slices of [B, T, V], taken without a copy."""
    B, T, V = 3, 9, 777
    b = synth.draw("tiny", device="cuda", N=B * T, V=V, dtype=torch.bfloat16)
    s3 = b.s.view(B, T, V)
    t3 = b.t.view(B, T, V)
    s = s3[:, :-1, :]
    t = t3[:, 1:, :]
    gout = b.gout[: B * (T - 1)]
    g = run_jsd(s, t, 0.7, None, gout)
    ref = oracle.jsd(s.reshape(-1, V).cpu(), t.reshape(-1, V).cpu(), 0.7,
                     gout=gout.cpu().double().numpy())
    assert_values(g["loss"], ref["loss"], torch.bfloat16, "loss")
    assert_grads(g["gs"].reshape(-1, V), ref["gs"], torch.bfloat16, "d/ds")
    assert_grads(g["gt"].reshape(-1, V), ref["gt"], torch.bfloat16, "d/dt")
    v = vj()
    out = v.jsd(s, t, 0.7)
    assert out.shape == (B, T - 1)


# ---- degenerate cases the method has --------------------------------------------------------

def test_empty_batch_and_single_token():
    v = vj()
    for N, V in ((0, 10), (1, 1), (1, 2), (3, 1)):
        s = torch.randn(N, V, device="cuda").requires_grad_()
        t = torch.randn(N, V, device="cuda").requires_grad_()
        out = v.jsd(s, t, 0.5)
        assert out.shape == (N,)
        out.sum().backward()
        assert s.grad.shape == s.shape
        if V == 1 and N:  # one token carries all the mass: 0 up to fp32 rounding
            assert torch.all(out.abs() <= 1e-6) and torch.all(s.grad.abs() <= 1e-6)


@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
def test_identical_inputs_give_zero_and_disjoint_give_H_beta(beta):
    b = synth.draw("tiny", device="cuda", N=32, V=4000, dtype=torch.bfloat16)
    g = run_jsd(b.s, b.s.clone(), beta)
    assert np.all(np.abs(g["loss"].numpy()) <= 2e-6)
    s = b.s.clone()
    t = b.t.clone()
    s[:, 2000:] = NINF
    t[:, :2000] = NINF
    g, _ = check_against_oracle(s, t, beta)
    Hb = -beta * math.log(beta) - (1 - beta) * math.log1p(-beta)
    np.testing.assert_allclose(g["loss"].numpy(), Hb, rtol=2e-5)
    assert torch.all(g["gs"].float().abs() <= 1e-6) and torch.all(g["gt"].float().abs() <= 1e-6)


def test_undefined_rows_give_nan_and_exact_zero_gradient_whatever_g():
    b = synth.draw("tiny", device="cuda", N=8, V=600, dtype=torch.bfloat16)
    s, t = b.s.clone(), b.t.clone()
    s[1] = NINF
    t[2] = NINF
    s[3] = NINF
    t[3] = NINF
    gout = b.gout.clone()
    gout[1] = float("nan")  # even a NaN upstream gradient leaves these rows at 0
    gout[2] = float("inf")
    for beta in (0.0, 0.5, 1.0):
        g = run_jsd(s, t, beta, None, gout)
        assert np.isnan(g["loss"].numpy()[[1, 2, 3]]).all()
        assert np.isfinite(g["loss"].numpy()[[0, 4, 5, 6, 7]]).all()
        for k in ("gs", "gt"):
            assert torch.all(g[k][1:4] == 0)
            assert (g[k][1:4].view(torch.int16) == 0).all()  # +0, not -0 or NaN


def test_kl_endpoints_infinite_on_masked_target_mass():
    b = synth.draw("tiny", device="cuda", N=6, V=300)
    s, t = b.s.clone(), b.t.clone()
    s[0, 17] = NINF  # teacher mass meets a masked student token
    t[1, 17] = -3.0e4  # underflowed mass, still finite logit
    s[1, 17] = NINF
    t[2, 5] = NINF  # both masked: finite
    s[2, 5] = NINF
    g, ref = check_against_oracle(s, t, 0.0)
    assert np.isinf(g["loss"].numpy()[[0, 1]]).all() and np.isfinite(g["loss"].numpy()[2:]).all()
    g, ref = check_against_oracle(t, s, 1.0)
    assert np.isinf(g["loss"].numpy()[[0, 1]]).all()
    assert np.all(np.isfinite(run_jsd(s, t, 0.5)["loss"].numpy()))


def test_large_offset_rows():
    b = synth.draw("tiny", device="cuda", N=16, V=5000)
    s = b.s.clone()
    t = b.t.clone()
    s[::2] += 1e4
    t[::2] += 1e4
    g, _ = check_against_oracle(s, t, 0.5, gout=b.gout)
    # the oracle of an offset row is the unshifted row [OPS-PR, Tests]
    ref0 = oracle.jsd((s[::2] - 1e4).cpu(), (t[::2] - 1e4).cpu(), 0.5)
    assert_values(g["loss"][::2], ref0["loss"], torch.float32, "offset rows vs unshifted")



@pytest.mark.parametrize("beta", [0.0, 0.4, 1.0])
@pytest.mark.parametrize("widths", [None, [1700, 0, 3300]])
def test_independent_large_shifts(beta, widths):
    """[JSD-PR, Validation]: independent large logit shifts.  Every row of each input
    gets its own offset (+-1e4, 3e3, -5e3 or none), so student and teacher rows sit
    far apart; each softmax is shift-invariant, so the oracle is the unshifted rows
    (recovered exactly: fl32(x + a) - a is exact by Sterbenz for |x| << |a|), for the
    loss and both gradients, on the pass-by-pass route, and for the loss on the
    one-call forward of the autograd op."""
    v = vj()
    b = synth.draw("tiny", device="cuda", N=16, V=5000)
    gen = torch.Generator().manual_seed(31)
    offs = torch.tensor([1e4, -1e4, 3e3, -5e3, 0.0])
    a = offs[torch.randint(0, 5, (16,), generator=gen)].cuda()[:, None]
    c = offs[torch.randint(0, 5, (16,), generator=gen)].cuda()[:, None]
    assert not torch.equal(a, c)
    s, t = b.s + a, b.t + c
    s0, t0 = s - a, t - c
    assert torch.equal(s0 + a, s) and torch.equal(t0 + c, t)
    g = run_jsd(s, t, beta, widths, b.gout)
    ref = oracle.jsd(s0.cpu(), t0.cpu(), beta, widths=widths, gout=b.gout.cpu().double().numpy())
    assert_values(g["loss"], ref["loss"], torch.float32, "shifted rows vs unshifted")
    assert_grads(g["gs"], ref["gs"], torch.float32, "d/ds of shifted rows")
    assert_grads(g["gt"], ref["gt"], torch.float32, "d/dt of shifted rows")
    loss = v.jsd(s, t, beta, split=widths)
    assert_values(loss, ref["loss"], torch.float32, "one-call forward of shifted rows")

def test_reruns_are_bitwise_identical():
    b = synth.draw("full_vocab", device="cuda", N=64, V=30011)
    g1 = run_jsd(b.s, b.t, 0.5, None, b.gout)
    g2 = run_jsd(b.s, b.t, 0.5, None, b.gout)
    for k in ("loss", "kl", "stats", "gs", "gt"):
        assert torch.equal(g1[k], g2[k]), k


def test_autograd_matches_the_abi_and_refuses_double_backward():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=10, V=700, dtype=torch.bfloat16)
    s = b.s.clone().requires_grad_()
    t = b.t.clone().requires_grad_()
    loss = v.jsd(s, t, 0.3)
    (loss * b.gout).sum().backward()
    g = run_jsd(b.s, b.t, 0.3, None, b.gout)
    assert torch.equal(loss.detach().cpu(), g["loss"])
    assert torch.equal(s.grad.cpu(), g["gs"]) and torch.equal(t.grad.cpu(), g["gt"])
    # a detached teacher gets no gradient and the student's is unchanged
    s2 = b.s.clone().requires_grad_()
    (v.jsd(s2, b.t, 0.3) * b.gout).sum().backward()
    assert torch.equal(s2.grad.cpu(), g["gs"])
    s3 = b.s.clone().requires_grad_()
    out = v.jsd(s3, b.t, 0.3).sum()
    (gr,) = torch.autograd.grad(out, s3, create_graph=True)
    with pytest.raises(RuntimeError):
        gr.sum().backward()


def test_bad_arguments_raise_before_any_launch():
    v = vj()
    s = torch.randn(4, 10, device="cuda")
    with pytest.raises(ValueError):
        v.jsd(s, s, 1.5)
    with pytest.raises(ValueError):
        v.jsd(s, s.half(), 0.5)
    with pytest.raises(ValueError):
        v.jsd(s, torch.randn(4, 11, device="cuda"), 0.5)


# The backward of 2 to 8 shards runs as one launch whose chunks walk each row's shards
# in order, more shards one launch each; empty and one-column shards, each gradient alone
@pytest.mark.parametrize("widths", [[2500] * 8, [2000] * 8 + [4000], [1, 0, 19999],
                                    [7, 3, 5000, 0, 14990]])
@pytest.mark.parametrize("want", [(True, True), (True, False), (False, True)])
@pytest.mark.parametrize("beta", [0.4, 0.0, 1.0])
def test_sharded_backward(widths, want, beta):
    b = synth.draw("robust", device="cuda", N=23, V=sum(widths))
    s, t = b.s.clone(), b.t.clone()
    s[4] = NINF  # undefined row: exact-zero gradients in every shard
    t[6, 3000:3500] = NINF
    check_against_oracle(s, t, beta, widths=widths, gout=b.gout, want_s=want[0],
                         want_t=want[1])


# ---- the backward's work-item numbering: each XCD takes runs of 256 consecutive row
# chunks and the grid is padded to whole rounds of 8 x 256 items, so item counts just
# below, at and above a round must still write every gradient element (the gradient
# buffers start as NaN, so an element left unwritten fails) ----------------------------

@pytest.mark.parametrize("N,V,detached", [
    (23, 44800, False),   # 23 rows x 89 chunks of 512 columns = 2047 items
    (32, 32000, False),   # 32 x 64 = 2048
    (683, 800, False),    # 683 x 3 = 2049
    (17, 122500, False),  # 17 x 241 = 4097
    (683, 1500, True),    # student gradient alone: 683 x 3 chunks of 1024 = 2049
])
def test_backward_item_rounds(N, V, detached):
    b = synth.draw("tp8_shard", device="cuda", N=N, V=V, dtype=torch.bfloat16)
    check_against_oracle(b.s, b.t, 0.5, gout=b.gout, want_t=not detached)
