"""GPU parity of the one-call forward and backward (vjsd_forward_backward and
vjsd_loss_forward_backward).

Every output is bit-identical to the two calls it replaces: vjsd_forward + vjsd_bwd, or
vjsd_loss_forward + vjsd_loss_backward, on the same inputs.  The gradients are also
checked against the fp64 oracle.  Cases covered:
- dtypes;
- the widths of the register-held rows, and of the two-sweep rows with their held-step
  boundaries;
- gradient views at the inputs' offset inside 16 bytes and at another one;
- one gradient or both;
- masks and undefined rows, and the loss options;
- the cases that run the two calls: beta = 0 / 1, several shards, a token mask, and
  register-held rows whose gradient views are not aligned.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_values, sample_rows, ulp

pytestmark = pytest.mark.gpu

NINF = float("-inf")
NAN = float("nan")
INT = {torch.float64: torch.int64, torch.float32: torch.int32, torch.bfloat16: torch.int16,
       torch.float16: torch.int16}


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def same_bits(a, b, what):
    """Bitwise identity (NaN payloads included), on the device."""
    assert a.shape == b.shape and a.dtype == b.dtype, what
    assert torch.equal(a.contiguous().view(INT[a.dtype]), b.contiguous().view(INT[b.dtype])), \
        f"{what}: not bit-identical"


def gview(x, off):
    """A NaN-filled gradient buffer shaped like x: a fresh tensor (off None), or columns
    [off, off + V) of a wider one."""
    if off is None:
        return torch.full_like(x, NAN)
    N, V = x.shape
    buf = torch.full((N, V + 16), NAN, dtype=x.dtype, device=x.device)
    return buf[:, off:off + V]


def run(s, t, beta, gout, want=(True, True), widths=None, goff=None, fused=True, opts=None,
        grad=None):
    """Forward and backward through the ABI, in one call or two; device tensors."""
    v = vj()
    N = s.shape[0]
    gs = gview(s, goff) if want[0] else None
    gt = gview(t, goff) if want[1] else None
    sh = v.ShardSet(s, t, widths=widths, gs=gs, gt=gt)
    part = v.new_part(N, sh.S, s.device)
    stats = torch.full((N, 4), NAN, dtype=torch.float64, device=s.device)
    kl = torch.full((N, 2), NAN, device=s.device)
    loss = torch.full((N,), NAN, device=s.device)
    out = torch.full((1,), NAN, device=s.device)
    if opts is None:
        if fused:
            v.vjsd_forward_backward(sh, beta, gout, part, stats, kl, loss)
        else:
            v.vjsd_forward(sh, beta, part, stats, kl, loss)
            v.vjsd_bwd(sh, stats, kl, beta, gout, part)
    else:
        o = v.loss_opts(N, **opts)
        if fused:
            v.vjsd_loss_forward_backward(sh, beta, o, grad, part, stats, kl, loss, out)
        else:
            v.vjsd_loss_forward(sh, beta, o, part, stats, kl, loss, out)
            v.vjsd_loss_backward(sh, beta, o, stats, kl, grad, part)
    torch.cuda.synchronize()
    return dict(stats=stats, kl=kl, loss=loss, out=out, gs=gs, gt=gt)


def assert_same(a, b):
    for k in ("stats", "kl", "loss", "out", "gs", "gt"):
        if a[k] is None:
            assert b[k] is None
            continue
        same_bits(a[k], b[k], k)


def check_two_calls(s, t, beta, gout=None, **kw):
    if gout is None:
        gen = torch.Generator(device=s.device).manual_seed(5)
        gout = torch.rand(s.shape[0], generator=gen, device=s.device) + 0.5
    one = run(s, t, beta, gout, fused=True, **kw)
    two = run(s, t, beta, gout, fused=False, **kw)
    assert_same(one, two)
    return one, gout


def check_oracle(s, t, beta, gout, res, rows=None, want=(True, True)):
    """Loss and gradients of (sampled) rows against the fp64 oracle."""
    dt = s.dtype
    rows = np.arange(s.shape[0]) if rows is None else rows
    sc, tc = s[rows].cpu(), t[rows].cpu()
    ref = oracle.jsd(sc, tc, beta, gout=gout[rows].cpu().double().numpy())
    assert_values(res["loss"][rows].cpu(), ref["loss"], dt, "loss")
    undefined = np.isnan(ref["loss"])[:, None]
    if want[0]:
        zero = (ref["gs"] == 0.0) & (~np.isfinite(sc.double().numpy()) | undefined)
        assert_grads(res["gs"][rows].cpu(), ref["gs"], dt, "d/ds", exact_zero=zero)
    if want[1]:
        zero = (ref["gt"] == 0.0) & (~np.isfinite(tc.double().numpy()) | undefined)
        assert_grads(res["gt"][rows].cpu(), ref["gt"], dt, "d/dt", exact_zero=zero)


# Register-held rows: 1000 .. 16384 16-bit columns on 256 lanes, 16392 .. 40960 on 512
# (fp32: half as many columns); 40968 / 20488 and wider: two sweeps, holding one
# register step and one LDS step (bf16), one register step (fp16) or four register
# steps and one LDS step (fp32); 135160 / 135176 leave 511 / 513 vectors past the last
# whole step.
@pytest.mark.parametrize("dtype,V", [
    (torch.bfloat16, 1000), (torch.bfloat16, 4096), (torch.bfloat16, 16032),
    (torch.bfloat16, 16392), (torch.bfloat16, 40960), (torch.bfloat16, 40968),
    (torch.bfloat16, 135160), (torch.bfloat16, 135176), (torch.bfloat16, 151936),
    (torch.float16, 8192), (torch.float16, 37984), (torch.float16, 75968),
    (torch.float32, 2000), (torch.float32, 20480), (torch.float32, 20488),
    (torch.float32, 57344), (torch.float32, 128256)])
def test_matches_the_two_calls(dtype, V):
    b = synth.draw("full_vocab", device="cuda", N=24, V=V, dtype=dtype)
    res, gout = check_two_calls(b.s, b.t, 0.3)
    check_oracle(b.s, b.t, 0.3, gout, res, rows=np.array([0, 7, 23]))


@pytest.mark.parametrize("want", [(True, False), (False, True), (False, False)])
@pytest.mark.parametrize("V", [16032, 151936])
def test_one_gradient_or_none(want, V):
    b = synth.draw("full_vocab", device="cuda", N=16, V=V)
    res, gout = check_two_calls(b.s, b.t, 0.5, want=want)
    check_oracle(b.s, b.t, 0.5, gout, res, rows=np.array([0, 15]), want=want)


# Held-step boundaries of the two sweeps (a step: 512 lanes x 4 vectors, 16384 16-bit or
# 8192 fp32 columns; fp32 holds one LDS step from 40960 columns, two from 49152), with
# rows 16-byte aligned, 2 bytes past a boundary (a scalar head), and gradient views at
# the inputs' offset or 1 element off it.
@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 49152), (torch.bfloat16, 49153),
                                     (torch.bfloat16, 49151), (torch.float16, 49160),
                                     (torch.float16, 32768), (torch.float16, 32767),
                                     (torch.float32, 40960), (torch.float32, 40964),
                                     (torch.float32, 40959), (torch.float32, 49152),
                                     (torch.float32, 49156), (torch.float32, 49151)])
@pytest.mark.parametrize("off", [0, 1])
def test_held_steps_and_gradient_offsets(dtype, V, off):
    b = synth.draw("tiny", device="cuda", N=9, V=V + 9, dtype=dtype)
    s, t = b.s[:, off:V + off], b.t[:, off:V + off]
    for goff in (None, off, off + 1):
        res, gout = check_two_calls(s, t, 0.5, goff=goff)
    check_oracle(s, t, 0.5, gout, res, rows=np.array([0, 8]))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_register_rows_with_unaligned_gradient_views(dtype):
    """A register-held row whose gradient views start off a 16-byte boundary runs the
    two calls; the views at the right offset with a row stride that is not a multiple
    of 16 bytes too."""
    b = synth.draw("full_vocab", device="cuda", N=12, V=8192, dtype=dtype)
    for goff in (1, 3):
        res, gout = check_two_calls(b.s, b.t, 0.4, goff=goff)
    check_oracle(b.s, b.t, 0.4, gout, res)


@pytest.mark.parametrize("dtype,V", [(torch.float32, 8000), (torch.bfloat16, 70000)])
def test_masked_tokens_and_undefined_rows(dtype, V):
    b = synth.draw("robust", device="cuda", N=20, V=V)
    s, t = b.s.to(dtype), b.t.to(dtype)
    s[7] = NINF  # student undefined: NaN loss, zero gradients
    t[8] = NINF  # teacher undefined
    s[9, 50:] = NINF  # partly masked
    s[10, :V - 3] = NINF  # mass only in the last three columns
    s[11, 123] = NINF  # student masks a token the teacher keeps
    t[11, 123] = 1.0
    res, gout = check_two_calls(s, t, 0.5)
    assert torch.isnan(res["loss"][[7, 8]]).all()
    for g in (res["gs"], res["gt"]):
        assert (g[[7, 8]] == 0).all()
    check_oracle(s, t, 0.5, gout, res)


@pytest.mark.parametrize("V", [16032, 151936])
@pytest.mark.parametrize("opts", [
    dict(temperature=2.0), dict(temperature=0.7, scale_t2=True),
    dict(mask=True, reduction="sum"), dict(mask=True, reduction="mean", temperature=1.5),
    dict(reduction="mean"), dict(reduction="sum", temperature=3.0, scale_t2=True)])
def test_loss_options(V, opts):
    b = synth.draw("full_vocab", device="cuda", N=32, V=V)
    opts = dict(opts)
    if opts.get("mask"):
        gen = torch.Generator(device="cuda").manual_seed(3)
        opts["mask"] = (torch.rand(32, generator=gen, device="cuda") > 0.3).to(torch.uint8)
    if opts.get("reduction", "none") == "none":
        grad = torch.rand(32, device="cuda") + 0.5
    else:
        grad = torch.tensor([0.75], device="cuda")
    one = run(b.s, b.t, 0.6, None, fused=True, opts=opts, grad=grad)
    two = run(b.s, b.t, 0.6, None, fused=False, opts=opts, grad=grad)
    assert_same(one, two)
    mask = opts.get("mask")
    ref = oracle.jsd_loss(b.s.cpu(), b.t.cpu(), 0.6, temperature=opts.get("temperature", 1.0),
                          scale_t2=opts.get("scale_t2", False),
                          mask=None if mask is None else mask.cpu().numpy(),
                          reduction=opts.get("reduction", "none"),
                          grad=grad.cpu().double().numpy() if grad.numel() > 1
                          else float(grad.item()))
    assert_values(one["loss"].cpu(), ref["rows"], b.s.dtype, "rows")
    scale = max(1.0, 1.0 / opts.get("temperature", 1.0))
    assert_grads(one["gs"].cpu(), ref["gs"], b.s.dtype, "d/ds", scale=scale)
    assert_grads(one["gt"].cpu(), ref["gt"], b.s.dtype, "d/dt", scale=scale)


@pytest.mark.parametrize("beta,widths", [(0.0, None), (1.0, None), (0.5, [1000, 0, 2002]),
                                         (0.2, [300] * 9 + [302])])
def test_cases_that_run_the_two_calls(beta, widths):
    b = synth.draw("tiny", device="cuda", N=12, V=3002, dtype=torch.float32)
    res, gout = check_two_calls(b.s, b.t, beta, widths=widths)
    ref = oracle.jsd(b.s.cpu(), b.t.cpu(), beta, widths=widths,
                     gout=gout.cpu().double().numpy())
    assert_values(res["loss"].cpu(), ref["loss"], torch.float32, "loss")
    assert_grads(res["gs"].cpu(), ref["gs"], torch.float32, "d/ds")
    assert_grads(res["gt"].cpu(), ref["gt"], torch.float32, "d/dt")


@pytest.mark.parametrize("name,beta", [("full_vocab", 0.1), ("full_vocab", 0.5),
                                       ("full_vocab", 0.9), ("tp8_shard", 0.5)])
def test_full_size(name, beta):
    """The route and sizes the benchmark times (8192 x 151936 bf16 at each of its betas,
    two sweeps; 8192 x 16032 bf16, register-held rows), with the workload's own upstream
    gradient: every output bit-identical to the two calls, sampled rows (the first and
    last among them) against the oracle."""
    b = synth.draw(name, device="cuda")
    one = run(b.s, b.t, beta, b.gout, fused=True)
    two = run(b.s, b.t, beta, b.gout, fused=False)
    assert_same(one, two)
    del two
    torch.cuda.empty_cache()
    rows = sample_rows(b.s.shape[0], 6, seed=17, must=(4095, 4096))
    check_oracle(b.s, b.t, beta, b.gout, one, rows=rows)


def test_empty_batch_and_bad_arguments():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=4, V=1000)
    e = torch.empty((0, 1000), dtype=b.s.dtype, device="cuda")
    r = run(e, e.clone(), 0.5, torch.empty(0, device="cuda"))
    assert r["loss"].numel() == 0
    # one shard of width 0: every row undefined (NaN loss), nothing to write, as two calls
    z = torch.empty((4, 0), dtype=b.s.dtype, device="cuda")
    one = run(z, z.clone(), 0.5, torch.ones(4, device="cuda"), fused=True)
    two = run(z, z.clone(), 0.5, torch.ones(4, device="cuda"), fused=False)
    assert torch.isnan(one["loss"]).all()
    assert_same(one, two)
    sh = v.ShardSet(b.s, b.t, gs=torch.empty_like(b.s))
    part = v.new_part(4, 1, "cuda")
    st = torch.empty((4, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((4, 2), device="cuda")
    loss = torch.empty(4, device="cuda")
    g = torch.ones(4, device="cuda")
    with pytest.raises(v.VjsdError):
        v.vjsd_forward_backward(sh, 1.5, g, part, st, kl, loss)
    with pytest.raises(v.VjsdError):
        v.vjsd_forward_backward(sh, float("nan"), g, part, st, kl, loss)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 16032), (torch.bfloat16, 151936),
                                     (torch.float16, 37984), (torch.float32, 20000)])
@pytest.mark.parametrize("reduction,upstream", [("mean", 1.0), ("sum", 0.5), ("mean", 4.0)])
def test_autograd_loss_with_gradients_in_the_forward(dtype, V, reduction, upstream):
    """jsd_loss(grad_in_forward=True): the loss and, for upstream gradients 1 and powers
    of two (which scale exactly), the gradients bit-identical to the default autograd
    path.  fp16 gradients reach the subnormal range (below 2^-14), where a power of two
    rounds again: there the two paths may differ by one rounding of the output."""
    v = vj()
    b = synth.draw("full_vocab", device="cuda", N=24, V=V, dtype=dtype)
    res = []
    for gif in (False, True):
        s = b.s.clone().requires_grad_()
        t = b.t.clone().requires_grad_()
        loss = v.jsd_loss(s, t, 0.4, temperature=1.5, scale_t2=True, reduction=reduction,
                          grad_in_forward=gif)
        (loss * upstream).backward()
        torch.cuda.synchronize()
        res.append((loss.detach(), s.grad, t.grad))
    same_bits(res[0][0], res[1][0], "loss")
    for a, c, what in zip(res[0][1:], res[1][1:], ("d/ds", "d/dt")):
        if dtype == torch.float16 and upstream != 1.0:
            a64, c64 = a.double().cpu().numpy(), c.double().cpu().numpy()
            err = np.abs(a64 - c64)
            assert np.all(err <= ulp(a64, dtype) + 2.0 ** -24), (what, float(err.max()))
        else:
            same_bits(a, c, what)


def test_autograd_loss_with_gradients_in_the_forward_other_scales_and_masks():
    """An upstream gradient that is not a power of two rounds twice (the unit gradient,
    then the product): within the oracle's bound in fp32; a mask (two calls inside)
    and teacher-only gradients go through the same op."""
    v = vj()
    b = synth.draw("robust", device="cuda", N=40, V=3000)
    mask = torch.rand(40, device="cuda") > 0.4
    s = b.s.clone().requires_grad_()
    t = b.t.clone().requires_grad_()
    loss = v.jsd_loss(s, t, 0.7, temperature=2.0, mask=mask, reduction="mean",
                      grad_in_forward=True)
    (loss * 0.3).backward()
    torch.cuda.synchronize()
    ref = oracle.jsd_loss(b.s.cpu(), b.t.cpu(), 0.7, temperature=2.0,
                          mask=mask.cpu().numpy(), reduction="mean", grad=0.3)
    assert_values(loss.detach().cpu().reshape(1), np.array([ref["out"]]), torch.float32, "loss")
    assert_grads(s.grad.cpu(), ref["gs"], torch.float32, "d/ds")
    assert_grads(t.grad.cpu(), ref["gt"], torch.float32, "d/dt")
    t2 = b.t.clone().requires_grad_()
    l2 = v.jsd_loss(b.s, t2, 0.7, reduction="sum", grad_in_forward=True)
    l2.backward()
    r2 = oracle.jsd_loss(b.s.cpu(), b.t.cpu(), 0.7, reduction="sum", grad=1.0)
    assert_grads(t2.grad.cpu(), r2["gt"], torch.float32, "d/dt")
    with pytest.raises(RuntimeError):
        l2.backward()  # the stored gradients were consumed


@pytest.mark.parametrize("V", [16032, 50000])
def test_causal_shift_views(V):
    """[B, T-1, V] slices of [B, T, V] tensors (rows through a batch stride, as the pages'
    callers shift logits against labels), with gradients into [B, T-1, V] slices of
    their own: the one call against the two calls bit for bit and against the oracle."""
    v = vj()
    B, T = 3, 9
    b = synth.draw("full_vocab", device="cuda", N=B * T, V=V)
    s = b.s.reshape(B, T, V)[:, :-1, :]
    t = b.t.reshape(B, T, V)[:, 1:, :]
    N = B * (T - 1)
    gout = torch.rand(N, device="cuda") + 0.5
    res = []
    for fused in (True, False):
        gbuf_s = torch.full((B, T, V), NAN, dtype=s.dtype, device="cuda")
        gbuf_t = torch.full((B, T, V), NAN, dtype=s.dtype, device="cuda")
        gs, gt = gbuf_s[:, :-1, :], gbuf_t[:, 1:, :]
        sh = v.ShardSet(s, t, gs=gs, gt=gt)
        part = v.new_part(N, 1, "cuda")
        st = torch.full((N, 4), NAN, dtype=torch.float64, device="cuda")
        kl = torch.full((N, 2), NAN, device="cuda")
        lo = torch.full((N,), NAN, device="cuda")
        if fused:
            v.vjsd_forward_backward(sh, 0.3, gout, part, st, kl, lo)
        else:
            v.vjsd_forward(sh, 0.3, part, st, kl, lo)
            v.vjsd_bwd(sh, st, kl, 0.3, gout, part)
        torch.cuda.synchronize()
        res.append(dict(stats=st, kl=kl, loss=lo, gs=gs.reshape(N, V), gt=gt.reshape(N, V),
                        out=torch.zeros(1, device="cuda")))
        # the rows outside the views are never written
        assert torch.isnan(gbuf_s[:, -1, :]).all() and torch.isnan(gbuf_t[:, 0, :]).all()
    assert_same(res[0], res[1])
    check_oracle(s.reshape(N, V), t.reshape(N, V), 0.3, gout, res[0], rows=np.array([0, 7, 8, N - 1]))
