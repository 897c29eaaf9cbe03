"""GPU parity of the teacher top-k forward KL (vtopk_kl_fwd / _bwd and the topk_kl
autograd op) against oracle.topk_kl: teacher top-k ids and log-probabilities from
the workloads' teacher logits, padding slots (ignore_index and -inf), dtypes, uneven
and empty shards, more shards than one gather launch covers, full coverage (equal to
the dense forward KL of the library's own KL path), the +inf / NaN rules, the range
error, and sampled rows of the full-size sibling workload."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_values

pytestmark = pytest.mark.gpu


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def teacher_topk(t, K, seed, pad=0.1, ignore=-100):
    """Top-K ids of the teacher and their fp32 log-probabilities; a fraction of the
    slots is padding (ignore_index, or -inf log-probability)."""
    tl = torch.log_softmax(t.float(), dim=-1)
    val, ids = tl.topk(K, dim=-1)
    g = torch.Generator(device=t.device).manual_seed(seed)
    u = torch.rand(ids.shape, generator=g, device=t.device)
    ids = torch.where(u < pad / 2, torch.full_like(ids, ignore), ids)
    val = torch.where((u >= pad / 2) & (u < pad), torch.full_like(val, float("-inf")), val)
    return ids.contiguous(), val.contiguous()


def run(s, ids, tl, widths=None, gout=None):
    v = vj()
    sh = v.ShardSet(s, widths=widths)
    N, S, V = sh.N, sh.S, sh.V
    part = v.new_part(N, S, s.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=s.device)
    kl = torch.full((N,), float("nan"), device=s.device)
    err = torch.zeros(1, dtype=torch.int32, device=s.device)
    v.vtopk_kl_fwd(sh, V, ids, tl, -100, part, stats, kl, err)
    gx = torch.full_like(s, float("nan"))
    if gout is not None:
        v.vtopk_kl_bwd(v.ShardSet(s, widths=widths, gs=gx), V, stats, ids, tl, -100, gout, part)
    torch.cuda.synchronize()
    return kl.cpu(), gx.cpu(), int(err.item())


def check(s, ids, tl, widths=None, seed=0):
    N = s.shape[0]
    g = torch.rand(N, generator=torch.Generator().manual_seed(seed), dtype=torch.float64) + 0.5
    kl, gx, err = run(s, ids, tl, widths, g.float().to(s.device))
    assert err == 0
    ref = oracle.topk_kl(s.cpu(), ids.cpu().numpy(), tl.cpu().double().numpy(), -100,
                         widths=widths, gout=g.numpy())
    assert_values(kl, ref["kl"], s.dtype, "top-k KL")
    und = np.isnan(ref["kl"])
    zero = (ref["gx"] == 0) & (~np.isfinite(s.cpu().double().numpy()) | und[:, None])
    assert_grads(gx, ref["gx"], s.dtype, "d/ds", exact_zero=zero)
    return kl, ref


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_topk_kl_full_rows(dtype):
    b = synth.draw("siblings", device="cuda", N=64, dtype=dtype)
    ids, tl = teacher_topk(b.t, 20, 1)
    check(b.s, ids, tl)


def test_topk_kl_shards_fp32():
    b = synth.draw("tiny", device="cuda", N=40, V=3000)
    ids, tl = teacher_topk(b.t, 12, 2)
    check(b.s, ids, tl, widths=[1000, 1500, 500])
    check(b.s, ids, tl, widths=[1501, 1499])


def test_topk_kl_more_shards_than_one_gather():
    b = synth.draw("tiny", device="cuda", N=24, V=2000, dtype=torch.bfloat16)
    ids, tl = teacher_topk(b.t, 30, 3)
    check(b.s, ids, tl, widths=[100] * 20)  # two gather launches (16 + 4 shards)


def test_topk_kl_full_coverage_is_dense_forward_kl():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=16, V=512)
    tl = torch.log_softmax(b.t.double(), -1).float()
    ids = torch.arange(512, device="cuda").repeat(16, 1)
    kl, _ = check(b.s, ids, tl.contiguous())
    dense = v.kl_div(b.s, b.t).cpu()  # the library's own one-pass KL(p_t || p_s)
    np.testing.assert_allclose(kl.numpy(), dense.numpy(), rtol=2e-5, atol=2e-6)


def test_topk_kl_infinities_undefined_and_range():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=6, V=400, dtype=torch.bfloat16)
    s = b.s.clone()
    ids, tl = teacher_topk(b.t, 5, 4, pad=0.0)
    s[1, ids[1, 2]] = float("-inf")  # teacher mass on a masked student token
    s[3] = float("-inf")  # undefined row
    tl[4, 0] = -1000.0  # underflowing mass still counts
    s[4, ids[4, 0]] = float("-inf")
    kl, _ = check(s, ids, tl)
    assert kl[1] == float("inf") and kl[4] == float("inf") and torch.isnan(kl[3])
    bad = ids.clone()
    bad[2, 1] = 400
    with pytest.raises(ValueError):
        v.topk_kl(s, bad, tl)
    _, _, err = run(s, bad, tl)
    assert err == 1


def test_topk_kl_full_size_sampled():
    b = synth.draw("siblings", device="cuda")
    ids, tl = teacher_topk(b.t, 20, 5)
    N = b.s.shape[0]
    g = torch.full((N,), 0.7, device="cuda")
    kl, gx, err = run(b.s, ids, tl, gout=g)
    assert err == 0 and torch.isfinite(kl).all()
    rows = np.array([0, 1, 777, 8191, 8192, N - 2, N - 1])
    ref = oracle.topk_kl(b.s[rows].cpu(), ids[rows].cpu().numpy(), tl[rows].cpu().double().numpy(),
                         -100, gout=np.full(rows.size, 0.7))
    assert_values(kl[rows], ref["kl"], b.s.dtype, "top-k KL")
    assert_grads(gx[rows], ref["gx"], b.s.dtype, "d/ds")


def test_autograd_topk_kl():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=12, V=700, dtype=torch.bfloat16)
    ids, tl = teacher_topk(b.t, 8, 6)
    s = b.s.clone().view(3, 4, 700).requires_grad_()
    kl = v.topk_kl(s, ids.view(3, 4, 8), tl.view(3, 4, 8))
    assert kl.shape == (3, 4)
    (kl * 1.5).sum().backward()
    ref = oracle.topk_kl(b.s.cpu(), ids.cpu().numpy(), tl.cpu().double().numpy(), -100,
                         gout=np.full(12, 1.5))
    assert_values(kl.detach().reshape(-1).cpu(), ref["kl"], torch.bfloat16, "top-k KL")
    assert_grads(s.grad.reshape(12, 700).cpu(), ref["gx"], torch.bfloat16, "d/ds")
    with pytest.raises(ValueError):
        v.topk_kl(s, ids.view(3, 4, 8), tl.view(3, 4, 8).requires_grad_())
