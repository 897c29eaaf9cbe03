"""GPU parity of the vocabulary-parallel cross-entropy (vce_fwd / vce_bwd and the
cross_entropy autograd op) against oracle.cross_entropy (itself pinned to torch's
cross_entropy): labels with ignore_index, none / sum / mean, dtypes, uneven shards,
rows with an ignored label never read (NaN here), the range error, no labelled
token, and sampled rows of the full-size sibling workload."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_grads, assert_values

pytestmark = pytest.mark.gpu

NAN = float("nan")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def labels_for(N, V, seed, ignore_frac=0.15, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    lab = torch.randint(0, V, (N,), generator=g)
    lab[torch.rand(N, generator=g) < ignore_frac] = -100
    return lab.to(device)


def run(x, labels, red, grad, widths=None):
    v = vj()
    sh = v.ShardSet(x, widths=widths)
    N, S, V = sh.N, sh.S, sh.V
    part = v.new_part(N, S, x.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=x.device)
    rows = torch.full((N,), NAN, device=x.device)
    out = torch.full((1,), NAN, device=x.device) if red != "none" else None
    err = torch.zeros(1, dtype=torch.int32, device=x.device)
    v.vce_fwd(sh, V, labels, -100, red, part, stats, rows, out, err)
    gx = torch.full_like(x, NAN)
    v.vce_bwd(v.ShardSet(x, widths=widths, gs=gx), V, stats, labels, -100, red, grad, part)
    torch.cuda.synchronize()
    return rows.cpu(), None if out is None else out.cpu(), gx.cpu(), int(err.item())


def check(x, labels, red, widths=None, seed=0, nan_ignored=True):
    N = x.shape[0]
    ign = (labels == -100)
    if nan_ignored:
        x = x.clone()
        x[ign] = NAN  # never read
    gg = torch.Generator().manual_seed(seed)
    grad = (torch.rand(N, generator=gg) + 0.5) if red == "none" else torch.tensor([0.9])
    rows, out, gx, err = run(x, labels, red, grad.to(x.device), widths)
    assert err == 0
    ref = oracle.cross_entropy(x.cpu(), labels.cpu().numpy(), -100, red,
                               grad=grad.double().numpy() if red == "none" else 0.9, widths=widths)
    assert_values(rows, ref["rows"], x.dtype, "cross-entropy rows")
    if red != "none":
        assert_values(out, np.array([ref["out"]]), x.dtype, red)
    ic = ign.cpu()
    assert (rows[ic] == 0).all() and (gx[ic] == 0).all()
    assert_grads(gx[~ic], ref["gx"][~ic.numpy()], x.dtype, "d/dx")


@pytest.mark.parametrize("red", ["none", "sum", "mean"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_ce_full_rows(red, dtype):
    b = synth.draw("siblings", device="cuda", N=48, dtype=dtype)
    check(b.s, labels_for(48, b.s.shape[1], 1), red)


def test_ce_shards_fp32():
    b = synth.draw("tiny", device="cuda", N=60, V=3001)
    lab = labels_for(60, 3001, 2)
    check(b.s, lab, "mean", widths=[1000, 1, 2000])
    check(b.s, lab, "none", widths=[1500, 1501])
    check(b.s, lab, "sum", widths=[100] * 30 + [1])  # several gather launches


def test_ce_undefined_row_and_no_label():
    b = synth.draw("tiny", device="cuda", N=10, V=500, dtype=torch.bfloat16)
    x = b.s.clone()
    lab = labels_for(10, 500, 3, ignore_frac=0.0)
    x[4] = float("-inf")  # an undefined labelled row: NaN, zero gradient
    rows, out, gx, err = run(x, lab, "mean", torch.tensor([1.0], device="cuda"))
    assert torch.isnan(rows[4]) and torch.isnan(out[0]) and (gx[4] == 0).all()
    none = torch.full((10,), -100, dtype=torch.int64, device="cuda")
    rows, out, gx, err = run(torch.full_like(x, NAN), none, "mean",
                             torch.tensor([1.0], device="cuda"))
    assert out.item() == 0.0 and (rows == 0).all() and (gx == 0).all()


def test_ce_label_out_of_range():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=8, V=300)
    lab = labels_for(8, 300, 4)
    lab[3] = 300
    with pytest.raises(ValueError):
        v.cross_entropy(b.s, lab)
    _, _, _, err = run(b.s, lab, "none", torch.ones(8, device="cuda"))
    assert err == 1


def test_ce_full_size_sampled():
    b = synth.draw("siblings", device="cuda")
    N, V = b.s.shape
    lab = labels_for(N, V, 5, ignore_frac=0.1)
    rows, out, gx, err = run(b.s, lab, "mean", torch.tensor([1.0], device="cuda"))
    assert err == 0
    keep = (lab != -100).cpu()
    np.testing.assert_allclose(out.item(), rows[keep].double().mean().item(), rtol=1e-6)
    samp = np.array([0, 1, 5000, N // 2, N - 1])
    cnt = int(keep.sum())
    ref = oracle.cross_entropy(b.s[samp].cpu(), lab[samp].cpu().numpy(), -100, "none",
                               grad=np.full(samp.size, 1.0 / cnt))
    assert_values(rows[samp], ref["rows"], b.s.dtype, "rows")
    assert_grads(gx[samp], ref["gx"], b.s.dtype, "d/dx")


def test_autograd_cross_entropy():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=12, V=900, dtype=torch.bfloat16)
    lab = labels_for(12, 900, 6)
    x = b.s.clone().view(3, 4, 900).requires_grad_()
    loss = v.cross_entropy(x, lab.view(3, 4), reduction="mean", split=[400, 500])
    (3.0 * loss).backward()
    ref = oracle.cross_entropy(b.s.cpu(), lab.cpu().numpy(), -100, "mean", grad=3.0)
    assert_values(loss.detach().reshape(1).cpu(), np.array([ref["out"]]), torch.bfloat16, "loss")
    assert_grads(x.grad.reshape(12, 900).cpu(), ref["gx"], torch.bfloat16, "d/dx")
    xf = b.s.float().clone().requires_grad_()
    tf = torch.nn.functional.cross_entropy(xf, lab, ignore_index=-100)
    np.testing.assert_allclose(loss.item(), tf.item(), rtol=1e-4)
