"""In-place masking of the per-token outputs.

[OPS-PR] DeepSpeed PR #8791 "Add vocabulary-parallel logprobs, entropy and KL ops":
section How (a fully -inf row, such as padding, returns NaN with zero gradient, so
masking its output is safe) and section Tests (in-place masking of outputs).  A
caller masks the padded rows of each op's output in place and backpropagates; the
gradients must equal those of the same masking done out of place, with padded rows
getting exactly zero, and the op's own saved state must not see the caller's write.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

N, V = 24, 700
PAD = [3, 11, 20]


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def inputs(dtype):
    g = torch.Generator().manual_seed(606)
    s = (2.0 * torch.randn(N, V, generator=g)).to(dtype)
    t = (0.8 * s.float() + 1.5 * torch.randn(N, V, generator=g)).to(dtype)
    s[PAD] = float("-inf")
    t[PAD] = float("-inf")
    pad = torch.zeros(N, dtype=torch.bool)
    pad[PAD] = True
    return s.cuda(), t.cuda(), pad.cuda()


def ops(v, t, ids, tlogp, labels):
    return {
        "jsd": lambda s: v.jsd(s, t, 0.4),
        "kl": lambda s: v.kl_div(s, t),
        "reverse_kl": lambda s: v.kl_div(s, t, reverse=True),
        "entropy": lambda s: v.entropy(s),
        "logprobs": lambda s: v.logprobs(s, ids),
        "topk_kl": lambda s: v.topk_kl(s, ids, tlogp),
        "cross_entropy": lambda s: v.cross_entropy(s, labels, reduction="none"),
        "jsd_loss": lambda s: v.jsd_loss(s, t, 0.4, temperature=2.0, reduction="none"),
    }


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("name", ["jsd", "kl", "reverse_kl", "entropy", "logprobs", "topk_kl",
                                  "cross_entropy", "jsd_loss"])
def test_in_place_masking_of_outputs(name, dtype):
    v = vj()
    s, t, pad = inputs(dtype)
    g = torch.Generator().manual_seed(7)
    ids = torch.randint(0, V, (N, 4), generator=g).cuda()
    tlogp = torch.log_softmax(torch.randn(N, 4, generator=g), -1).cuda()
    labels = torch.randint(0, V, (N,), generator=g).cuda()
    fn = ops(v, t, ids, tlogp, labels)[name]

    x1 = s.clone().requires_grad_()
    out1 = fn(x1)
    rowpad = pad.view(N, *([1] * (out1.dim() - 1))).expand_as(out1)
    assert torch.isnan(out1[rowpad]).all(), "padded rows have no distribution"
    w = torch.rand(out1.shape, generator=g).cuda() + 0.5
    ref = torch.where(rowpad, torch.zeros_like(out1), out1)
    (ref * w).sum().backward()

    x2 = s.clone().requires_grad_()
    out2 = fn(x2)
    out2.masked_fill_(rowpad, 0.0)
    (out2 * w).sum().backward()
    torch.cuda.synchronize()

    assert torch.equal(out2, ref.detach())
    assert torch.equal(x2.grad, x1.grad)
    assert torch.all(x2.grad[pad] == 0)
    assert torch.isfinite(x2.grad).all()
