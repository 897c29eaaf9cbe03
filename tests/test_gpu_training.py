"""Three SGD updates of a vocabulary-sharded LM head trained through the JSD op,
against the same training run done densely by the fp64 oracle.

[JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel generalized JSD with
Triton kernels", section Validation: the pages check a head-only training run, a few
SGD steps with the head split over 1, 2 and 4 ranks, against the same run unsplit.
Here the ranks are S logical shards on one GPU: shard k owns rows [v_k, v_k+1) of
the student head W, computes its own logit slice h W_k^T, and is paired with the
teacher's logits over the same columns; the per-token JSD merges the shards on the
device, and autograd carries each shard's logit gradient back into its own rows of
W.  The teacher is frozen.

Tolerance, derived from the per-element gradient bound of the fp32 path (1e-4
relative + 1e-7 absolute on dL/dlogits, tests/parity.py): the head gradient G^T h
of one step then differs by at most
    B = (1e-4 + (N + 2) 2^-24) (|G|^T |h|) + 1e-7 sum_n |h_n|
per element (the gradient bound carried through the product, plus its fp32
accumulation), and the head after three steps by lr * sum_steps B, doubled to cover
the earlier steps' differences fed back through the logits.  Per-step losses: the
fp32 value bound (1e-5 relative + 1e-6) plus the same doubling.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

N, D, V = 64, 48, 1000
LR = 2.0
STEPS = 3
SPLITS = {
    1: [1000],
    2: [501, 499],
    4: [260, 240, 0, 500],  # uneven, one rank owning no vocabulary
}


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def problem(seed=4242):
    g = torch.Generator().manual_seed(seed)
    h = torch.randn(N, D, generator=g)
    w0 = torch.randn(V, D, generator=g) * (2.0 / D ** 0.5)
    tl = 0.8 * (h @ w0.T) + 1.5 * torch.randn(N, V, generator=g)
    return h, w0, tl.contiguous()


def dense_oracle(h, w0, tl, beta):
    """Plain fp64 training: dense logits, the oracle's JSD and its logit gradient
    (mean over tokens), the head gradient G^T h, an SGD step; also the per-step
    bound B of the module docstring."""
    h64 = h.double().numpy()
    w = w0.double().numpy().copy()
    t64 = tl.double()
    losses, bounds = [], np.zeros_like(w)
    for _ in range(STEPS):
        logits = torch.from_numpy(h64 @ w.T)
        res = oracle.jsd(logits, t64, beta, gout=np.full(N, 1.0 / N))
        G = res["gs"]
        losses.append(float(res["loss"].mean()))
        bounds += LR * ((1e-4 + (N + 2) * 2.0 ** -24) * (np.abs(G).T @ np.abs(h64))
                        + 1e-7 * np.abs(h64).sum(axis=0)[None, :])
        w -= LR * (G.T @ h64)
    return np.asarray(losses), w, 2.0 * bounds


def sharded_gpu(h, w0, tl, beta, widths):
    v = vj()
    hs = h.cuda()
    heads, teach, c = [], [], 0
    for wk in widths:
        heads.append(w0[c:c + wk].clone().cuda().requires_grad_())
        teach.append(tl[:, c:c + wk].contiguous().cuda())
        c += wk
    losses = []
    for _ in range(STEPS):
        logits = [hs @ w.T for w in heads]
        loss = v.jsd(logits, teach, beta).mean()
        losses.append(loss.item())
        loss.backward()
        with torch.no_grad():
            for w in heads:
                w -= LR * w.grad
                w.grad = None
    torch.cuda.synchronize()
    return np.asarray(losses), torch.cat([w.detach().cpu() for w in heads]).double().numpy()


@pytest.mark.parametrize("beta", [0.3, 0.0, 1.0])
@pytest.mark.parametrize("S", sorted(SPLITS))
def test_three_sgd_updates_of_a_sharded_head(S, beta):
    h, w0, tl = problem()
    ref_losses, ref_w, wbound = dense_oracle(h, w0, tl, beta)
    losses, w = sharded_gpu(h, w0, tl, beta, SPLITS[S])
    lbound = 2.0 * (1e-6 + 1e-5 * np.abs(ref_losses))
    assert np.all(np.abs(losses - ref_losses) <= lbound), (losses, ref_losses)
    err = np.abs(w - ref_w)
    assert np.all(err <= wbound), float((err / wbound).max())
    # the updates are real: the loss falls and the head moved far beyond the bound
    assert ref_losses[-1] < ref_losses[0]
    assert np.abs(ref_w - w0.double().numpy()).max() > 100 * wbound.max()
