"""The Python binding on the host (CPU only): every same-name wrapper and every
autograd op marshals its arguments into the C entry point it names.  The library's
entry points are replaced by a recorder for these tests, so nothing is launched and
no GPU is needed; what is checked is the marshalling (sizes, shard tables, strides,
workspace sizes, argument order), not the arithmetic."""
import ctypes

import pytest
import torch

abi = pytest.importorskip("vocab_sharded_softmax_amd._abi")
import vocab_sharded_softmax_amd as vj  # noqa: E402
from vocab_sharded_softmax_amd import functional  # noqa: E402


class Recorder:
    """Stands in for the library: records entry-point calls; the two pure helpers
    (workspace size, error text) still come from the real library."""

    def __init__(self, real):
        self.calls = []
        self.vjsd_workspace_bytes = real.vjsd_workspace_bytes
        self.vjsd_strerror = real.vjsd_strerror

    def __getattr__(self, name):
        if name.startswith("v"):
            def fn(*args):
                self.calls.append((name, args))
                return 0
            return fn
        raise AttributeError(name)


@pytest.fixture
def rec(monkeypatch):
    r = Recorder(abi.lib)
    monkeypatch.setattr(abi, "lib", r)
    monkeypatch.setattr(abi, "_require_gpu", lambda x, name: None)
    monkeypatch.setattr(abi, "_stream", lambda s: 0)
    return r


def shards_of(arr, S):
    return [arr[k] for k in range(S)]


def test_shardset_views_and_splits():
    x = torch.randn(6, 10, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        abi.ShardSet(x, x)


def test_wrappers_pass_sizes_and_shards(rec):
    B, T, V = 2, 5, 12
    x = torch.randn(B, T + 1, V, dtype=torch.bfloat16)
    s, t = x[:, :-1, :], x[:, 1:, :]  # causal-shift views
    sh = abi.ShardSet(s, t, widths=[5, 0, 7])
    assert (sh.N, sh.S, sh.V, sh.lead_shape) == (B * T, 3, V, (B, T))
    a = shards_of(sh.arr, 3)
    assert [k.vocab_start for k in a] == [0, 5, 5] and [k.width for k in a] == [5, 0, 7]
    assert a[0].s.row_stride == V and a[0].s.rows_per_batch == T and a[0].s.batch_stride == (T + 1) * V
    assert a[2].s.p == s.data_ptr() + 5 * 2 and a[2].t.p == t.data_ptr() + 5 * 2
    N = sh.N
    part = torch.empty(abi.part_floats(N, 3))
    stats = torch.empty(N, 4, dtype=torch.float64)
    kl = torch.empty(N, 2)
    loss = torch.empty(N)
    g = torch.empty(N)
    vj.vjsd_stats(sh, 3, part)
    vj.vjsd_merge(part, 3, N, 3, stats)
    vj.vjsd_fwd(sh, stats, 0.25, part, kl, loss)
    vj.vjsd_forward(sh, 0.25, part, stats, kl, loss)
    shg = abi.ShardSet(s, t, widths=[5, 0, 7], gs=torch.empty(B, T, V, dtype=torch.bfloat16))
    vj.vjsd_bwd(shg, stats, kl, 0.25, g, part)
    vj.vkl_fwd(sh, True, part, stats, kl, loss)
    vj.vkl_bwd(shg, True, stats, kl, g, part)
    vj.ventropy_fwd(sh, part, stats, loss)
    vj.ventropy_bwd(shg, stats, loss, g, part)
    ids = torch.zeros(N, 3, dtype=torch.int64)
    out = torch.empty(N, 3)
    err = torch.zeros(1, dtype=torch.int32)
    sh2 = abi.ShardSet(s, widths=[5, 7])
    vj.vlogprobs_fwd(sh2, V, ids, -100, part, stats, out, err)
    vj.vlogprobs_bwd(abi.ShardSet(s, widths=[5, 7], gs=torch.empty(B, T, V, dtype=torch.bfloat16)),
                     V, stats, ids, -100, torch.empty(N, 3), part)
    mask = torch.ones(N, dtype=torch.uint8)
    opts = abi.loss_opts(N, 2.0, True, mask, "mean")
    assert (opts.temperature, opts.scale_t2, opts.mask, opts.reduction) == (2.0, 1, mask.data_ptr(), 2)
    vj.vjsd_loss_forward(sh, 0.25, opts, part, stats, kl, loss, torch.empty(1))
    vj.vjsd_loss_backward(shg, 0.25, opts, stats, kl, torch.empty(1), part)
    vj.vjsd_forward_backward(shg, 0.25, g, part, stats, kl, loss)
    vj.vjsd_loss_forward_backward(shg, 0.25, opts, torch.empty(1), part, stats, kl, loss,
                                  torch.empty(1))
    with pytest.raises(ValueError):  # per-token losses need N upstream gradients
        vj.vjsd_loss_forward_backward(shg, 0.25, abi.loss_opts(N), torch.empty(1), part, stats,
                                      kl, loss)
    with pytest.raises(ValueError):  # a per-token backward needs N upstream gradients
        vj.vjsd_loss_backward(shg, 0.25, abi.loss_opts(N), stats, kl, torch.empty(1), part)
    with pytest.raises(ValueError):
        abi.loss_opts(N, reduction="avg")
    names = [c[0] for c in rec.calls]
    assert names == ["vjsd_stats", "vjsd_merge", "vjsd_fwd", "vjsd_forward", "vjsd_bwd", "vkl_fwd", "vkl_bwd",
                     "ventropy_fwd", "ventropy_bwd", "vlogprobs_fwd", "vlogprobs_bwd",
                     "vjsd_loss_forward", "vjsd_loss_backward", "vjsd_forward_backward",
                     "vjsd_loss_forward_backward"]
    args = dict(rec.calls)
    assert args["vjsd_stats"][1:5] == (3, N, 2, 3)
    assert args["vjsd_fwd"][5] == 0.25 and args["vjsd_bwd"][6] == 0.25
    fb = args["vjsd_forward_backward"]
    assert fb[1:6] == (3, N, 2, 0.25, g.data_ptr()) and fb[9] == loss.data_ptr()
    assert args["vlogprobs_fwd"][4:8] == (V, ids.data_ptr(), 3, -100)
    for name, a in rec.calls:  # every pointer argument is set
        assert all(v is not None for v in a if not isinstance(v, (int, float))), name
    # a workspace that is too small is refused before the call
    with pytest.raises(ValueError):
        vj.vjsd_fwd(sh, stats, 0.25, torch.empty(10), kl, loss)


def test_autograd_ops_marshal_forward_and_backward(rec):
    s = torch.randn(4, 9, requires_grad=True)
    t = torch.randn(4, 9, requires_grad=True)
    loss = functional.jsd(s, t, 0.5, split=[4, 5])
    loss.sum().backward()
    assert s.grad.shape == s.shape and t.grad.shape == t.shape
    loss = functional.kl_div(s, t.detach(), reverse=True)
    loss.sum().backward()
    dl = functional.jsd_loss(s, t, 0.5, temperature=2.0, scale_t2=True,
                             mask=torch.tensor([True, False, True, True]), reduction="mean")
    assert dl.shape == ()
    dl.backward()
    with pytest.raises(ValueError):
        functional.jsd_loss(s, t, 0.5, mask=torch.ones(3, dtype=torch.bool))
    with pytest.raises(ValueError):
        functional.jsd_loss(s, t, 0.5, temperature=0.0)
    # gradients in the forward: one call, then one scale per wanted gradient
    n0 = len(rec.calls)
    dl = functional.jsd_loss(s, t.detach(), 0.5, reduction="sum", grad_in_forward=True)
    dl.backward()
    assert [c[0] for c in rec.calls[n0:]] == ["vjsd_loss_forward_backward", "vlin_scale"]
    assert rec.calls[n0 + 1][1][1:3] == (s.numel(), 0)  # the student gradient, fp32
    with pytest.raises(ValueError):
        functional.jsd_loss(s, t, 0.5, reduction="none", grad_in_forward=True)
    e = functional.entropy([s[:, :4], s[:, 4:]])
    assert e.shape == (4,)
    lp = functional.logprobs(s, torch.tensor([0, 1, 2, -100]))
    assert lp.shape == (4,)
    lp.sum().backward()
    names = [c[0] for c in rec.calls]
    assert names.count("vjsd_bwd") == 1 and names.count("vkl_bwd") == 1
    assert "vlogprobs_bwd" in names
    bwd = [a for n, a in rec.calls if n == "vjsd_bwd"][0]
    assert bwd[1] == 2  # two shards
