"""The no-allocation JSD backward (vjsd_bwd_noalloc) against vjsd_bwd.

Both run the same kernels on the same forward outputs, so the gradients must agree
bit for bit.  Two calls in a row, the second with fewer rows, check that the shared
device scratch is rewritten before it is read; a mixed shard layout and a
teacher-detached call cover the other backward launches.  Sizes beyond the scratch
are refused before anything is enqueued.
"""
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

NAN = float("nan")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def forward(v, s, t, beta, widths=None):
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    part = v.new_part(N, S, s.device)
    stats = torch.empty((N, 4), dtype=torch.float64, device=s.device)
    kl = torch.empty((N, 2), dtype=torch.float32, device=s.device)
    loss = torch.empty((N,), dtype=torch.float32, device=s.device)
    v.vjsd_forward(sh, beta, part, stats, kl, loss)
    return stats, kl, part


def both_backwards(s, t, gout, beta, widths=None, want_t=True):
    v = vj()
    stats, kl, part = forward(v, s, t, beta, widths)
    ref_s, ref_t = torch.full_like(s, NAN), torch.full_like(t, NAN) if want_t else None
    v.vjsd_bwd(v.ShardSet(s, t, widths=widths, gs=ref_s, gt=ref_t), stats, kl, beta, gout, part)
    gs, gt = torch.full_like(s, NAN), torch.full_like(t, NAN) if want_t else None
    v.vjsd_bwd_noalloc(v.ShardSet(s, t, widths=widths, gs=gs, gt=gt), stats, kl, beta, gout)
    torch.cuda.synchronize()
    assert torch.equal(gs.view(torch.int16), ref_s.view(torch.int16))
    if want_t:
        assert torch.equal(gt.view(torch.int16), ref_t.view(torch.int16))


def test_two_calls_in_a_row_second_smaller():
    b = synth.draw("full_vocab", device="cuda", N=3000, V=20000)
    both_backwards(b.s, b.t, b.gout, 0.3)
    small = synth.draw("tiny", device="cuda", N=37, V=1000, dtype=torch.bfloat16)
    both_backwards(small.s, small.t, small.gout, 0.7)


def test_shards_endpoints_and_detached_teacher():
    b = synth.draw("tiny", device="cuda", N=257, V=3001, dtype=torch.bfloat16)
    for beta in (0.0, 0.5, 1.0):
        both_backwards(b.s, b.t, b.gout, beta, widths=[1500, 0, 1501])
    both_backwards(b.s, b.t, b.gout, 0.5, want_t=False)


def test_at_the_scratch_limit_and_beyond():
    v = vj()
    N = 65536
    b = synth.draw("tiny", device="cuda", N=N, V=64, dtype=torch.bfloat16)
    both_backwards(b.s, b.t, b.gout, 0.5)
    big = synth.draw("tiny", device="cuda", N=N + 1, V=64, dtype=torch.bfloat16)
    stats, kl, _ = forward(v, big.s, big.t, 0.5)
    gs = torch.zeros_like(big.s)
    with pytest.raises(v.VjsdArgumentError, match="65536"):
        v.vjsd_bwd_noalloc(v.ShardSet(big.s, big.t, gs=gs), stats, kl, 0.5, big.gout)
    torch.cuda.synchronize()
    assert torch.count_nonzero(gs) == 0  # refused before anything ran
