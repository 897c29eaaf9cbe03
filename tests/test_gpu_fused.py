"""GPU parity of the whole-forward call (vjsd_forward): against the fp64 oracle and
against the three separate launches, over dtypes, the beta = 0 / 1 branches (one-pass
KL), row widths at each register-tile size of the rows held in registers (256 lanes up
to 16384 16-bit / 8192 fp32 columns, 512 lanes up to 40960 / 20480) and on both sides of
each limit, batch sizes, masks, offsets, unaligned rows (swept twice) and several
shards (one launch up to eight, three launches beyond)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_stats, assert_values

pytestmark = pytest.mark.gpu

NINF = float("-inf")


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def forward(s, t, beta, widths=None, fused=True):
    v = vj()
    sh = v.ShardSet(s, t, widths=widths)
    N, S = sh.N, sh.S
    part = v.new_part(N, S, s.device)
    stats = torch.full((N, 4), float("nan"), dtype=torch.float64, device=s.device)
    kl = torch.full((N, 2), float("nan"), device=s.device)
    loss = torch.full((N,), float("nan"), device=s.device)
    if fused:
        v.vjsd_forward(sh, beta, part, stats, kl, loss)
    else:
        v.vjsd_stats(sh, 3, part)
        v.vjsd_merge(part, S, N, 3, stats)
        v.vjsd_fwd(sh, stats, beta, part, kl, loss)
    torch.cuda.synchronize()
    return stats.cpu(), kl.cpu(), loss.cpu()


def check(s, t, beta, widths=None):
    dt = s.dtype
    st, kl, loss = forward(s, t, beta, widths)
    sc, tc = s.reshape(-1, s.shape[-1]).cpu(), t.reshape(-1, t.shape[-1]).cpu()
    ref = oracle.jsd(sc, tc, beta, widths=widths, grads=False)
    assert_stats(st, *oracle.stats(sc, widths=widths), 0, "student stats")
    assert_stats(st, *oracle.stats(tc, widths=widths), 1, "teacher stats")
    assert_values(loss, ref["loss"], dt, "loss")
    assert_values(kl[:, 0], ref["kt"], dt, "KL(p_t||M)")
    assert_values(kl[:, 1], ref["ks"], dt, "KL(p_s||M)")
    # the three-launch path agrees within rounding
    st3, kl3, loss3 = forward(s, t, beta, widths, fused=False)
    fin = np.isfinite(loss.numpy())
    np.testing.assert_allclose(loss.numpy()[fin], loss3.numpy()[fin], rtol=2e-6, atol=2e-7)
    assert np.array_equal(np.isnan(loss.numpy()), np.isnan(loss3.numpy()))
    assert np.array_equal(np.isinf(loss.numpy()), np.isinf(loss3.numpy()))
    return loss


# 1000 / 4096 / 8192 / 16032 / 16384: the row held in registers (1, 2, 4, 8 vectors
# per lane of 256); 16392: 6 vectors per lane of 512; 135160 and wider: the row swept
# twice (135160 / 135168 / 135176 leave 511, 512 and 513 vectors after the last whole
# step of 4 vectors per lane of the 512-lane workgroup)
@pytest.mark.parametrize("V", [1000, 4096, 8192, 16032, 16384, 16392, 135160, 135168, 135176,
                               151936])
@pytest.mark.parametrize("beta", [0.5, 0.0, 1.0])
def test_one_pass_forward_bf16(V, beta):
    b = synth.draw("full_vocab", device="cuda", N=40, V=V)
    check(b.s, b.t, beta)


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
@pytest.mark.parametrize("V", [3000, 8192, 12000, 128256])
def test_one_pass_forward_other_dtypes(dtype, V):
    b = synth.draw("tiny", device="cuda", N=24, V=V, dtype=dtype)
    check(b.s, b.t, 0.3)


# 512-lane workgroups holding 6, 8 or 10 vectors per lane of each input: the widths at
# and one vector past each tile (16-bit: 24576 / 32768 / 40960 columns; fp32: 12288 /
# 16384 / 20480), a ragged last tile, and one vector past the last (swept twice); the
# one-rank shares of the pages' short batch (N=1024 rows at 37984 columns) sampled
@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 16392), (torch.bfloat16, 24576),
                                     (torch.bfloat16, 24584), (torch.bfloat16, 32768),
                                     (torch.bfloat16, 32776), (torch.bfloat16, 37984),
                                     (torch.bfloat16, 40960), (torch.bfloat16, 40968),
                                     (torch.float16, 20000), (torch.float16, 40960),
                                     (torch.float32, 8196), (torch.float32, 12288),
                                     (torch.float32, 16388), (torch.float32, 20480),
                                     (torch.float32, 20484)])
def test_wide_register_rows(dtype, V):
    b = synth.draw("full_vocab", device="cuda", N=21, V=V, dtype=dtype)
    check(b.s, b.t, 0.5)
    check(b.s, b.t, 0.1)


def test_wide_register_rows_masks_and_undefined_rows():
    b = synth.draw("robust", device="cuda", N=30, V=30000)  # fp32 -> bf16 below
    s, t = b.s.to(torch.bfloat16), b.t.to(torch.bfloat16)
    s[7] = NINF  # student undefined
    t[8] = NINF  # teacher undefined
    s[9, 50:] = NINF  # partly masked
    s[10, :29997] = NINF  # mass only in the last three columns (the ragged last tile)
    s[11, 123] = NINF  # forward KL of row 11 infinite
    t[11, 123] = 1.0
    loss = check(s, t, 0.5)
    assert np.isnan(loss.numpy()[[7, 8]]).all()
    lf = check(s, t, 0.0)
    assert np.isinf(lf.numpy()[11])


def test_wide_register_rows_pages_short_batch_sampled():
    b = synth.draw("full_vocab", device="cuda", N=1024, V=37984)
    for beta in (0.3, 0.9):
        st, kl, loss = forward(b.s, b.t, beta)
        rows = np.array([0, 1, 511, 512, 1022, 1023])
        ref = oracle.jsd(b.s[rows].cpu(), b.t[rows].cpu(), beta, grads=False)
        assert_values(loss[rows], ref["loss"], torch.bfloat16, "loss")
        assert_values(kl[rows, 0], ref["kt"], torch.bfloat16, "KL(p_t||M)")
        assert_values(kl[rows, 1], ref["ks"], torch.bfloat16, "KL(p_s||M)")
        # each route sums a row's V terms in fp32 in its own order: rounding of order
        # sqrt(V) * 2^-24 relative; four times that, plus the fp32 tolerance's absolute part
        st3, kl3, loss3 = forward(b.s, b.t, beta, fused=False)
        rtol = 4.0 * np.sqrt(b.s.shape[1]) * 2.0 ** -24
        np.testing.assert_allclose(loss.numpy(), loss3.numpy(), rtol=rtol, atol=1e-6)
        np.testing.assert_allclose(kl.numpy(), kl3.numpy(), rtol=rtol, atol=1e-6)


@pytest.mark.parametrize("N", [1, 7, 100, 4097])
def test_one_pass_forward_batch_sizes(N):
    b = synth.draw("full_vocab", device="cuda", N=N, V=16032)
    check(b.s, b.t, 0.9)


# wide rows in batches larger than the number of CUs (41000: just past the rows held in
# registers)
@pytest.mark.parametrize("N,V", [(700, 41000), (300, 140000)])
def test_swept_twice_forward_large_batches(N, V):
    b = synth.draw("full_vocab", device="cuda", N=N, V=V)
    check(b.s, b.t, 0.7)


@pytest.mark.parametrize("dtype,V", [(torch.float32, 40000), (torch.bfloat16, 140000)])
def test_swept_twice_forward_masks_and_undefined_rows(dtype, V):
    b = synth.draw("robust", device="cuda", N=20, V=V)
    s, t = b.s.to(dtype), b.t.to(dtype)
    s[7] = NINF  # student undefined
    t[8] = NINF  # teacher undefined
    s[9, 50:] = NINF  # partly masked
    s[10, :V - 3] = NINF  # mass only in the last three columns (the sweeps' scalar tail)
    s[11, 123] = NINF  # forward KL of row 11 infinite
    t[11, 123] = 1.0
    loss = check(s, t, 0.5)
    assert np.isnan(loss.numpy()[[7, 8]]).all()
    lf = check(s, t, 0.0)
    assert np.isinf(lf.numpy()[11])


def test_one_pass_forward_masks_offsets_undefined_rows():
    b = synth.draw("robust", device="cuda", N=200, V=8000)  # fp32: one workgroup per row
    s, t = b.s.clone(), b.t.clone()
    s[7] = NINF  # student undefined
    t[8] = NINF  # teacher undefined
    s[9, 50:] = NINF  # partly masked
    s[11, 123] = NINF  # forward KL of row 11 infinite
    t[11, 123] = 1.0
    loss = check(s, t, 0.5)
    assert np.isnan(loss.numpy()[[7, 8]]).all()
    lf = check(s, t, 0.0)
    assert np.isinf(lf.numpy()[11])


@pytest.mark.parametrize("name", ["tp8_shard", "full_vocab"])
def test_one_pass_forward_full_size_sampled(name):
    b = synth.draw(name, device="cuda")
    st, kl, loss = forward(b.s, b.t, 0.5)
    rows = np.array([0, 1, 2, 1000, 4095, 4096, 8190, 8191])
    ref = oracle.jsd(b.s[rows].cpu(), b.t[rows].cpu(), 0.5, grads=False)
    assert_values(loss[rows], ref["loss"], torch.bfloat16, "loss")
    assert torch.isfinite(loss).all()
    st3, kl3, loss3 = forward(b.s, b.t, 0.5, fused=False)
    np.testing.assert_allclose(loss.numpy(), loss3.numpy(), rtol=2e-6, atol=2e-7)


def test_layouts_outside_the_register_path():
    b = synth.draw("tiny", device="cuda", N=12, V=1002, dtype=torch.bfloat16)
    check(b.s[:, 1:1001], b.t[:, 1:1001], 0.5)  # rows not 16-byte aligned
    check(b.s[:, :1001], b.t[:, :1001], 0.5)  # width not a multiple of 16 bytes
    check(b.s[:, 1:1001], b.t[:, 2:1002], 0.5)  # student and teacher misaligned apart
    check(b.s, b.t, 0.5, widths=[500, 0, 502])  # several shards
    c = synth.draw("tiny", device="cuda", N=6, V=20003, dtype=torch.bfloat16)
    check(c.s[:, 3:20003], c.t[:, 1:20001], 0.3)  # wide, unaligned: swept twice


def test_autograd_uses_the_one_pass_forward():
    v = vj()
    b = synth.draw("tiny", device="cuda", N=10, V=4096, dtype=torch.bfloat16)
    s = b.s.clone().requires_grad_()
    loss = v.jsd(s, b.t, 0.5)
    _, _, ref = forward(b.s, b.t, 0.5)
    assert torch.equal(loss.detach().cpu(), ref)
    loss.sum().backward()
    assert torch.isfinite(s.grad.float()).all()


# 2 to 8 shards run as one launch (per-shard statistics merged in the workgroup), 9
# and more as the three launches; single-column, empty and all-but-one-empty shards
@pytest.mark.parametrize("widths", [[9000, 11000], [1, 0, 19999], [2500] * 8,
                                    [2000] * 8 + [4000], [0, 0, 20000, 0],
                                    [7, 3, 5000, 0, 14990]])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_sharded_forward(dtype, widths):
    V = sum(widths)
    b = synth.draw("robust", device="cuda", N=37, V=V)
    s, t = b.s.to(dtype).clone(), b.t.to(dtype).clone()
    s[5] = NINF  # student undefined
    t[6] = NINF  # teacher undefined
    s[7, 100:] = NINF  # partly masked, across shard boundaries
    t[8, 2000:2600] = NINF
    loss = check(s, t, 0.4, widths=widths)
    assert np.isnan(loss.numpy()[[5, 6]]).all()
    assert np.isfinite(np.delete(loss.numpy(), [5, 6])).all()


# fp32 rows in 2 to 8 shards hold the widest shard's last five or six full steps (four in
# registers, one or two in LDS: 40960 or 49152 columns) on chip through the merge: the
# widest shard with exactly five or six full steps (an empty prefix) and one column short
# of them (no hold; one LDS step); the widest shard first, in the middle (after shards
# that leave it 4 bytes past a 16-byte boundary: a scalar head before its held steps)
# and last; two equally wide shards (the first holds); masked tokens inside the held
# columns
@pytest.mark.parametrize("widths", [[40960, 100], [40959, 100], [49152, 100], [49151, 100],
                                    [60000, 0, 40000, 28256], [3000, 50001, 7],
                                    [40960, 40960], [1, 2, 45000, 3, 0, 5, 6, 7]])
def test_sharded_forward_held_steps(widths):
    V = sum(widths)
    b = synth.draw("robust", device="cuda", N=23, V=V)  # fp32
    s, t = b.s.clone(), b.t.clone()
    s[5] = NINF  # student undefined
    t[6] = NINF  # teacher undefined
    s[7, 100:] = NINF  # partly masked, across shard boundaries
    q = int(np.argmax(widths))
    end = sum(widths[:q + 1])
    t[8, end - 9000:end - 8000] = NINF  # inside the widest shard's held columns
    loss = check(s, t, 0.4, widths=widths)
    assert np.isnan(loss.numpy()[[5, 6]]).all()
    assert np.isfinite(np.delete(loss.numpy(), [5, 6])).all()
    lf = check(s, t, 0.0, widths=widths)  # forward KL: teacher mass on row 7's masked tokens
    assert np.isinf(lf.numpy()[7])


def test_sharded_forward_separate_tensors():
    """Per-shard tensors with their own allocations and alignments (one shard's rows
    start 2 bytes past a 16-byte boundary), against the oracle on the concatenation."""
    v = vj()
    b = synth.draw("full_vocab", device="cuda", N=29, V=30001)
    cuts = [0, 7001, 7001, 19000, 30001]
    ws = [cuts[i + 1] - cuts[i] for i in range(4)]
    ss, ts = [], []
    for i in range(4):
        a, c = cuts[i], cuts[i + 1]
        if i == 2:  # an unaligned view of a wider buffer
            bs = torch.empty((29, c - a + 1), dtype=b.s.dtype, device="cuda")
            bt = torch.empty((29, c - a + 1), dtype=b.t.dtype, device="cuda")
            bs[:, 1:] = b.s[:, a:c]
            bt[:, 1:] = b.t[:, a:c]
            ss.append(bs[:, 1:])
            ts.append(bt[:, 1:])
        else:
            ss.append(b.s[:, a:c].contiguous())
            ts.append(b.t[:, a:c].contiguous())
    sh = v.ShardSet(ss, ts)
    N = 29
    part = v.new_part(N, 4, "cuda")
    stats = torch.empty((N, 4), dtype=torch.float64, device="cuda")
    kl = torch.empty((N, 2), dtype=torch.float32, device="cuda")
    loss = torch.empty((N,), dtype=torch.float32, device="cuda")
    v.vjsd_forward(sh, 0.6, part, stats, kl, loss)
    torch.cuda.synchronize()
    sc, tc = b.s.cpu(), b.t.cpu()
    ref = oracle.jsd(sc, tc, 0.6, widths=ws, grads=False)
    assert_values(loss.cpu(), ref["loss"], b.s.dtype, "loss")
    assert_stats(stats.cpu(), *oracle.stats(sc, widths=ws), 0, "student stats")
    assert_stats(stats.cpu(), *oracle.stats(tc, widths=ws), 1, "teacher stats")


# The two-sweep forward holds the statistics sweep's last full steps on chip (a step is
# 512 lanes x 4 vectors: 16384 16-bit or 8192 fp32 columns; 16-bit formats hold 2 steps,
# fp32 4 in registers and 1 or 2 in LDS, as many as the row has past the 4).  Widths
# where the held steps take the whole body (empty prefix and rest), one column more or
# fewer, and rows 2 bytes past a 16-byte boundary (a scalar head before the held body);
# fp32 at 5 steps (one in LDS), between 5 and 6, and at 6 (two in LDS).
@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 32768), (torch.bfloat16, 32769),
                                     (torch.bfloat16, 32767), (torch.bfloat16, 49160),
                                     (torch.float16, 16392), (torch.float16, 32768),
                                     (torch.float16, 32769), (torch.float16, 32767),
                                     (torch.float32, 40960), (torch.float32, 40964),
                                     (torch.float32, 40959), (torch.float32, 45000),
                                     (torch.float32, 49152), (torch.float32, 49156),
                                     (torch.float32, 49151), (torch.float32, 57344)])
def test_held_steps_boundaries(dtype, V):
    b = synth.draw("tiny", device="cuda", N=9, V=V + 9, dtype=dtype)
    check(b.s[:, :V], b.t[:, :V], 0.5)  # rows 16-byte aligned when V + 9 allows it
    check(b.s[:, 1:V + 1], b.t[:, 1:V + 1], 0.5)  # a scalar head before the body
    check(b.s[:, 8:V + 8], b.t[:, 8:V + 8], 0.3)
