"""Pins of the fp64 oracle against facts other than itself (CPU only).

Each test ties the oracle to something the pages or the mathematics fix: the
probability-domain brute force with finite-difference gradients, closed forms
(0 for identical inputs, H(beta) for disjoint supports, ln V for a uniform row,
the one-hot / uniform mixture), library routines a special case reduces to
(log_softmax, cross entropy, Categorical entropy, logsumexp in fp64),
invariances the pages state (large common offset, reduced vocabulary, shard
split, empty shard) and the pages' contracts (NaN with zero gradient for a fully
-inf row, +inf KL on underflowed target mass, ignore_index).

Page keys: [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel
generalized JSD with Triton kernels"; [OPS-PR] DeepSpeed PR #8791 "Add
vocabulary-parallel logprobs, entropy and KL ops".
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

NINF = float("-inf")
BETAS = [0.0, 0.1, 0.3, 0.5, 0.9, 1.0]


def rnd(n, v, seed, scale=2.0, dtype=torch.float32):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(n, v, generator=g, dtype=torch.float64) * scale).to(dtype)


def H_beta(b):
    return -b * math.log(b) - (1 - b) * math.log1p(-b)


# ---- statistics ---------------------------------------------------------------------

def test_stats_match_fp64_logsumexp():
    x = rnd(16, 37, 1, 4.0)
    m, lz = oracle.stats(x)
    xd = x.double()
    assert np.array_equal(m, xd.max(1).values.numpy())
    ref = (torch.logsumexp(xd, 1) - xd.max(1).values).numpy()
    np.testing.assert_allclose(lz, ref, rtol=1e-13, atol=1e-13)


def test_stats_shift_invariance_and_split():
    x = torch.round(rnd(8, 50, 2) * 1024) / 1024  # on a 2^-10 grid: +64 stays exact
    m0, l0 = oracle.stats(x)
    m1, l1 = oracle.stats(x + 64.0)
    np.testing.assert_allclose(m1, m0 + 64.0, rtol=0, atol=0)
    np.testing.assert_allclose(l1, l0, rtol=1e-13, atol=1e-13)
    for widths in ([50], [25, 25], [10, 0, 40], [0, 50, 0], [1] * 50):
        m2, l2 = oracle.stats(x, widths=widths)
        np.testing.assert_array_equal(m2, m0)
        np.testing.assert_allclose(l2, l0, rtol=1e-13, atol=1e-13)


def test_stats_reduced_vocabulary():
    """-inf columns are equivalent to removing them [OPS-PR, Tests]."""
    x = rnd(4, 30, 3)
    keep = torch.ones(30, dtype=torch.bool)
    keep[[0, 7, 8, 29]] = False
    xm = x.clone()
    xm[:, ~keep] = NINF
    np.testing.assert_allclose(np.stack(oracle.stats(xm)),
                               np.stack(oracle.stats(x[:, keep].contiguous())),
                               rtol=1e-13, atol=1e-13)


def test_widening_of_stored_formats_is_exact():
    """Every fp16 and bf16 bit pattern widens to the value the libraries give."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    for dt in (torch.float16, torch.bfloat16):
        x = bits.view(dt).reshape(256, 256)
        finite = torch.isfinite(x.double())
        x = torch.where(finite, x, torch.zeros((), dtype=dt))
        r = oracle.jsd(x, x, 0.5, grads=False)  # runs the reader on every pattern
        assert r["loss"].shape == (256,)
        m, _ = oracle.stats(x)
        np.testing.assert_array_equal(m, x.double().max(1).values.numpy())
        # single-column rows: the max is the element itself
        col = x.reshape(-1, 1).contiguous()
        m1, lz1 = oracle.stats(col)
        np.testing.assert_array_equal(m1, col.double().flatten().numpy())
        assert np.all(lz1 == 0.0)


# ---- JSD against the brute force and finite differences -----------------------------

@pytest.mark.parametrize("beta", BETAS)
def test_jsd_matches_probability_domain_brute_force(beta):
    s = rnd(6, 11, 10)
    t = rnd(6, 11, 11, 3.0)
    t[1, 3] = NINF  # partial masks on either side
    s[2, 5] = NINF
    t[3, [0, 4]] = NINF
    s[3, [4, 9]] = NINF
    r = oracle.jsd(s, t, beta, widths=[4, 0, 7])
    for i in range(6):
        ref = brute.jsd(s[i].tolist(), t[i].tolist(), beta)
        if math.isinf(ref):
            assert r["loss"][i] == ref
        else:
            assert r["loss"][i] == pytest.approx(ref, rel=1e-12, abs=1e-14)


@pytest.mark.parametrize("beta", BETAS)
def test_jsd_gradients_match_finite_differences(beta):
    s = rnd(3, 6, 20)
    t = rnd(3, 6, 21, 1.5)
    t[2, 1] = NINF
    s[2, 4] = NINF
    gout = np.array([1.0, 0.7, 1.3])
    r = oracle.jsd(s, t, beta, gout=gout)
    for i in range(3):
        if math.isinf(r["loss"][i]):
            continue
        sv, tv = s[i].tolist(), t[i].tolist()
        fs = brute.fd_grad(lambda z: gout[i] * brute.jsd(z, tv, beta), sv)
        ft = brute.fd_grad(lambda z: gout[i] * brute.jsd(sv, z, beta), tv)
        np.testing.assert_allclose(r["gs"][i], fs, rtol=1e-6, atol=1e-9)
        np.testing.assert_allclose(r["gt"][i], ft, rtol=1e-6, atol=1e-9)


def test_identical_inputs_give_zero():
    x = rnd(5, 40, 30)
    for beta in BETAS:
        r = oracle.jsd(x, x, beta)
        assert np.all(np.abs(r["loss"]) < 1e-14)
        assert np.all(np.abs(r["gs"]) < 1e-15) and np.all(np.abs(r["gt"]) < 1e-15)


@pytest.mark.parametrize("beta", [0.1, 0.3, 0.5, 0.9])
def test_disjoint_supports_give_H_beta_and_zero_gradient(beta):
    """Disjoint supports reach the upper bound H(beta) exactly."""
    s = rnd(4, 20, 40)
    t = rnd(4, 20, 41)
    s[:, 10:] = NINF
    t[:, :10] = NINF
    r = oracle.jsd(s, t, beta)
    np.testing.assert_allclose(r["loss"], H_beta(beta), rtol=1e-13)
    np.testing.assert_allclose(r["kt"], -math.log(beta), rtol=1e-13)
    np.testing.assert_allclose(r["ks"], -math.log1p(-beta), rtol=1e-13)
    assert np.all(np.abs(r["gs"]) < 1e-15) and np.all(np.abs(r["gt"]) < 1e-15)


def test_bounds_and_symmetry():
    s = rnd(20, 33, 50, 3.0)
    t = rnd(20, 33, 51, 1.0)
    for beta in [0.1, 0.25, 0.5, 0.8]:
        r = oracle.jsd(s, t, beta)
        assert np.all(r["loss"] >= 0) and np.all(r["loss"] <= H_beta(beta) + 1e-15)
        q = oracle.jsd(t, s, 1.0 - beta)  # swap roles and weights
        np.testing.assert_allclose(r["loss"], q["loss"], rtol=1e-12)
        np.testing.assert_allclose(r["gs"], q["gt"], rtol=1e-10, atol=1e-16)
        np.testing.assert_allclose(r["gt"], q["gs"], rtol=1e-10, atol=1e-16)
    # the endpoints swap into each other as well
    np.testing.assert_allclose(oracle.jsd(s, t, 0.0)["loss"], oracle.jsd(t, s, 1.0)["loss"],
                               rtol=1e-12)


def test_entropy_form_of_the_jsd():
    """JSD = H(M) - beta H(p_t) - (1 - beta) H(p_s), evaluated by library routines."""
    s = rnd(7, 25, 60)
    t = rnd(7, 25, 61, 0.7)
    for beta in [0.2, 0.5, 0.7]:
        ps = torch.softmax(s.double(), 1)
        pt = torch.softmax(t.double(), 1)
        M = beta * pt + (1 - beta) * ps
        ent = lambda p: torch.special.entr(p).sum(1)
        ref = ent(M) - beta * ent(pt) - (1 - beta) * ent(ps)
        np.testing.assert_allclose(oracle.jsd(s, t, beta, grads=False)["loss"], ref.numpy(),
                                   rtol=1e-11, atol=1e-15)


def test_one_hot_teacher_against_uniform_student_closed_form():
    V = 50
    s = torch.zeros(1, V)
    t = torch.full((1, V), NINF)
    t[0, 7] = 0.0
    for beta in [0.1, 0.5, 0.9]:
        r = oracle.jsd(s, t, beta)
        Ma = beta + (1 - beta) / V
        KT = -math.log(Ma)
        KS = (1 / V) * math.log((1 / V) / Ma) - ((V - 1) / V) * math.log(1 - beta)
        assert r["kt"][0] == pytest.approx(KT, rel=1e-13)
        assert r["ks"][0] == pytest.approx(KS, rel=1e-13)
        assert r["loss"][0] == pytest.approx(beta * KT + (1 - beta) * KS, rel=1e-13)


def test_two_token_closed_form():
    """V = 2: softmax is the logistic function of the logit difference."""
    s = torch.tensor([[0.3, -1.1], [2.0, 2.0], [-5.0, 4.0]])
    t = torch.tensor([[1.7, 0.2], [0.0, 3.0], [1.0, 1.5]])
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    for beta in [0.1, 0.5, 0.9]:
        r = oracle.jsd(s, t, beta, grads=False)
        for i in range(3):
            a = sig(s[i, 0].item() - s[i, 1].item())
            b = sig(t[i, 0].item() - t[i, 1].item())
            m = beta * b + (1 - beta) * a
            kl = lambda p, q: p * math.log(p / q) + (1 - p) * math.log((1 - p) / (1 - q))
            assert r["loss"][i] == pytest.approx(beta * kl(b, m) + (1 - beta) * kl(a, m),
                                                 rel=1e-12)


# ---- endpoints ------------------------------------------------------------------------

def test_endpoints_are_the_kl_definitions():
    s = rnd(9, 31, 70)
    t = rnd(9, 31, 71, 1.2)
    lps = torch.log_softmax(s.double(), 1)
    lpt = torch.log_softmax(t.double(), 1)
    fwd = (lpt.exp() * (lpt - lps)).sum(1)
    rev = (lps.exp() * (lps - lpt)).sum(1)
    np.testing.assert_allclose(oracle.kl_div(s, t)["loss"], fwd.numpy(), rtol=1e-12)
    np.testing.assert_allclose(oracle.kl_div(s, t, reverse=True)["loss"], rev.numpy(),
                               rtol=1e-12)
    # gradients of the endpoints against fp64 autograd of the library form
    sd = s.double().requires_grad_()
    td = t.double().requires_grad_()
    g = torch.linspace(0.5, 1.5, 9, dtype=torch.float64)
    for reverse, val in ((False, None), (True, None)):
        a = torch.log_softmax(sd, 1)
        b = torch.log_softmax(td, 1)
        f = (a.exp() * (a - b)).sum(1) if reverse else (b.exp() * (b - a)).sum(1)
        gs_, gt_ = torch.autograd.grad((f * g).sum(), (sd, td))
        r = oracle.kl_div(s, t, reverse=reverse, gout=g.numpy())
        np.testing.assert_allclose(r["gs"], gs_.numpy(), rtol=1e-10, atol=1e-15)
        np.testing.assert_allclose(r["gt"], gt_.numpy(), rtol=1e-10, atol=1e-15)


def test_forward_kl_to_one_hot_teacher_is_cross_entropy():
    s = rnd(6, 40, 80)
    y = torch.tensor([0, 3, 39, 17, 17, 5])
    t = torch.full((6, 40), NINF)
    t[torch.arange(6), y] = 1.0
    ce = torch.nn.functional.cross_entropy(s.double(), y, reduction="none")
    np.testing.assert_allclose(oracle.kl_div(s, t)["loss"], ce.numpy(), rtol=1e-12)


def test_endpoints_are_branches_not_limits():
    """[JSD-PR, Changes]: beta=0 / 1 are explicit branches; the interior tends to 0."""
    s = rnd(4, 20, 90)
    t = rnd(4, 20, 91)
    for b_int, b_end in ((1e-9, 0.0), (1 - 1e-9, 1.0)):
        near = oracle.jsd(s, t, b_int)["loss"]
        end = oracle.jsd(s, t, b_end)["loss"]
        assert np.all(near < 1e-7) and np.all(end > 1e-3)


# ---- masks, undefined rows, infinite KL, offsets, splits ------------------------------

def test_fully_masked_row_is_nan_with_zero_gradient():
    """[OPS-PR, review]: no distribution -> NaN value, exactly zero gradient."""
    s = rnd(3, 12, 100)
    t = rnd(3, 12, 101)
    s[0] = NINF  # student undefined
    t[1] = NINF  # teacher undefined
    for beta in BETAS:
        r = oracle.jsd(s, t, beta, gout=np.array([7.0, 7.0, 1.0]))
        assert math.isnan(r["loss"][0]) and math.isnan(r["loss"][1])
        assert not math.isnan(r["loss"][2])
        for k in ("gs", "gt"):
            assert np.all(r[k][:2] == 0.0)
            assert np.all(np.isfinite(r[k][2]))
    e = oracle.entropy(s)
    assert math.isnan(e["ent"][0]) and np.all(e["gx"][0] == 0.0)
    ids = np.array([[0, -100], [1, 2], [3, 4]])
    lp = oracle.logprobs(s, ids)
    assert math.isnan(lp["out"][0, 0]) and lp["out"][0, 1] == 0.0
    assert np.all(lp["gx"][0] == 0.0)


def test_kl_is_infinite_when_target_mass_meets_a_masked_token():
    """[OPS-PR, Tests]: decided on logits, even when the mass underflows."""
    s = rnd(2, 10, 110)
    t = rnd(2, 10, 111)
    s[:, 4] = NINF
    t[0, 4] = -1000.0  # mass underflows to exactly 0 even in fp64
    t[1, 4] = NINF  # both masked: finite
    r = oracle.kl_div(s, t)
    assert r["loss"][0] == math.inf and math.isfinite(r["loss"][1])
    # the non-target (student) side gradient stays finite
    assert np.all(np.isfinite(r["gs"]))
    rr = oracle.kl_div(t, s, reverse=True)
    assert rr["loss"][0] == math.inf and math.isfinite(rr["loss"][1])
    # interior JSD never goes infinite
    assert np.all(np.isfinite(oracle.jsd(s, t, 0.5)["loss"]))


def test_masked_tokens_reduce_the_vocabulary():
    s = rnd(5, 24, 120)
    t = rnd(5, 24, 121)
    drop = [2, 3, 11, 23]
    keep = [j for j in range(24) if j not in drop]
    sm, tm = s.clone(), t.clone()
    sm[:, drop] = NINF
    tm[:, drop] = NINF
    for beta in BETAS:
        a = oracle.jsd(sm, tm, beta)
        b = oracle.jsd(s[:, keep].contiguous(), t[:, keep].contiguous(), beta)
        np.testing.assert_allclose(a["loss"], b["loss"], rtol=1e-12)
        np.testing.assert_allclose(a["gs"][:, keep], b["gs"], rtol=1e-10, atol=1e-16)
        assert np.all(a["gs"][:, drop] == 0.0) and np.all(a["gt"][:, drop] == 0.0)


def test_large_common_offset_changes_nothing():
    """[OPS-PR, How]: +1e4 on a row; the oracle for it is the unshifted row."""
    base = rnd(6, 64, 130)
    shifted = (base + 1e4).float()  # stored values
    unshifted = shifted - 1e4  # exact (Sterbenz): the same logits without offset
    assert torch.equal((unshifted + 1e4), shifted)
    for beta in BETAS:
        a = oracle.jsd(shifted, shifted.flip(1).contiguous(), beta)
        b = oracle.jsd(unshifted, unshifted.flip(1).contiguous(), beta)
        np.testing.assert_allclose(a["loss"], b["loss"], rtol=1e-11, atol=1e-14)
        np.testing.assert_allclose(a["gs"], b["gs"], rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(oracle.entropy(shifted)["ent"], oracle.entropy(unshifted)["ent"],
                               rtol=1e-12)


@pytest.mark.parametrize("widths", [[60, 0, 40, 28], [128], [1, 127], [0, 0, 128],
                                    [64, 64], [127, 1, 0]])
def test_results_do_not_depend_on_the_shard_split(widths):
    s = rnd(4, 128, 140)
    t = rnd(4, 128, 141)
    t[1, 100:] = NINF
    for beta in BETAS:
        a = oracle.jsd(s, t, beta, widths=widths)
        b = oracle.jsd(s, t, beta)
        np.testing.assert_allclose(a["loss"], b["loss"], rtol=1e-12)
        np.testing.assert_allclose(a["gs"], b["gs"], rtol=1e-10, atol=1e-17)
        np.testing.assert_allclose(a["gt"], b["gt"], rtol=1e-10, atol=1e-17)
    np.testing.assert_allclose(oracle.entropy(s, widths=widths)["ent"],
                               oracle.entropy(s)["ent"], rtol=1e-12)


def test_gradient_rows_sum_to_zero():
    """Softmax gradients have the form p * (a - E_p a), which sums to 0."""
    s = rnd(5, 70, 150)
    t = rnd(5, 70, 151)
    for beta in BETAS:
        r = oracle.jsd(s, t, beta)
        assert np.all(np.abs(r["gs"].sum(1)) < 1e-14)
        assert np.all(np.abs(r["gt"].sum(1)) < 1e-14)
    assert np.all(np.abs(oracle.entropy(s)["gx"].sum(1)) < 1e-14)
    ids = np.array([[1, 2, 2], [3, -100, 4], [0, 0, 0], [5, 6, 7], [8, 9, 69]])
    assert np.all(np.abs(oracle.logprobs(s, ids)["gx"].sum(1)) < 1e-14)


# ---- entropy and logprobs ---------------------------------------------------------------

def test_entropy_closed_forms_and_library():
    V = 37
    x = torch.zeros(2, V)
    x[1] = NINF
    x[1, 5] = 3.0
    e = oracle.entropy(x)
    assert e["ent"][0] == pytest.approx(math.log(V), rel=1e-14)
    assert e["ent"][1] == 0.0
    y = rnd(8, V, 160)
    ref = torch.distributions.Categorical(logits=y.double()).entropy()
    np.testing.assert_allclose(oracle.entropy(y)["ent"], ref.numpy(), rtol=1e-12)
    for i in range(3):
        fd = brute.fd_grad(brute.entropy, y[i].tolist())
        np.testing.assert_allclose(oracle.entropy(y)["gx"][i], fd, rtol=1e-6, atol=1e-9)


def test_logprobs_against_log_softmax_and_autograd():
    x = rnd(6, 19, 170)
    ids = np.array([[0, 5, 18], [-100, 2, 2], [7, -100, -100], [1, 1, 1], [18, 0, 3],
                    [4, 4, -100]])
    g = np.linspace(0.5, 1.5, 18).reshape(6, 3)
    r = oracle.logprobs(x, ids, gout=g, widths=[5, 0, 14])
    xd = x.double().requires_grad_()
    lp = torch.log_softmax(xd, 1)
    valid = torch.tensor(ids != -100)
    idt = torch.tensor(np.where(ids == -100, 0, ids))
    ref = torch.where(valid, lp.gather(1, idt), torch.zeros((), dtype=torch.float64))
    np.testing.assert_allclose(r["out"], ref.detach().numpy(), rtol=1e-13, atol=1e-15)
    assert np.all(r["out"][ids == -100] == 0.0)
    (gx,) = torch.autograd.grad((ref * torch.tensor(g)).sum(), xd)
    np.testing.assert_allclose(r["gx"], gx.numpy(), rtol=1e-12, atol=1e-15)
    # the probabilities of a row sum to one
    all_ids = np.tile(np.arange(19), (6, 1))
    assert np.allclose(np.exp(oracle.logprobs(x, all_ids, grads=False)["out"]).sum(1), 1.0,
                       rtol=1e-14)


def test_logprobs_rejects_out_of_range_ids():
    x = rnd(2, 8, 180)
    for bad in (8, -1, 1 << 40):
        with pytest.raises(ValueError):
            oracle.logprobs(x, np.array([[0, bad], [1, 2]]))
    oracle.logprobs(x, np.array([[0, -7], [1, 2]]), ignore_index=-7)


def test_half_precision_inputs_follow_their_fp32_widening():
    """The oracle reads bf16 / fp16 storage exactly: it equals the fp32 upcast."""
    s = rnd(4, 33, 190)
    t = rnd(4, 33, 191)
    for dt in (torch.float16, torch.bfloat16):
        a = oracle.jsd(s.to(dt), t.to(dt), 0.3)
        b = oracle.jsd(s.to(dt).float(), t.to(dt).float(), 0.3)
        np.testing.assert_array_equal(a["loss"], b["loss"])
        np.testing.assert_array_equal(a["gs"], b["gs"])
