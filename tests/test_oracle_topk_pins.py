"""Pins of the oracle's teacher top-k forward KL (``oracle.topk_kl``), CPU only.

What fixes it, independently of its own arithmetic:
  - full coverage: with every id listed and the teacher's exact log-probabilities,
    it is the dense forward KL(p_t || p_s) of the pinned per-token oracle, gradients
    included;
  - a one-hot teacher (one id, log-probability 0) gives the cross-entropy of that id
    (textbook ``cross_entropy`` in fp64);
  - padding: ignored ids and -inf teacher log-probabilities change nothing;
  - +inf when the teacher has mass (even an underflowing amount) on an id whose
    student logit is -inf; NaN and zero gradient for an undefined student row;
  - central finite differences of the value with respect to the student logits.
Every check also runs against planted mistakes in a copy of the function's source.
"""
import inspect

import numpy as np
import pytest
import torch

import oracle


def _data(seed, N=4, V=9):
    g = torch.Generator().manual_seed(seed)
    s = torch.randn(N, V, generator=g, dtype=torch.float64) * 2
    te = torch.randn(N, V, generator=g, dtype=torch.float64) * 2
    return s, te


def check_full_coverage_is_dense_forward_kl(fn):
    s, te = _data(1)
    N, V = s.shape
    tl = torch.log_softmax(te, 1).numpy()
    ids = np.tile(np.arange(V), (N, 1))
    g = np.array([1.0, 0.5, 2.0, 1.5])
    a = fn(s, ids, tl, gout=g)
    b = oracle.jsd(s, te, 0.0, gout=g)
    np.testing.assert_allclose(a["kl"], b["loss"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["gx"], b["gs"], rtol=1e-10, atol=1e-14)
    perm = np.stack([np.random.default_rng(r).permutation(V) for r in range(N)])
    c = fn(s, perm, np.take_along_axis(tl, perm, 1), gout=g)  # slot order is irrelevant
    np.testing.assert_allclose(c["kl"], b["loss"], rtol=1e-12, atol=1e-14)


def check_one_hot_teacher_is_cross_entropy(fn):
    s, _ = _data(2)
    y = torch.tensor([3, 0, 8, 5])
    r = fn(s, y[:, None].numpy(), np.zeros((4, 1)), gout=np.ones(4))
    ce = torch.nn.functional.cross_entropy(s, y, reduction="none").numpy()
    np.testing.assert_allclose(r["kl"], ce, rtol=1e-13)
    sr = s.clone().requires_grad_()
    torch.nn.functional.cross_entropy(sr, y, reduction="sum").backward()
    np.testing.assert_allclose(r["gx"], sr.grad.numpy(), rtol=1e-12, atol=1e-15)


def check_padding_changes_nothing(fn):
    s, te = _data(3)
    tl = torch.log_softmax(te, 1).numpy()
    ids = np.array([[1, 4, 2], [0, 8, 3], [5, 6, 7], [2, 2, 1]])
    t = np.take_along_axis(tl, ids, 1)
    g = np.array([1.0, 2.0, 0.5, 1.0])
    a = fn(s, ids, t, gout=g)
    pad_ids = np.concatenate([ids, np.full((4, 2), -100), ids[:, :1]], 1)
    pad_t = np.concatenate([t, np.array([[0.3, -2.0]] * 4), np.full((4, 1), -np.inf)], 1)
    b = fn(s, pad_ids, pad_t, gout=g)
    np.testing.assert_allclose(b["kl"], a["kl"], rtol=1e-14)
    np.testing.assert_allclose(b["gx"], a["gx"], rtol=1e-14, atol=1e-16)


def check_infinities_and_undefined_rows(fn):
    s, te = _data(4)
    s[1, 4] = float("-inf")
    s[2] = float("-inf")
    ids = np.array([[0, 1], [4, 2], [0, 1], [3, 4]])
    t = np.array([[-1.0, -2.0], [-1000.0, -0.5], [-1.0, -1.0], [-1.0, -3.0]])
    r = fn(s, ids, t, gout=np.ones(4))
    assert r["kl"][1] == np.inf  # exp(-1000) underflows, the mass is still there
    assert np.isnan(r["kl"][2]) and not r["gx"][2].any()
    assert np.isfinite(r["kl"][[0, 3]]).all()
    z = fn(s, np.array([[4, -100]] * 4), np.array([[-np.inf, 0.0]] * 4), gout=np.ones(4))
    assert z["kl"][1] == 0.0  # no teacher mass on the masked token: no +inf
    assert np.isnan(z["kl"][2]) and not z["gx"][2].any()  # undefined even with no valid slot


def check_finite_differences(fn):
    s, te = _data(5, N=3, V=6)
    ids = np.array([[0, 2, 5], [1, 1, 3], [4, -100, 0]])
    t = np.array([[-0.7, -1.2, -2.5], [-0.4, -1.9, -3.0], [-0.2, 0.0, -1.7]])
    g = np.array([0.9, 1.3, 0.6])
    r = fn(s, ids, t, gout=g)
    h = 1e-6
    fd = np.zeros(s.shape)
    for i in range(3):
        for j in range(6):
            x = s.clone()
            x[i, j] += h
            hi = np.dot(g, fn(x, ids, t, grads=False)["kl"])
            x[i, j] -= 2 * h
            lo = np.dot(g, fn(x, ids, t, grads=False)["kl"])
            fd[i, j] = (hi - lo) / (2 * h)
    np.testing.assert_allclose(r["gx"], fd, rtol=2e-6, atol=1e-9)


CHECKS = [check_full_coverage_is_dense_forward_kl, check_one_hot_teacher_is_cross_entropy,
          check_padding_changes_nothing, check_infinities_and_undefined_rows,
          check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_topk_pins(check):
    check(oracle.topk_kl)


MUTANTS = [
    ("ratio_sign", "* (t - lps)", "* (lps - t)"),
    ("weight_without_exp", "-g[:, None] * np.exp(np.where(valid, t, 0.0))",
     "-g[:, None] * np.where(valid, t, 0.0)"),
    ("gradient_weight_sign", "w = np.where(valid, -g[:, None]", "w = np.where(valid, g[:, None]"),
    ("padding_counted", "valid = (idv != ignore_index) & (t > -np.inf)", "valid = (t > -np.inf)"),
    ("inf_rule_lost", "terms = np.where(valid & (lps == -np.inf), np.inf, terms)", "pass"),
    ("undefined_not_nan", "kl = np.where(undefined, np.nan, kl)", "pass"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.topk_kl)
    assert src.count(old) == 1, old
    ns = {"np": np, "logprobs": oracle.logprobs, "stats": oracle.stats}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["topk_kl"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_topk_pins_catch_planted_mistake(name, old, new):
    fn = _mutant(old, new)
    failed = []
    for check in CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(fn)
        except (AssertionError, ValueError):
            failed.append(check.__name__)
    assert failed, f"no pin caught {name}"
