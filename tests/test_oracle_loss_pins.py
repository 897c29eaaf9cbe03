"""Pins of the oracle's distillation loss (``oracle.jsd_loss``): temperature, T^2
scaling, masked sum / mean reductions and the chain rule through them (CPU only).

What fixes each part, independently of the function's own arithmetic:
  - T = 1, no mask, no reduction is the per-token JSD (itself pinned elsewhere);
  - scale equivariance: dividing 2s, 2t by T = 2 gives the T = 1 loss of s, t
    exactly, with gradients halved (powers of two are exact in fp64);
  - the high-temperature limit: T^2 JSD_beta -> beta (1-beta) / (2V) sum_i (d_i - dbar)^2
    with d = t - s (the second-order expansion of both KL-to-mixture terms around
    the uniform distribution; 1 / (2V) for the KL endpoints), within O(1/T);
  - reduction identities: one kept row returns that row, the mean over all rows
    times N is the sum, no kept rows give 0 with zero gradients, and a masked
    undefined row does not reach the result;
  - central finite differences of the reduced loss with respect to the raw logits.
Every check runs against the oracle, and against planted mistakes in a copy of
its source, each of which must fail at least one check.
"""
import inspect
import math

import numpy as np
import pytest
import torch

import oracle

BETAS = [0.3, 0.0, 1.0]


def _data(seed, N=4, V=9, scale=2.0):
    g = torch.Generator().manual_seed(seed)
    s = torch.randn(N, V, generator=g, dtype=torch.float64) * scale
    t = torch.randn(N, V, generator=g, dtype=torch.float64) * scale
    return s, t


def check_t1_is_per_token_jsd(fn):
    s, t = _data(1)
    for beta in BETAS:
        g = np.linspace(0.5, 1.5, s.shape[0])
        got = fn(s, t, beta, grad=g)
        ref = oracle.jsd(s, t, beta, gout=g)
        np.testing.assert_array_equal(got["rows"], ref["loss"])
        np.testing.assert_allclose(got["gs"], ref["gs"], rtol=0, atol=0)
        np.testing.assert_allclose(got["gt"], ref["gt"], rtol=0, atol=0)


def check_scale_equivariance(fn):
    s, t = _data(2)
    g = np.array([1.0, 0.5, 2.0, 1.25])
    for beta in BETAS:
        a = fn(s, t, beta, temperature=1.0, grad=g)
        b = fn(2 * s, 2 * t, beta, temperature=2.0, grad=g)
        c = fn(s / 2, t / 2, beta, temperature=0.5, grad=g)
        np.testing.assert_allclose(b["rows"], a["rows"], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(c["rows"], a["rows"], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(2 * b["gs"], a["gs"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(2 * b["gt"], a["gt"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(c["gs"] / 2, a["gs"], rtol=1e-12, atol=1e-15)


def check_high_temperature_limit(fn):
    s, t = _data(3, N=3, V=40)
    d = (t - s).numpy()
    dc = d - d.mean(axis=1, keepdims=True)
    V = s.shape[1]
    for beta in BETAS:
        w = beta * (1 - beta) if 0 < beta < 1 else 1.0
        lim = w / (2 * V) * (dc ** 2).sum(axis=1)
        T = 1e4
        scaled = fn(s, t, beta, temperature=T, scale_t2=True, grads=False)["rows"]
        plain = fn(s, t, beta, temperature=T, grads=False)["rows"]
        np.testing.assert_allclose(scaled, lim, rtol=1e-4)
        np.testing.assert_allclose(plain * T * T, lim, rtol=1e-4)


def check_reductions(fn):
    s, t = _data(4, N=5)
    s[2] = float("-inf")  # an undefined row, masked out below
    for beta in BETAS:
        per = fn(s, t, beta, temperature=1.5, scale_t2=True, grads=False)["rows"]
        assert np.isnan(per[2])
        keep = np.array([1, 1, 0, 1, 1], np.uint8)
        ref = per[keep.astype(bool)]
        m = fn(s, t, beta, temperature=1.5, scale_t2=True, mask=keep, reduction="mean", grad=1.0)
        u = fn(s, t, beta, temperature=1.5, scale_t2=True, mask=keep, reduction="sum", grad=1.0)
        assert np.isfinite(m["out"]) and np.isfinite(u["out"])
        np.testing.assert_allclose(m["out"] * 4, u["out"], rtol=1e-13)
        np.testing.assert_allclose(u["out"], math.fsum(ref), rtol=1e-13)
        assert m["rows"][2] == 0.0 and not m["gs"][2].any() and not m["gt"][2].any()
        for k in (0, 3):
            one = np.zeros(5, np.uint8)
            one[k] = 1
            r = fn(s, t, beta, temperature=1.5, scale_t2=True, mask=one, reduction="mean", grad=1.0)
            assert r["out"] == per[k]
            assert not r["gs"][np.arange(5) != k].any()
        z = fn(s, t, beta, mask=np.zeros(5, np.uint8), reduction="mean", grad=1.0)
        assert z["out"] == 0.0 and not z["gs"].any() and not z["gt"].any()


def check_finite_differences(fn):
    s, t = _data(5, N=3, V=5)
    keep = np.array([1, 0, 1], np.uint8)
    h = 1e-6
    for beta in BETAS:
        for red, kw in (("mean", dict(scale_t2=True)), ("sum", {}), ("none", dict(scale_t2=True))):
            grad = np.array([0.7, 1.1, 1.3]) if red == "none" else 0.8

            def value(a, b):
                r = fn(a, b, beta, temperature=1.7, mask=keep, reduction=red, grads=False, **kw)
                return float(np.dot(grad, r["rows"])) if red == "none" else grad * r["out"]

            got = fn(s, t, beta, temperature=1.7, mask=keep, reduction=red, grad=grad, **kw)
            for which, key in ((0, "gs"), (1, "gt")):
                fd = np.zeros(s.shape)
                for i in range(s.shape[0]):
                    for j in range(s.shape[1]):
                        ab = [s.clone(), t.clone()]
                        ab[which][i, j] += h
                        hi = value(*ab)
                        ab[which][i, j] -= 2 * h
                        lo = value(*ab)
                        fd[i, j] = (hi - lo) / (2 * h)
                np.testing.assert_allclose(got[key], fd, rtol=2e-6, atol=1e-9,
                                           err_msg=f"{key} beta={beta} {red}")


CHECKS = [check_t1_is_per_token_jsd, check_scale_equivariance, check_high_temperature_limit,
          check_reductions, check_finite_differences]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_loss_pins(check):
    check(oracle.jsd_loss)


# (name, text in the oracle's source, planted replacement)
MUTANTS = [
    ("temperature_multiplies", "st = s.double() / T", "st = s.double() * T"),
    ("grad_missing_inv_temperature", 'res["gs"] = np.where(keep[:, None], ref["gs"] / T, 0.0)',
     'res["gs"] = np.where(keep[:, None], ref["gs"], 0.0)'),
    ("t2_missing_in_gradient", "g = np.where(keep, g * fac, 0.0)", "g = np.where(keep, g, 0.0)"),
    ("t2_missing_in_rows", 'rows = np.where(keep, ref["loss"] * fac, 0.0)',
     'rows = np.where(keep, ref["loss"], 0.0)'),
    ("mean_grad_over_all_rows",
     "g = np.full(N, (0.0 if grad is None else float(grad)) / max(count, 1))",
     "g = np.full(N, (0.0 if grad is None else float(grad)) / N)"),
    ("mean_value_over_all_rows", 'out = tot / max(count, 1) if reduction == "mean" else tot',
     'out = tot / N if reduction == "mean" else tot'),
    ("masked_rows_not_zeroed", 'rows = np.where(keep, ref["loss"] * fac, 0.0)',
     'rows = ref["loss"] * fac'),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.jsd_loss)
    assert src.count(old) == 1, old
    ns = {"np": np, "jsd": oracle.jsd}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["jsd_loss"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_loss_pins_catch_planted_mistake(name, old, new):
    fn = _mutant(old, new)
    failed = []
    for check in CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught {name}"
