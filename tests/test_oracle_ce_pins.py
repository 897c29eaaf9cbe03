"""Pins of the oracle's cross-entropy (``oracle.cross_entropy``), CPU only: it is the
textbook ``torch.nn.functional.cross_entropy`` in fp64 (with ignore_index, every
reduction, and its autograd gradient), independent of the vocabulary split; a mean
over no labelled token is 0 with zero gradients (the reading of an empty selection);
an undefined row with a label is NaN with zero gradient.  Planted mistakes in a copy
of the function each fail a check."""
import inspect

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _data(seed, N=6, V=11):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(N, V, generator=g, dtype=torch.float64) * 2
    y = torch.randint(0, V, (N,), generator=g)
    y[1] = -100
    y[4] = -100
    return x, y


def check_is_torch_cross_entropy(fn):
    x, y = _data(1)
    for red in ("none", "sum", "mean"):
        grad = torch.rand(6, dtype=torch.float64) + 0.5 if red == "none" else torch.tensor(0.7, dtype=torch.float64)
        xr = x.clone().requires_grad_()
        ref = F.cross_entropy(xr, y, ignore_index=-100, reduction=red)
        (ref * grad).sum().backward()
        got = fn(x, y.numpy(), -100, red, grad=grad.numpy() if red == "none" else float(grad))
        val = got["rows"] if red == "none" else got["out"]
        np.testing.assert_allclose(val, ref.detach().numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(got["gx"], xr.grad.numpy(), rtol=1e-12, atol=1e-15)
        for w in ([4, 7], [1, 0, 10], [11]):
            sh = fn(x, y.numpy(), -100, red, grad=grad.numpy() if red == "none" else float(grad),
                    widths=w)
            np.testing.assert_allclose(sh["rows"], got["rows"], rtol=1e-13, atol=1e-15)


def check_no_label_and_undefined(fn):
    x, y = _data(2)
    none = np.full(6, -100)
    r = fn(x, none, -100, "mean", grad=1.0)
    assert r["out"] == 0.0 and not r["gx"].any() and not r["rows"].any()
    x[2] = float("-inf")
    r = fn(x, y.numpy(), -100, "mean", grad=1.0)
    assert np.isnan(r["rows"][2]) and np.isnan(r["out"]) and not r["gx"][2].any()
    assert r["rows"][1] == 0.0 and not r["gx"][1].any()


CHECKS = [check_is_torch_cross_entropy, check_no_label_and_undefined]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_ce_pins(check):
    check(oracle.cross_entropy)


MUTANTS = [
    ("sign", "rows = np.where(valid, -lp[\"out\"][:, 0], 0.0)", "rows = np.where(valid, lp[\"out\"][:, 0], 0.0)"),
    ("mean_over_all", "out = tot / max(count, 1) if reduction == \"mean\" else tot",
     "out = tot / N if reduction == \"mean\" else tot"),
    ("grad_sign", "gout=-g[:, None]", "gout=g[:, None]"),
    ("mean_grad_over_all", "g = np.full(N, (0.0 if grad is None else float(grad)) / max(count, 1))",
     "g = np.full(N, (0.0 if grad is None else float(grad)) / N)"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.cross_entropy)
    assert src.count(old) == 1, old
    ns = {"np": np, "logprobs": oracle.logprobs}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["cross_entropy"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_ce_pins_catch_planted_mistake(name, old, new):
    fn = _mutant(old, new)
    failed = []
    for check in CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught {name}"
