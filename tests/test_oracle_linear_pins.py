"""Pins of the oracle's fused-linear distillation loss (``oracle.linear_jsd``), CPU only.

The function is the per-token loss of ``oracle.jsd_loss`` evaluated on the products
``hs @ ws^T`` and ``ht @ wt^T``; its gradients with respect to the student's hidden
states and head weight come from the chain rule.  They are pinned by
  * central finite differences of the returned value on tiny shapes (every reduction,
    a temperature with T^2 scaling, a token mask, the KL endpoints);
  * the identity head (V = D, W = I), where the function is ``jsd_loss`` itself;
  * invariances the mathematics fixes: a vector added to every head row shifts each
    row's logits by a constant (softmax is unchanged, so is everything else); the
    gradient of the head weight sums to zero over the vocabulary; an orthogonal
    change of the teacher's hidden basis changes nothing; scaling the hidden states
    by a and the head by 1/a leaves the logits, scales gh by 1/a and gw by a;
  * masked tokens contribute nothing: exactly zero gradient rows, and the mean equals
    the mean over the kept tokens alone.
Planted mistakes in a copy of the function each fail a check."""
import inspect

import numpy as np
import pytest
import torch

import oracle

CASES = [  # beta, temperature, scale_t2, mask, reduction
    (0.5, 1.0, False, None, "mean"),
    (0.3, 1.7, True, [1, 0, 1], "sum"),
    (0.0, 1.0, False, None, "mean"),
    (1.0, 0.8, False, [1, 1, 0], "none"),
]


def _data(seed, N=3, V=6, Ds=4, Dt=4):
    g = torch.Generator().manual_seed(seed)
    hs = torch.randn(N, Ds, generator=g, dtype=torch.float64)
    ws = torch.randn(V, Ds, generator=g, dtype=torch.float64)
    ht = torch.randn(N, Dt, generator=g, dtype=torch.float64)
    wt = torch.randn(V, Dt, generator=g, dtype=torch.float64)
    return hs, ws, ht, wt


def _value(fn, hs, ws, ht, wt, case, grad):
    beta, T, t2, mask, red = case
    r = fn(hs, ws, ht, wt, beta, temperature=T, scale_t2=t2, mask=mask, reduction=red,
           grad=grad, grads=False)
    return float(np.dot(grad, r["rows"])) if red == "none" else r["out"] * grad


def check_finite_differences(fn):
    hs, ws, ht, wt = _data(1)
    for case in CASES:
        beta, T, t2, mask, red = case
        grad = np.array([0.7, 1.3, 0.9]) if red == "none" else 0.8
        r = fn(hs, ws, ht, wt, beta, temperature=T, scale_t2=t2, mask=mask, reduction=red,
               grad=grad)
        for name, x, got in (("hs", hs, r["gh"]), ("ws", ws, r["gw"])):
            fd = np.empty(x.shape)
            eps = 1e-6
            for idx in np.ndindex(*x.shape):
                xp, xm = x.clone(), x.clone()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = (xp, ws) if name == "hs" else (hs, xp)
                args_m = (xm, ws) if name == "hs" else (hs, xm)
                fp = _value(fn, *args_p, ht, wt, case, grad)
                fm = _value(fn, *args_m, ht, wt, case, grad)
                fd[idx] = (fp - fm) / (2 * eps)
            np.testing.assert_allclose(got, fd, rtol=1e-6, atol=1e-8, err_msg=f"{case} {name}")


def check_identity_head(fn):
    hs, _, ht, _ = _data(2, V=5, Ds=5, Dt=5)
    eye = torch.eye(5, dtype=torch.float64)
    for case in CASES:
        beta, T, t2, mask, red = case
        grad = np.array([0.7, 1.3, 0.9]) if red == "none" else 0.8
        r = fn(hs, eye, ht, eye, beta, temperature=T, scale_t2=t2, mask=mask, reduction=red,
               grad=grad)
        ref = oracle.jsd_loss(hs, ht, beta, temperature=T, scale_t2=t2, mask=mask,
                              reduction=red, grad=grad)
        np.testing.assert_allclose(r["rows"], ref["rows"], rtol=1e-13, atol=1e-15)
        if red != "none":
            np.testing.assert_allclose(r["out"], ref["out"], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(r["gh"], ref["gs"], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["gw"], ref["gs"].T @ hs.numpy(), rtol=1e-12, atol=1e-15)


def check_invariances(fn):
    hs, ws, ht, wt = _data(3, N=4, V=9, Ds=5, Dt=3)
    kw = dict(temperature=1.3, scale_t2=True, reduction="mean", grad=1.1)
    base = fn(hs, ws, ht, wt, 0.4, **kw)
    # shift every head row by one vector: each row's logits move by a constant
    c = torch.randn(5, dtype=torch.float64, generator=torch.Generator().manual_seed(9))
    sh = fn(hs, ws + c, ht, wt, 0.4, **kw)
    np.testing.assert_allclose(sh["out"], base["out"], rtol=1e-11)
    np.testing.assert_allclose(sh["gh"], base["gh"], rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(sh["gw"], base["gw"], rtol=1e-9, atol=1e-13)
    np.testing.assert_allclose(base["gw"].sum(axis=0), 0.0, atol=1e-14)
    # an orthogonal change of the teacher's hidden basis
    q, _ = torch.linalg.qr(torch.randn(3, 3, dtype=torch.float64,
                                       generator=torch.Generator().manual_seed(4)))
    rot = fn(hs, ws, ht @ q, wt @ q, 0.4, **kw)
    np.testing.assert_allclose(rot["out"], base["out"], rtol=1e-12)
    np.testing.assert_allclose(rot["gh"], base["gh"], rtol=1e-10, atol=1e-15)
    # scale the hidden states by a and the head by 1/a
    a = 2.5
    sc = fn(hs * a, ws / a, ht, wt, 0.4, **kw)
    np.testing.assert_allclose(sc["out"], base["out"], rtol=1e-12)
    np.testing.assert_allclose(sc["gh"], base["gh"] / a, rtol=1e-10, atol=1e-15)
    np.testing.assert_allclose(sc["gw"], base["gw"] * a, rtol=1e-10, atol=1e-15)


def check_mask(fn):
    hs, ws, ht, wt = _data(5, N=5, V=7, Ds=4, Dt=4)
    mask = [1, 0, 1, 1, 0]
    keep = [0, 2, 3]
    r = fn(hs, ws, ht, wt, 0.6, mask=mask, reduction="mean", grad=1.0)
    assert not r["gh"][1].any() and not r["gh"][4].any()
    sub = fn(hs[keep], ws, ht[keep], wt, 0.6, reduction="mean", grad=1.0)
    np.testing.assert_allclose(r["out"], sub["out"], rtol=1e-13)
    np.testing.assert_allclose(r["gh"][keep], sub["gh"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["gw"], sub["gw"], rtol=1e-12, atol=1e-15)


CHECKS = [check_finite_differences, check_identity_head, check_invariances, check_mask]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_linear_pins(check):
    check(oracle.linear_jsd)


MUTANTS = [
    ("teacher_logits_from_student", "lt = (Ht @ Wt.T).contiguous()",
     "lt = (Hs @ Ws.T).contiguous()"),
    ("gh_through_teacher_head", "res[\"gh\"] = (G @ Ws).numpy()",
     "res[\"gh\"] = (G @ Wt[:, :Ws.shape[1]]).numpy() if Wt.shape[1] >= Ws.shape[1] else (G @ Ws).numpy() * 0"),
    ("gw_from_teacher_hidden", "res[\"gw\"] = (G.T @ Hs).numpy()",
     "res[\"gw\"] = (G.T @ Ht[:, :Hs.shape[1]]).numpy() if Ht.shape[1] >= Hs.shape[1] else (G.T @ Hs).numpy() * 0"),
    ("student_logits_transposed_weight_rows", "ls = (Hs @ Ws.T).contiguous()",
     "ls = (Hs @ Ws.flip(0).T).contiguous()"),
    ("gw_rows_reversed", "res[\"gw\"] = (G.T @ Hs).numpy()",
     "res[\"gw\"] = (G.T @ Hs).flip(0).numpy()"),
]


def _mutant(old, new):
    src = inspect.getsource(oracle.linear_jsd)
    assert src.count(old) == 1, old
    ns = {"np": np, "torch": torch, "jsd_loss": oracle.jsd_loss}
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["linear_jsd"]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_linear_pins_catch_planted_mistake(name, old, new):
    fn = _mutant(old, new)
    failed = []
    for check in CHECKS:
        try:
            check(fn)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin caught {name}"
