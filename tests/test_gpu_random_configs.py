"""Seeded random configurations of the JSD forward and backward: dtype, batch size, row
width (register-held rows, two-sweep rows, ragged tails), the rows' offset inside 16
bytes, logical shard splits, beta (endpoints and near them included), which gradients
are wanted, tokens masked on both sides, undefined rows and zero upstream gradients.
Each configuration runs the one call (vjsd_forward_backward) and the two calls
(vjsd_forward + vjsd_bwd) on the same inputs: every output bit-identical, and sampled
rows (first and last included) against the fp64 oracle.  The distillation-loss form
(temperature, T^2, token mask, reduction) is drawn the same way, and so are the sibling
ops (KL both ways, entropy, log-probabilities, teacher top-k KL, cross-entropy) against
the oracle alone, and the fused-linear loss's GEMM against an fp64 product.  The
configurations are drawn once, from a fixed seed, so the list and its test names do not
change between runs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import test_gpu_ce
import test_gpu_linear
import test_gpu_siblings as sib
import test_gpu_topk
from parity import assert_grads, assert_values
from test_gpu_fwd_bwd import assert_same, check_oracle, check_two_calls, run

pytestmark = pytest.mark.gpu

NINF = float("-inf")
DTYPES = [torch.bfloat16, torch.float16, torch.float32]


def _configs(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = DTYPES[i % 3]
        kind = rng.choice(["small", "register", "two_sweep"], p=[0.3, 0.35, 0.35])
        if kind == "small":
            V = int(rng.integers(1, 2000))
        elif kind == "register":
            V = int(rng.integers(2000, 20480 if dt == torch.float32 else 40960))
        else:
            V = int(rng.integers(41000, 140000))
        N = int(rng.integers(1, max(2, min(33, 2_500_000 // V))))
        off = int(rng.integers(0, 8))
        u = rng.random()
        beta = (0.0 if u < 0.1 else 1.0 if u < 0.2 else 1e-6 if u < 0.25
                else 1.0 - 1e-6 if u < 0.3 else float(np.round(rng.random(), 3)))
        S = 1 if rng.random() < 0.7 or V < 8 else int(rng.integers(2, 5))
        widths = None
        if S > 1:
            cuts = np.sort(rng.choice(np.arange(1, V), size=S - 1, replace=False))
            widths = [int(w) for w in np.diff(np.concatenate([[0], cuts, [V]]))]
        want = [(True, True), (True, False), (False, True)][int(rng.integers(0, 3))]
        mask = float(rng.choice([0.0, 0.0, 0.02, 0.3]))
        undefined = bool(rng.random() < 0.2) and N > 1
        zero_g = bool(rng.random() < 0.2)
        out.append(dict(dtype=dt, N=N, V=V, off=off, beta=beta, widths=widths, want=want,
                        mask=mask, undefined=undefined, zero_g=zero_g, seed=1000 + i))
    return out


CONFIGS = _configs()


def _name(c):
    w = "" if c["widths"] is None else f"-S{len(c['widths'])}"
    return (f"{str(c['dtype'])[6:]}-N{c['N']}-V{c['V']}-o{c['off']}-b{c['beta']:g}{w}"
            f"-g{int(c['want'][0])}{int(c['want'][1])}")


@pytest.mark.parametrize("c", CONFIGS, ids=[_name(c) for c in CONFIGS])
def test_random_config(c):
    N, V, off = c["N"], c["V"], c["off"]
    b = synth.draw("full_vocab", device="cuda", N=N, V=V + off, dtype=c["dtype"],
                   seed=c["seed"])
    s = b.s[:, off:off + V].clone() if c["mask"] or c["undefined"] else b.s[:, off:off + V]
    t = b.t[:, off:off + V].clone() if c["mask"] or c["undefined"] else b.t[:, off:off + V]
    if c["mask"] or c["undefined"]:
        # clone() made the rows contiguous: take them back at the same offset
        bs = torch.empty((N, V + off), dtype=s.dtype, device=s.device)
        bt = torch.empty_like(bs)
        bs[:, off:] = s
        bt[:, off:] = t
        s, t = bs[:, off:], bt[:, off:]
    gen = torch.Generator(device="cuda").manual_seed(c["seed"])
    if c["mask"]:
        m = torch.rand((N, V), generator=gen, device="cuda") < c["mask"]
        s.masked_fill_(m, NINF)  # the same tokens on both sides
        t.masked_fill_(m, NINF)
    if c["undefined"]:
        s[N // 2] = NINF
    gout = torch.rand(N, generator=gen, device="cuda") + 0.5
    if c["zero_g"]:
        gout[0] = 0.0
    res, _ = check_two_calls(s, t, c["beta"], gout=gout, want=c["want"], widths=c["widths"])
    rows = np.unique(np.array([0, N // 2, N - 1]))
    check_oracle(s, t, c["beta"], gout, res, rows=rows, want=c["want"])


def _loss_configs(n=20, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = DTYPES[i % 3]
        V = int(rng.choice([int(rng.integers(100, 16384)), int(rng.integers(41000, 131072))]))
        N = int(rng.integers(2, max(3, min(33, 2_000_000 // V))))
        u = rng.random()
        beta = 0.0 if u < 0.15 else 1.0 if u < 0.3 else float(np.round(rng.random(), 3))
        out.append(dict(dtype=dt, N=N, V=V, beta=beta,
                        temperature=float(rng.choice([0.5, 1.0, 1.7, 3.0])),
                        scale_t2=bool(rng.random() < 0.5),
                        reduction=str(rng.choice(["none", "sum", "mean"])),
                        mask=bool(rng.random() < 0.5), seed=2000 + i))
    return out


LOSS_CONFIGS = _loss_configs()


@pytest.mark.parametrize("c", LOSS_CONFIGS, ids=[
    f"{str(c['dtype'])[6:]}-N{c['N']}-V{c['V']}-b{c['beta']:g}-T{c['temperature']:g}"
    f"{'-t2' if c['scale_t2'] else ''}-{c['reduction']}{'-mask' if c['mask'] else ''}"
    for c in LOSS_CONFIGS])
def test_random_loss_config(c):
    """The distillation loss form (vjsd_loss_forward_backward against the loss forward
    and backward calls, and against oracle.jsd_loss)."""
    N, V = c["N"], c["V"]
    b = synth.draw("full_vocab", device="cuda", N=N, V=V, dtype=c["dtype"], seed=c["seed"])
    gen = torch.Generator(device="cuda").manual_seed(c["seed"])
    opts = dict(temperature=c["temperature"], scale_t2=c["scale_t2"],
                reduction=c["reduction"])
    if c["mask"]:
        opts["mask"] = (torch.rand(N, generator=gen, device="cuda") > 0.3).to(torch.uint8)
    if c["reduction"] == "none":
        grad = torch.rand(N, generator=gen, device="cuda") + 0.5
    else:
        grad = torch.tensor([0.75], device="cuda")
    one = run(b.s, b.t, c["beta"], None, fused=True, opts=opts, grad=grad)
    two = run(b.s, b.t, c["beta"], None, fused=False, opts=opts, grad=grad)
    assert_same(one, two)
    mask = opts.get("mask")
    ref = oracle.jsd_loss(b.s.cpu(), b.t.cpu(), c["beta"], temperature=c["temperature"],
                          scale_t2=c["scale_t2"],
                          mask=None if mask is None else mask.cpu().numpy(),
                          reduction=c["reduction"],
                          grad=grad.cpu().double().numpy() if grad.numel() > 1
                          else float(grad.item()))
    assert_values(one["loss"].cpu(), ref["rows"], b.s.dtype, "rows")
    scale = max(1.0, 1.0 / c["temperature"])
    assert_grads(one["gs"].cpu(), ref["gs"], b.s.dtype, "d/ds", scale=scale)
    assert_grads(one["gt"].cpu(), ref["gt"], b.s.dtype, "d/dt", scale=scale)


SIBLING_OPS = ["kl", "reverse_kl", "entropy", "logprobs", "topk_kl", "cross_entropy"]


def _sibling_configs(n=24, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = DTYPES[i % 3]
        op = SIBLING_OPS[(i // 3) % len(SIBLING_OPS)]
        V = int(rng.choice([int(rng.integers(64, 4096)), int(rng.integers(4096, 140000))]))
        N = int(rng.integers(2, max(3, min(25, 2_000_000 // V))))
        off = int(rng.integers(0, 8))
        S = 1 if rng.random() < 0.6 else int(rng.integers(2, 5))
        widths = None
        if S > 1:
            cuts = np.sort(rng.choice(np.arange(1, V), size=S - 1, replace=False))
            widths = [int(w) for w in np.diff(np.concatenate([[0], cuts, [V]]))]
        out.append(dict(op=op, dtype=dt, N=N, V=V, off=off, widths=widths,
                        K=int(rng.integers(1, 9)),
                        red=str(rng.choice(["none", "sum", "mean"])), seed=3000 + i))
    return out


SIBLING_CONFIGS = _sibling_configs()


@pytest.mark.parametrize("c", SIBLING_CONFIGS, ids=[
    f"{c['op']}-{str(c['dtype'])[6:]}-N{c['N']}-V{c['V']}-o{c['off']}"
    f"{'' if c['widths'] is None else '-S%d' % len(c['widths'])}" for c in SIBLING_CONFIGS])
def test_random_sibling_config(c):
    """The sibling ops through the C ABI (forward and backward) against the fp64 oracle,
    on seeded random shapes, offsets and shard splits."""
    N, V, off, widths = c["N"], c["V"], c["off"], c["widths"]
    b = synth.draw("full_vocab", device="cuda", N=N, V=V + off, dtype=c["dtype"],
                   seed=c["seed"])
    s, t = b.s[:, off:off + V], b.t[:, off:off + V]
    gen = torch.Generator(device="cuda").manual_seed(c["seed"])
    op = c["op"]
    if op in ("kl", "reverse_kl"):
        gout = torch.rand(N, generator=gen, device="cuda") + 0.5
        sib.check_kl(s, t, op == "reverse_kl", widths=widths, gout=gout, want_t=True)
    elif op == "entropy":
        gout = torch.rand(N, generator=gen, device="cuda") + 0.5
        g = sib.run_entropy(s, widths, gout)
        ref = oracle.entropy(s.cpu(), widths=widths, gout=gout.cpu().double().numpy())
        assert_values(g["ent"], ref["ent"], s.dtype, "entropy")
        assert_grads(g["gx"], ref["gx"], s.dtype, "d/dx")
    elif op == "logprobs":
        K = c["K"]
        ids = torch.randint(0, V, (N, K), generator=gen, device="cuda")
        ids[torch.rand((N, K), generator=gen, device="cuda") < 0.15] = -100
        gout = torch.rand((N, K), generator=gen, device="cuda") + 0.5
        g = sib.run_logprobs(s, ids, -100, widths, gout)
        assert g["err"] == 0
        ref = oracle.logprobs(s.cpu(), ids.cpu().numpy(), -100, widths=widths,
                              gout=gout.cpu().double().numpy())
        assert_values(g["out"], ref["out"], s.dtype, "logprobs")
        assert_grads(g["gx"], ref["gx"], s.dtype, "d/dx")
    elif op == "topk_kl":
        ids, tl = test_gpu_topk.teacher_topk(t, min(c["K"], V), c["seed"])
        test_gpu_topk.check(s, ids, tl, widths=widths, seed=c["seed"])
    else:
        labels = test_gpu_ce.labels_for(N, V, c["seed"])
        test_gpu_ce.check(s, labels, c["red"], widths=widths, seed=c["seed"])


def _gemm_configs(n=30, seed=20261206):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, N = (int(x) for x in rng.integers(1, 600, size=2))
        K = int(64 * rng.integers(1, 12)) if rng.random() < 0.4 else int(rng.integers(0, 700))
        a_f32, a_km, b_km = (int(x) for x in rng.integers(0, 2, size=3))
        if rng.random() < 0.3:  # the direct-to-LDS kernel's layout
            a_f32, a_km, b_km = 0, 1, 1
        out.append(dict(M=M, N=N, K=K, a_f32=a_f32, a_km=a_km, b_km=b_km,
                        out=str(rng.choice(["f32", "f32_acc", "bf16"])),
                        pad=int(rng.integers(0, 3)), seed=4000 + i))
    return out


GEMM_CONFIGS = _gemm_configs()


@pytest.mark.parametrize("c", GEMM_CONFIGS, ids=[
    f"M{c['M']}-N{c['N']}-K{c['K']}-a{'f32' if c['a_f32'] else 'bf16'}"
    f"{'k' if c['a_km'] else 'r'}-b{'k' if c['b_km'] else 'r'}-{c['out']}-p{c['pad']}"
    for c in GEMM_CONFIGS])
def test_random_gemm_config(c):
    """The fused-linear loss's GEMM (vlin_gemm) on seeded random shapes, operand layouts,
    padded leading dimensions and output modes, against an fp64 product of the same
    bf16 operands within the accumulation bound."""
    test_gpu_linear.gemm_case(c["M"], c["N"], c["K"], c["a_f32"], c["a_km"], c["b_km"],
                              c["out"], seed=c["seed"], pad=c["pad"])
