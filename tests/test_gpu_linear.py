"""GPU parity of the fused-linear path: the matrix-core GEMM (vlin_gemm) in every
operand layout and output mode against an fp64 product of the same bf16 operands, and
the fused-linear loss (vljsd, linear_jsd) against oracle.linear_jsd.

Tolerances follow from the arithmetic.  A product of two bf16 values is exact in
fp32; the MFMA sums K of them in fp32, so |C - C_exact| <= (K + 2) u sum_k |a_k b_k|
with u = 2^-24.  A bf16 result adds its rounding, |x| 2^-8.  The loss sees logits
with that error (here at most about 1e-6 relative) on top of the fp32 divergence
tolerance of 1e-5 relative + 1e-6 absolute, so the loss is held to 1e-4 relative +
1e-5 absolute.  The gradients come from the logit gradient G rounded to bf16 (error
<= 2^-8 |G|) times bf16 operands, summed in fp32, then rounded to bf16; with G itself
within 1e-4 of the oracle's (the fp32 divergence-gradient tolerance), each element is
held to (2^-8 + 1e-4 + (K + 2) u) sum |G| |operand| + 2^-8 |ref| + 1e-7.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def vj():
    import vocab_sharded_softmax_amd as v
    return v


def bf16_exact(x: torch.Tensor) -> np.ndarray:
    """The values an operand contributes: bf16 as stored, fp32 rounded to bf16."""
    return x.to(torch.bfloat16).double().cpu().numpy()


def gemm_case(M, N, K, a_f32, a_km, b_km, out, seed, pad=0, acc_init=None):
    v = vj()
    g = torch.Generator(device="cuda").manual_seed(seed)
    adt = torch.float32 if a_f32 else torch.bfloat16
    a_shape = (M, K) if a_km else (K, M)
    b_shape = (N, K) if b_km else (K, N)
    qa = 4 if a_f32 else 8
    # leading dimensions padded to the required multiple, plus `pad` extra columns
    lda = -(-a_shape[1] // qa) * qa + pad * qa
    ldb = -(-b_shape[1] // 8) * 8 + pad * 8
    abuf = torch.randn((a_shape[0], max(lda, 1)), generator=g, device="cuda").to(adt)
    bbuf = torch.randn((b_shape[0], max(ldb, 1)), generator=g, device="cuda").to(torch.bfloat16)
    a = abuf[:, :a_shape[1]]
    b = bbuf[:, :b_shape[1]]
    A = bf16_exact(a) if a_km else bf16_exact(a).T
    B = bf16_exact(b) if b_km else bf16_exact(b).T
    ref = A @ B.T
    mag = np.abs(A) @ np.abs(B).T
    cdt = torch.bfloat16 if out == "bf16" else torch.float32
    ldc = N + 3
    cbuf = torch.full((M, ldc), float("nan"), device="cuda", dtype=cdt)
    if out == "f32_acc":
        init = torch.randn((M, N), generator=g, device="cuda")
        cbuf[:, :N] = init
        ref = ref + init.double().cpu().numpy()
        mag = mag + np.abs(init.double().cpu().numpy())
    v.vlin_gemm(M, N, K, v.lin_operand(a if a_km else a, a_km, "a"),
                v.lin_operand(b, b_km, "b"), cbuf, out)
    torch.cuda.synchronize()
    got = cbuf[:, :N].double().cpu().numpy()
    tol = (K + 2) * U * mag
    if out == "bf16":
        tol = tol * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    assert np.all(err <= tol + 1e-30), (
        f"M={M} N={N} K={K} a_f32={a_f32} a_km={a_km} b_km={b_km} out={out}: "
        f"max err/tol {np.max(err / (tol + 1e-30)):.3g}")
    # the padding columns of C are never written
    assert torch.isnan(cbuf[:, N:].float()).all()


LAYOUTS = [(af, akm, bkm) for af in (0, 1) for akm in (1, 0) for bkm in (1, 0)]


@pytest.mark.parametrize("a_f32,a_km,b_km", LAYOUTS)
@pytest.mark.parametrize("out", ["f32", "f32_acc", "bf16"])
def test_gemm_layouts_ragged(a_f32, a_km, b_km, out):
    # several tiles in every direction, ragged in M, N and K (K not a multiple of 8)
    gemm_case(300, 200, 139, a_f32, a_km, b_km, out, seed=11 + a_f32 + 2 * a_km + 4 * b_km,
              pad=1)


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (128, 128, 64), (129, 127, 65), (5, 300, 1024),
                                   (257, 3, 8), (64, 64, 0)])
def test_gemm_edge_shapes(M, N, K):
    for a_f32, a_km, b_km in ((0, 1, 1), (1, 1, 0), (1, 0, 0)):
        gemm_case(M, N, K, a_f32, a_km, b_km, "f32", seed=M + N + K)
    gemm_case(M, N, K, 0, 1, 1, "bf16", seed=5)


@pytest.mark.parametrize("M,N,K", [(300, 200, 128), (257, 513, 192), (1, 1, 64), (129, 300, 3584),
                                   (256, 256, 64)])
@pytest.mark.parametrize("out", ["f32", "f32_acc", "bf16"])
def test_gemm_direct_to_lds_path(M, N, K, out):
    # both operands bf16 and k-major with K a multiple of 64: the kernel whose global
    # loads go straight into LDS (two stages of k = 64); ragged M and N
    gemm_case(M, N, K, 0, 1, 1, out, seed=M * 7 + N + K, pad=1)


def test_gemm_long_reduction():
    # the gradient-of-hidden shape: a long reduction over a vocabulary-sized K
    gemm_case(96, 136, 20000, 1, 1, 0, "bf16", seed=3)


def _lin_ref(b, beta, T, t2, mask, red):
    return oracle.linear_jsd(b.hs.cpu(), b.ws.cpu(), b.ht.cpu(), b.wt.cpu(), beta, temperature=T,
                             scale_t2=t2, mask=None if mask is None else mask.cpu().numpy(),
                             reduction=red, grad=1.0, grads=red != "none")


def _grad_tol(G, other, ref):
    mag = np.abs(G) @ np.abs(other)
    K = G.shape[1]
    return (2.0 ** -8 + 1e-4 + (K + 2) * U) * mag + 2.0 ** -8 * np.abs(ref) + 1e-7


def _check_linear(b, beta, T=1.0, t2=False, mask=None, red="mean", chunk=4096, group=0):
    v = vj()
    N, V = b.hs.shape[0], b.ws.shape[0]
    st = v.lin_head(b.hs, b.ws, "student")
    te = v.lin_head(b.ht, b.wt, "teacher")
    opts = v.loss_opts(N, T, t2, mask, red)
    ws = torch.empty(max(1, v.vljsd_workspace_bytes(N, V, b.hs.shape[1], chunk, group)),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((N if red == "none" else 1,), float("nan"), device="cuda")
    gh = gw = None
    if red != "none":
        gh = torch.full_like(b.hs, float("nan"))
        gw = torch.full_like(b.ws, float("nan"))
    v.vljsd(st, te, N, V, beta, opts, chunk, ws, out, gh, gw, group=group)
    torch.cuda.synchronize()
    ref = _lin_ref(b, beta, T, t2, mask, red)
    want = ref["rows"] if red == "none" else np.array([ref["out"]])
    got = out.double().cpu().numpy()
    np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-5,
                               err_msg=f"loss beta={beta} T={T} red={red} chunk={chunk}")
    if red == "none":
        return
    G = ref["G"]  # the oracle's logit gradient, for the bound
    ghg = gh.double().cpu().numpy()
    gwg = gw.double().cpu().numpy()
    tol_h = _grad_tol(G, b.ws.double().cpu().numpy(), ref["gh"])
    tol_w = _grad_tol(G.T, b.hs.double().cpu().numpy(), ref["gw"])
    eh = np.abs(ghg - ref["gh"])
    ew = np.abs(gwg - ref["gw"])
    assert np.all(eh <= tol_h), f"grad_h: max err/tol {np.max(eh / tol_h):.3g}"
    assert np.all(ew <= tol_w), f"grad_w: max err/tol {np.max(ew / tol_w):.3g}"
    if mask is not None:  # dropped tokens: exactly zero rows
        drop = (mask.cpu().numpy() == 0)
        assert not ghg[drop].any()


@pytest.mark.parametrize("chunk,group", [(10_000, 0), (128, 0), (100, 0), (64, 128), (100, 100),
                                         (128, 1), (3, 0), (7, 20)])
def test_linear_jsd_chunks_and_groups(chunk, group):
    # one block; several blocks in one group; three groups (the head gradient summed
    # in fp32 across them: the store, accumulate and final convert epilogues); chunks
    # below 8 tokens taken 8 at a time (each chunk's columns of the transposed logit
    # gradient start 8 tokens apart), in one group and in thirteen
    b = synth.draw_linear("cuda", N=300, V=1000, Ds=72, Dt=56, seed=7)
    _check_linear(b, 0.5, chunk=chunk, group=group)


@pytest.mark.parametrize("chunk,group", [(300, 0), (128, 128)])
def test_linear_jsd_vocabulary_multiple_of_64(chunk, group):
    # V a multiple of 64: the hidden-gradient product runs on the direct-to-LDS kernel
    # with its K (the vocabulary) split over work items and the fp32 partials summed
    b = synth.draw_linear("cuda", N=300, V=1024, Ds=64, Dt=48, seed=12)
    _check_linear(b, 0.5, T=1.5, t2=True, red="mean", chunk=chunk, group=group)


@pytest.mark.parametrize("beta", [0.0, 0.3, 1.0])
def test_linear_jsd_betas_temperature_mask(beta):
    b = synth.draw_linear("cuda", N=257, V=777, Ds=64, Dt=96, seed=8)
    g = torch.Generator(device="cuda").manual_seed(3)
    mask = (torch.rand(257, generator=g, device="cuda") > 0.2).to(torch.uint8)
    _check_linear(b, beta, T=2.0, t2=True, mask=mask, red="mean", chunk=128, group=128)
    _check_linear(b, beta, T=0.7, red="sum", chunk=1000)
    _check_linear(b, beta, red="none", chunk=64)


def test_linear_jsd_no_kept_token_and_empty():
    v = vj()
    b = synth.draw_linear("cuda", N=40, V=300, Ds=32, Dt=32, seed=9)
    mask = torch.zeros(40, dtype=torch.uint8, device="cuda")
    _check_linear(b, 0.5, mask=mask, red="mean", chunk=16)
    # no tokens: the sum is 0 and the head gradient exactly 0
    e = synth.draw_linear("cuda", N=0, V=300, Ds=32, Dt=32, seed=9)
    out = torch.full((1,), float("nan"), device="cuda")
    gw = torch.full_like(e.ws, float("nan"))
    v.vljsd(v.lin_head(e.hs, e.ws, "student"), v.lin_head(e.ht, e.wt, "teacher"), 0, 300, 0.5,
            v.loss_opts(0, 1.0, False, None, "sum"), 16, None, out, None, gw)
    torch.cuda.synchronize()
    assert out.item() == 0.0 and not gw.float().any()


def test_linear_jsd_autograd():
    v = vj()
    b = synth.draw_linear("cuda", N=3 * 70, V=500, Ds=48, Dt=40, seed=10)
    hs = b.hs.view(3, 70, 48).clone().requires_grad_()
    ws = b.ws.clone().requires_grad_()
    loss = v.linear_jsd(hs, ws, b.ht.view(3, 70, 40), b.wt, 0.4, temperature=1.5,
                        scale_t2=True, reduction="mean", chunk=64)
    (loss * 0.25).backward()
    ref = oracle.linear_jsd(b.hs.cpu(), b.ws.cpu(), b.ht.cpu(), b.wt.cpu(), 0.4,
                            temperature=1.5, scale_t2=True, reduction="mean", grad=0.25)
    np.testing.assert_allclose(loss.item(), ref["out"], rtol=1e-4, atol=1e-5)
    G = ref["G"]
    gh = hs.grad.reshape(-1, 48).double().cpu().numpy()
    gw = ws.grad.double().cpu().numpy()
    # one more rounding: the bf16 gradient scaled by 0.25 is exact (a power of two)
    assert np.all(np.abs(gh - ref["gh"]) <= _grad_tol(G, b.ws.double().cpu().numpy(), ref["gh"]))
    assert np.all(np.abs(gw - ref["gw"]) <= _grad_tol(G.T, b.hs.double().cpu().numpy(),
                                                       ref["gw"]))
    with pytest.raises(ValueError):
        v.linear_jsd(hs, ws, b.ht.view(3, 70, 40).clone().requires_grad_(), b.wt)
    with pytest.raises(ValueError):
        v.linear_jsd(hs, ws, b.ht.view(3, 70, 40), b.wt, reduction="none")


def test_linear_full_size_sampled():
    """The fused-linear workload at its full size (N=8192, V=151936, D=3584, chunk
    1024, as the benchmark runs it): per-token losses of sampled rows, and the
    hidden-state gradient rows of those tokens, against the oracle on those rows."""
    v = vj()
    b = synth.draw_linear("cuda")
    N, V, D = b.hs.shape[0], b.ws.shape[0], b.hs.shape[1]
    st = v.lin_head(b.hs, b.ws, "student")
    te = v.lin_head(b.ht, b.wt, "teacher")
    ws = torch.empty(v.vljsd_workspace_bytes(N, V, D, 1024, 0), dtype=torch.uint8, device="cuda")
    rows = torch.full((N,), float("nan"), device="cuda")
    v.vljsd(st, te, N, V, 0.5, v.loss_opts(N, 1.0, False, None, "none"), 1024, ws, rows)
    out = torch.full((1,), float("nan"), device="cuda")
    gh = torch.full_like(b.hs, float("nan"))
    v.vljsd(st, te, N, V, 0.5, v.loss_opts(N, 1.0, False, None, "sum"), 1024, ws, out, gh, None)
    torch.cuda.synchronize()
    del ws
    sample = np.array([0, 1, 1023, 1024, 4095, 4096, 5000, N - 1])
    hs_s, ht_s = b.hs[sample].cpu(), b.ht[sample].cpu()
    ref = oracle.linear_jsd(hs_s, b.ws.cpu(), ht_s, b.wt.cpu(), 0.5, reduction="sum", grad=1.0,
                            head_grad=False)
    np.testing.assert_allclose(rows[sample].double().cpu().numpy(), ref["rows"], rtol=1e-4,
                               atol=1e-5)
    np.testing.assert_allclose(out.item(), rows.double().sum().item(), rtol=1e-5)
    tol = _grad_tol(ref["G"], b.ws.cpu().double().numpy(), ref["gh"])
    err = np.abs(gh[sample].double().cpu().numpy() - ref["gh"])
    assert np.all(err <= tol), f"grad_h rows: max err/tol {np.max(err / tol):.3g}"
