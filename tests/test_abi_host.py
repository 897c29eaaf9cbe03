"""The C ABI on the host (CPU only): the library loads, exports every entry point
``include/vjsd.h`` declares, and rejects invalid arguments before anything is
enqueued.  No call here reaches a GPU: every call either fails validation or has
N == 0, which returns before any HIP call.
"""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vjsd.h")

abi = pytest.importorskip("vocab_sharded_softmax_amd._abi")
lib = abi.lib
Shard, View = abi.Shard, abi.View

OK, ARG, DTYPE, BETA, LAYOUT, EMPTY, SCRATCH = 0, -1, -2, -3, -4, -5, -7
FAKE = 0x10000  # a well-aligned address that is never dereferenced here


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"VJSD_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_every_declared_entry_point_is_exported():
    names = declared_functions()
    assert len(names) == 27
    for n in names:
        assert hasattr(lib, n), n
    # and nothing else of the library's own code is exported
    out = os.popen(f"nm -D --defined-only {abi.LIB_PATH}").read().split("\n")
    own = {ln.split()[-1] for ln in out if ln.strip() and (" T " in ln)}
    own = {n for n in own if n.startswith(("vjsd", "vkl", "ventropy", "vlogprobs", "vtopk", "vce",
                                            "vlin", "vljsd"))}
    assert own == set(names)


def test_strerror_and_workspace():
    for code in (0, -1, -2, -3, -4, -5, -6, 7):
        assert isinstance(lib.vjsd_strerror(code), bytes)
    assert lib.vjsd_workspace_bytes(0, 4) == 0
    # per-row constants (16 floats) + per (shard, row) partials (8 floats) + a 64-byte
    # scalar tail (the kept-row count of a masked mean)
    assert lib.vjsd_workspace_bytes(8192, 1) == 8192 * (16 + 8) * 4 + 64
    assert lib.vjsd_workspace_bytes(4096, 4) == 4096 * (16 + 4 * 8) * 4 + 64
    for N, S in ((1, 1), (64, 3), (8192, 1), (16384, 7)):  # the binding sizes it the same way
        assert abi.part_floats(N, S) * 4 == lib.vjsd_workspace_bytes(N, S)


def shards(widths, ptr=FAKE, rs=None, start=0, es=2, grads=False):
    arr = (Shard * len(widths))()
    c = start
    V = sum(widths)
    for k, w in enumerate(widths):
        p = ptr + c * es if ptr else None
        v = View(p, V if rs is None else rs, 0, 0)
        g = View(p + (1 << 30) if (grads and p) else None, V if rs is None else rs, 0, 0)
        arr[k] = Shard(c, w, v, v, g, g)
        c += w
    return arr


def fwd(arr, S, N, dt=2, beta=0.5, stats=FAKE, part=FAKE, kl=FAKE, loss=FAKE):
    return lib.vjsd_fwd(arr, S, N, dt, stats, beta, part, kl, loss, None)


def test_empty_batch_is_valid_and_enqueues_nothing():
    a = shards([5, 0, 7])
    assert lib.vjsd_forward(a, 3, 0, 2, 0.5, None, None, None, None, None) == OK
    assert lib.vjsd_stats(a, 3, 0, 2, 3, None, None) == OK
    assert lib.vjsd_merge(None, 3, 0, 3, None, None) == OK
    assert fwd(a, 3, 0, stats=None, part=None, kl=None, loss=None) == OK
    assert lib.vjsd_bwd(a, 3, 0, 2, None, None, 0.5, None, None, None) == OK
    assert lib.vkl_fwd(a, 3, 0, 2, 0, None, None, None, None, None) == OK
    assert lib.ventropy_fwd(a, 3, 0, 2, None, None, None, None) == OK
    b = shards([5, 7])
    assert lib.vlogprobs_fwd(b, 2, 0, 2, 12, None, 4, -100, None, None, None, None, None) == OK


@pytest.mark.parametrize("beta", [-0.1, 1.0000001, math.nan, math.inf, -math.inf])
def test_beta_outside_unit_interval_is_rejected(beta):
    a = shards([10])
    assert fwd(a, 1, 4, beta=beta) == BETA
    assert lib.vjsd_forward(a, 1, 4, 2, beta, FAKE, FAKE, FAKE, FAKE, None) == BETA
    assert lib.vjsd_bwd(a, 1, 4, 2, FAKE, FAKE, beta, FAKE, FAKE, None) == BETA


def test_dtype_and_sizes_are_checked():
    a = shards([10])
    assert fwd(a, 1, 4, dt=3) == DTYPE
    assert fwd(a, 1, 4, dt=-1) == DTYPE
    assert fwd(a, 1, -1) == ARG
    assert fwd(a, 0, 4) == ARG
    assert fwd(None, 1, 4) == ARG
    assert fwd(a, 1, 1 << 31) == ARG
    assert lib.vjsd_stats(a, 1, 4, 2, 0, FAKE, None) == ARG
    assert lib.vjsd_stats(a, 1, 4, 2, 4, FAKE, None) == ARG
    assert lib.vjsd_merge(FAKE, 1, 4, 5, FAKE, None) == ARG


def test_null_buffers_are_rejected():
    a = shards([10])
    assert fwd(a, 1, 4, stats=None) == ARG
    assert lib.vjsd_forward(a, 1, 4, 2, 0.5, None, FAKE, FAKE, FAKE, None) == ARG
    assert fwd(a, 1, 4, kl=None) == ARG
    assert fwd(a, 1, 4, loss=None) == ARG
    assert lib.vjsd_stats(a, 1, 4, 2, 3, None, None) == ARG
    a2 = shards([5, 5])
    assert fwd(a2, 2, 4, part=None) == ARG  # several shards need the workspace
    assert lib.vjsd_bwd(a, 1, 4, 2, FAKE, FAKE, 0.5, None, FAKE, None) == ARG
    assert lib.vjsd_bwd(a, 1, 4, 2, FAKE, FAKE, 0.5, FAKE, None, None) == ARG  # no workspace
    assert lib.vjsd_merge(None, 1, 4, 3, FAKE, None) == ARG


def test_views_are_checked():
    assert fwd(shards([10], ptr=None), 1, 4) == ARG  # null logits with width > 0
    assert fwd(shards([10], ptr=FAKE + 1), 1, 4) == ARG  # not element-aligned
    assert fwd(shards([10], rs=9), 1, 4) == ARG  # overlapping rows
    assert fwd(shards([10], rs=-10), 1, 4) == ARG
    a = shards([10])
    a[0].s.rows_per_batch = 3
    a[0].s.batch_stride = 25  # batches overlap: needs >= 2 * 10 + 10
    assert fwd(a, 1, 6) == ARG
    # an empty shard may carry a null pointer
    b = shards([4, 0, 6])
    b[1].s.p = None
    b[1].t.p = None
    assert fwd(b, 3, 0) == OK


def test_shards_must_be_ordered_and_contiguous():
    a = shards([4, 6])
    a[1].vocab_start = 5
    assert fwd(a, 2, 4) == LAYOUT
    a[1].vocab_start = 3
    assert fwd(a, 2, 4) == LAYOUT
    a = shards([4, 6])
    a[0].width = -1
    assert fwd(a, 2, 4) == ARG


def test_logprobs_rejects_empty_shards_and_bad_vocabulary():
    a = shards([5, 0, 7])
    assert lib.vlogprobs_fwd(a, 3, 4, 2, 12, FAKE, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == EMPTY
    assert lib.vlogprobs_bwd(a, 3, 4, 2, 12, FAKE, FAKE, 3, -100, FAKE, FAKE, None) == EMPTY
    b = shards([5, 7])
    assert lib.vlogprobs_fwd(b, 2, 4, 2, 13, FAKE, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == LAYOUT
    c = shards([5, 7], start=1)
    assert lib.vlogprobs_fwd(c, 2, 4, 2, 13, FAKE, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == LAYOUT
    assert lib.vlogprobs_fwd(b, 2, 4, 2, 12, None, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == ARG
    assert lib.vlogprobs_fwd(b, 2, 4, 2, 12, FAKE, -1, -100, FAKE, FAKE, FAKE, FAKE, None) == ARG
    assert lib.vlogprobs_fwd(b, 2, 4, 2, 12, FAKE, 3, -100, FAKE, FAKE, FAKE, None, None) == ARG


def test_entropy_and_kl_check_their_arguments():
    a = shards([10])
    assert lib.ventropy_fwd(a, 1, 4, 7, FAKE, FAKE, FAKE, None) == DTYPE
    assert lib.ventropy_fwd(a, 1, 4, 2, None, FAKE, FAKE, None) == ARG
    assert lib.ventropy_bwd(a, 1, 4, 2, FAKE, FAKE, None, FAKE, None) == ARG
    assert lib.ventropy_bwd(a, 1, 4, 2, FAKE, FAKE, FAKE, None, None) == ARG
    assert lib.vkl_fwd(a, 1, 4, 2, 1, FAKE, FAKE, None, FAKE, None) == ARG
    assert lib.vkl_bwd(a, 1, 4, 2, 1, FAKE, FAKE, None, FAKE, None) == ARG


def _opts(T=1.0, t2=0, mask=None, red=0):
    return ctypes.byref(abi.LossOpts(T, t2, mask, red))


def test_loss_entry_points_check_their_options():
    a = shards([10])
    fwd_ = lambda o, out=FAKE, N=4: lib.vjsd_loss_forward(a, 1, N, 2, 0.5, o, FAKE, FAKE, FAKE, FAKE,
                                                          out, None)
    bwd_ = lambda o: lib.vjsd_loss_backward(a, 1, 4, 2, 0.5, o, FAKE, FAKE, FAKE, FAKE, None)
    for T in (0.0, -1.0, float("nan"), float("inf")):
        assert fwd_(_opts(T=T)) == ARG
        assert bwd_(_opts(T=T)) == ARG
    for red in (-1, 3):
        assert fwd_(_opts(red=red)) == ARG
        assert bwd_(_opts(red=red)) == ARG
    assert fwd_(_opts(red=2), out=None) == ARG  # a reduction needs out
    assert fwd_(None, N=0) == OK  # no reduction, no rows: nothing to do
    assert lib.vjsd_loss_forward(a, 1, 4, 2, 1.5, None, FAKE, FAKE, FAKE, FAKE, None, None) == BETA
    assert lib.vjsd_loss_forward(a, 1, 4, 2, 0.5, None, None, FAKE, FAKE, FAKE, None, None) == ARG
    assert lib.vjsd_loss_backward(a, 1, 4, 2, 0.5, None, FAKE, FAKE, None, FAKE, None) == ARG


def test_topk_kl_checks_its_arguments():
    a = shards([5, 7])
    f = lambda *x: lib.vtopk_kl_fwd(a, 2, 4, 2, 12, *x, None)
    assert f(FAKE, None, 3, -100, FAKE, FAKE, FAKE, FAKE) == ARG  # no teacher log-probs
    assert f(FAKE, FAKE, 3, -100, FAKE, FAKE, None, FAKE) == ARG  # no kl
    assert f(FAKE, FAKE, 3, -100, FAKE, FAKE, FAKE, None) == ARG  # no error flag
    assert lib.vtopk_kl_fwd(a, 2, 4, 7, 12, FAKE, FAKE, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == DTYPE
    assert lib.vtopk_kl_fwd(a, 2, 4, 2, 13, FAKE, FAKE, 3, -100, FAKE, FAKE, FAKE, FAKE, None) == LAYOUT
    assert lib.vtopk_kl_fwd(shards([5, 0, 7]), 3, 4, 2, 12, FAKE, FAKE, 3, -100, FAKE, FAKE, FAKE,
                            FAKE, None) == EMPTY
    b = lambda *x: lib.vtopk_kl_bwd(a, 2, 4, 2, 12, *x, None)
    assert b(FAKE, FAKE, None, 3, -100, FAKE, FAKE) == ARG
    assert b(FAKE, FAKE, FAKE, 3, -100, None, FAKE) == ARG
    assert lib.vtopk_kl_fwd(a, 2, 0, 2, 12, None, None, 3, -100, None, None, None, None, None) == OK


def test_cross_entropy_checks_its_arguments():
    a = shards([5, 7])
    f = lambda red, *x: lib.vce_fwd(a, 2, 4, 2, 12, FAKE, -100, red, *x, None)
    assert f(3, FAKE, FAKE, FAKE, FAKE, FAKE) == ARG  # bad reduction
    assert f(2, FAKE, FAKE, FAKE, None, FAKE) == ARG  # a reduction needs out
    assert f(0, FAKE, FAKE, None, None, FAKE) == ARG  # no rows
    assert f(0, FAKE, FAKE, FAKE, None, None) == ARG  # no error flag
    assert lib.vce_fwd(a, 2, 4, 2, 12, None, -100, 0, FAKE, FAKE, FAKE, None, FAKE, None) == ARG
    assert lib.vce_fwd(a, 2, 4, 2, 13, FAKE, -100, 0, FAKE, FAKE, FAKE, None, FAKE, None) == LAYOUT
    assert lib.vce_fwd(a, 2, 0, 2, 12, None, -100, 0, None, None, None, None, None, None) == OK
    assert lib.vce_bwd(a, 2, 4, 2, 12, FAKE, FAKE, -100, 5, FAKE, FAKE, None) == ARG
    assert lib.vce_bwd(a, 2, 4, 2, 12, FAKE, FAKE, -100, 0, None, FAKE, None) == ARG


def test_membw_probe_checks_its_arguments():
    assert lib.vjsd_membw_probe(FAKE, 2 * FAKE, 1024, 2, None) == ARG  # unknown op
    assert lib.vjsd_membw_probe(FAKE, 2 * FAKE, 0, 0, None) == ARG  # empty
    assert lib.vjsd_membw_probe(FAKE, 2 * FAKE, 1000 + 4, 0, None) == ARG  # not whole words
    assert lib.vjsd_membw_probe(FAKE + 4, 2 * FAKE, 1024, 0, None) == ARG  # misaligned src
    assert lib.vjsd_membw_probe(FAKE, 2 * FAKE + 8, 1024, 1, None) == ARG  # misaligned dst
    assert lib.vjsd_membw_probe(None, 2 * FAKE, 1024, 0, None) == ARG
    assert lib.vjsd_membw_probe(FAKE, None, 1024, 1, None) == ARG
    assert lib.vjsd_membw_probe(FAKE, FAKE + 512, 1024, 1, None) == ARG  # overlapping copy


def test_default_split_matches_the_pages_uneven_example():
    """101 columns over two ranks give 51 / 50 (DeepSpeed PR #8309 timeline)."""
    import synth

    assert synth.default_split(101, 2) == [51, 50]
    assert synth.default_split(128256, 8) == [16032] * 8
    assert synth.default_split(5, 8) == [1, 1, 1, 1, 1, 0, 0, 0]


def test_linear_gemm_validates_before_any_launch():
    Op = abi.LinOperand
    a, b = Op(FAKE, 64, 2, 1), Op(FAKE, 64, 2, 1)
    g = lib.vlin_gemm
    assert g(0, 5, 64, a, b, FAKE, 5, 0, None) == OK  # no rows: nothing to do
    assert g(4, 0, 64, a, b, FAKE, 5, 0, None) == OK
    assert g(-1, 5, 64, a, b, FAKE, 5, 0, None) == ARG
    assert g(4, 5, -2, a, b, FAKE, 5, 0, None) == ARG
    assert g(4, 5, 64, a, b, FAKE, 5, 3, None) == ARG  # no such output mode
    assert g(4, 5, 64, Op(FAKE, 64, 1, 1), b, FAKE, 5, 0, None) == DTYPE  # fp16 operand
    assert g(4, 5, 64, a, Op(FAKE, 64, 0, 1), FAKE, 5, 0, None) == DTYPE  # fp32 only for A
    assert g(4, 5, 64, Op(FAKE + 8, 64, 2, 1), b, FAKE, 5, 0, None) == ARG  # not 16-byte aligned
    assert g(4, 5, 64, Op(FAKE, 68, 2, 1), b, FAKE, 5, 0, None) == ARG  # ld not a multiple of 8
    assert g(4, 5, 64, Op(FAKE, 56, 2, 1), b, FAKE, 5, 0, None) == ARG  # ld shorter than K
    assert g(40, 5, 64, Op(FAKE, 32, 2, 0), b, FAKE, 5, 0, None) == ARG  # i-major: ld < M
    assert g(4, 5, 64, Op(FAKE, 66, 0, 1), b, FAKE, 5, 0, None) == ARG  # fp32: ld % 4
    assert g(4, 5, 64, Op(FAKE, 64, 2, 2), b, FAKE, 5, 0, None) == ARG  # kmajor is 0 or 1
    assert g(4, 5, 64, a, b, FAKE, 4, 0, None) == ARG  # ldc < N
    assert g(4, 5, 64, a, b, None, 5, 0, None) == ARG  # no C
    assert g(4, 5, 64, a, b, FAKE + 2, 5, 0, None) == ARG  # fp32 C not element aligned


def test_linear_jsd_validates_before_any_launch():
    H = abi.LinHead
    st, te = H(FAKE, 64, FAKE, 64, 64), H(FAKE, 64, FAKE, 64, 64)
    f = lib.vljsd
    opts = abi.LossOpts(1.0, 0, None, 2)
    none = abi.LossOpts(1.0, 0, None, 0)
    by = ctypes.byref

    def call(N=16, V=100, beta=0.5, o=opts, chunk=8, group=0, ws=FAKE, out=FAKE, gh=None,
             ldgh=0, gw=None, ldgw=0, s=st, t=te):
        return f(by(s), by(t), N, V, beta, by(o), chunk, group, ws, out, gh, ldgh, gw, ldgw,
                 None)

    assert call(N=-1) == ARG
    assert call(V=0) == ARG
    assert call(chunk=0) == ARG
    assert call(group=-1) == ARG
    assert call(out=None) == ARG
    assert call(beta=1.5) == BETA
    assert call(beta=float("nan")) == BETA
    assert call(o=abi.LossOpts(0.0, 0, None, 2)) == ARG  # temperature
    assert call(s=H(FAKE + 8, 64, FAKE, 64, 64)) == ARG  # hidden not 16-byte aligned
    assert call(s=H(FAKE, 60, FAKE, 64, 56)) == ARG  # ldh not a multiple of 8
    assert call(t=H(FAKE, 64, FAKE, 56, 64)) == ARG  # ldw shorter than dim
    assert call(s=H(FAKE, 64, FAKE, 64, 0)) == ARG  # no width
    assert call(o=none, gh=FAKE, ldgh=64) == ARG  # gradients need a reduction
    assert call(gh=FAKE, ldgh=32) == ARG  # grad_h row stride < dim
    assert call(gw=FAKE + 1, ldgw=64) == ARG  # grad_w not element aligned
    assert call(ws=None) == ARG
    assert call(ws=FAKE + 16) == ARG  # workspace 256-byte aligned
    # no tokens, no reduction, no gradients: nothing to enqueue
    assert call(N=0, o=none, ws=None, s=H(None, 64, FAKE, 64, 64)) == OK


def test_linear_workspace_and_scale():
    w = lib.vljsd_workspace_bytes
    assert w(16, 0, 8, 4, 0) == 0 and w(16, 10, 0, 4, 0) == 0 and w(16, 10, 8, 0, 0) == 0
    assert w(16, 10, 8, 4, -1) == 0
    al = lambda x: (x + 255) // 256 * 256
    # two fp32 logit blocks of C rows (row stride V rounded up to 8) and the chunk's bf16
    # logit gradient; the group's logit gradient and hidden states transposed (token rows
    # padded to 8; a group is 4 GiB worth of whole chunks by default); the student head
    # transposed; the hidden-gradient product's fp32 partials when its K is split; the
    # per-token losses, the chunk's statistics / KL pair / pass workspace, the count, and
    # the fp32 head-gradient accumulator only with more than one group
    N, V, D, C = 8192, 151936, 3584, 4096
    ldl = V
    # (16 x 14 tiles of the hidden-gradient product: not split)
    expect = (2 * al(C * ldl * 4) + al(C * ldl * 2) + al(V * N * 2) + al(D * N * 2)
              + al(D * V * 2) + al(N * 4)
              + al(C * 32) + al(C * 8) + al(lib.vjsd_workspace_bytes(C, 1)) + al(8))
    assert w(N, V, D, C, 0) == expect
    C = 1024  # 4 x 14 tiles: K split 4 ways
    expect = (2 * al(C * ldl * 4) + al(C * ldl * 2) + al(V * N * 2) + al(D * N * 2)
              + al(D * V * 2) + al(4 * C * D * 4) + al(N * 4)
              + al(C * 32) + al(C * 8) + al(lib.vjsd_workspace_bytes(C, 1)) + al(8))
    assert w(N, V, D, C, 0) == expect
    # the default plan at that size holds less than the unfused route's bf16 logits of
    # both sides and the student's logit gradient
    assert w(N, V, D, 1024, 0) < 3 * N * V * 2
    # with a fixed group the workspace does not grow with N past one group, but for the
    # per-token losses (4 bytes a token)
    assert (w(16384, V, D, 1024, 4096) - al(16384 * 4)
            == w(65536, V, D, 1024, 4096) - al(65536 * 4))
    # chunks of 100 over 300 tokens are taken 96 at a time (whole multiples of 8); groups
    # of 150 tokens are 2 chunks, 192 tokens: two groups, so an accumulator
    ldl = 1008
    # (V = 1001 is no multiple of 64: no K split)
    expect = (2 * al(96 * ldl * 4) + al(96 * ldl * 2) + al(1001 * 192 * 2) + al(16 * 192 * 2)
              + al(16 * 1008 * 2) + al(300 * 4) + al(96 * 32) + al(96 * 8)
              + al(lib.vjsd_workspace_bytes(96, 1)) + al(8) + al(1001 * 16 * 4))
    assert w(300, 1001, 16, 100, 150) == expect
    s = lib.vlin_scale
    assert s(FAKE, 10, 3, FAKE, None) == DTYPE
    assert s(FAKE, 10, -1, FAKE, None) == DTYPE
    assert s(FAKE, 0, 2, FAKE, None) == OK
    assert s(FAKE + 2, 10, 1, FAKE, None) == ARG  # fp16 accepted, alignment still checked
    assert s(FAKE, -1, 2, FAKE, None) == ARG
    assert s(FAKE + 4, 10, 0, FAKE, None) == ARG
    assert s(FAKE, 10, 0, None, None) == ARG


def test_noalloc_backward_checks_before_any_device_call():
    """vjsd_bwd_noalloc validates like vjsd_bwd and refuses more rows than its scratch
    holds, all on the host (no device is touched here)."""
    a = shards([8], grads=True)
    assert lib.vjsd_bwd_noalloc(a, 1, 0, 2, None, None, 0.5, None, None) == OK
    assert lib.vjsd_bwd_noalloc(a, 1, 4, 2, FAKE, FAKE, 1.5, FAKE, None) == BETA
    assert lib.vjsd_bwd_noalloc(a, 1, 4, 7, FAKE, FAKE, 0.5, FAKE, None) == DTYPE
    assert lib.vjsd_bwd_noalloc(a, 1, 4, 2, FAKE, None, 0.5, FAKE, None) == ARG
    big = 65536 + 1
    assert lib.vjsd_bwd_noalloc(a, 1, big, 2, FAKE, FAKE, 0.5, FAKE, None) == SCRATCH
    assert b"65536" in lib.vjsd_strerror(SCRATCH)


def fb(arr, S, N, dt=2, beta=0.5, grad=FAKE, part=FAKE, stats=FAKE, kl=FAKE, loss=FAKE):
    return lib.vjsd_forward_backward(arr, S, N, dt, beta, grad, part, stats, kl, loss, None)


def test_forward_backward_arguments_are_checked_before_any_launch():
    a = shards([10], grads=True)
    assert fb(a, 1, 0, grad=None, part=None, stats=None, kl=None, loss=None) == OK
    for beta in (-0.1, 1.5, math.nan):
        assert fb(a, 1, 4, beta=beta) == BETA
    assert fb(a, 1, 4, dt=3) == DTYPE
    for k in ("grad", "part", "stats", "kl", "loss"):
        assert fb(a, 1, 4, **{k: None}) == ARG, k
    bad = shards([10], grads=True)
    bad[0].gs.p = bad[0].gs.p + 1  # a gradient view that is not element-aligned
    assert fb(bad, 1, 4) == ARG
    over = shards([10], grads=True)
    over[0].gt.row_stride = 9  # overlapping gradient rows
    assert fb(over, 1, 4) == ARG
    lay = shards([4, 6], grads=True)
    lay[1].vocab_start = 5
    assert fb(lay, 2, 4) == LAYOUT


def test_loss_forward_backward_options_are_checked():
    a = shards([10], grads=True)
    LossOpts = abi.LossOpts

    def call(opts, out=FAKE, N=4):
        return lib.vjsd_loss_forward_backward(a, 1, N, 2, 0.5, ctypes.byref(opts), FAKE, FAKE,
                                              FAKE, FAKE, FAKE, out, None)
    assert call(LossOpts(0.0, 0, None, 0)) == ARG  # temperature must be > 0
    assert call(LossOpts(math.nan, 0, None, 0)) == ARG
    assert call(LossOpts(1.0, 0, None, 3)) == ARG  # no such reduction
    assert call(LossOpts(1.0, 0, None, 2), out=None) == ARG  # a reduction needs out
    assert call(LossOpts(1.0, 0, None, 0), N=0, out=None) == OK
