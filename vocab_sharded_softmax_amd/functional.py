"""Autograd ops over libvjsd: per-token JSD, KL, entropy and log-probabilities.

Page keys: [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel
generalized JSD with Triton kernels"; [OPS-PR] DeepSpeed PR #8791 "Add
vocabulary-parallel logprobs, entropy and KL ops".

Logits are GPU tensors ``[N, V]`` or ``[B, T, V]`` (views with unit vocabulary
stride, such as causal-shift slices, are taken without a copy), or a list of
per-shard tensors ``[..., V_k]``; ``split`` cuts a whole tensor into logical
vocabulary shards.  Outputs are fp32 per token, shaped like the leading
dimensions.  The per-token ops leave temperature, masking, reduction and T^2
scaling to the caller [JSD-PR, Changes]; ``jsd_loss`` fuses them into the passes.
Only first-order gradients exist: a second backward raises [OPS-PR, Limitations].
Every step runs in libvjsd's HIP kernels.
"""
from __future__ import annotations

import torch
from torch.autograd.function import once_differentiable

from . import _abi
from ._abi import ShardSet

__all__ = ["jsd", "jsd_loss", "kl_div", "entropy", "logprobs", "topk_kl", "cross_entropy",
           "linear_jsd"]


def _unpack(n_shards: int, tensors):
    if n_shards == 0:
        return tensors[0]
    return list(tensors[:n_shards])


def _grads_like(x, listed):
    if listed:
        return [torch.empty(t.shape, dtype=t.dtype, device=t.device) for t in x]
    return torch.empty(x.shape, dtype=x.dtype, device=x.device)


def _flat(g):
    return g if isinstance(g, list) else [g]


class _JSD(torch.autograd.Function):
    @staticmethod
    def forward(ctx, beta, split, n_shards, *tensors):
        half = len(tensors) // 2
        s = _unpack(n_shards, tensors[:half])
        t = _unpack(n_shards, tensors[half:])
        sh = ShardSet(s, t, widths=split)
        dev = (s[0] if n_shards else s).device
        N, S = sh.N, sh.S
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        kl = torch.empty((N, 2), dtype=torch.float32, device=dev)
        loss = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        _abi.vjsd_forward(sh, beta, part, stats, kl, loss)
        ctx.beta, ctx.split, ctx.n_shards = beta, split, n_shards
        ctx.save_for_backward(stats, kl, *tensors)
        return loss

    @staticmethod
    @once_differentiable
    def backward(ctx, gloss):
        stats, kl, *tensors = ctx.saved_tensors
        half = len(tensors) // 2
        n = ctx.n_shards
        s = _unpack(n, tensors[:half])
        t = _unpack(n, tensors[half:])
        need = ctx.needs_input_grad[3:]
        want_s, want_t = any(need[:half]), any(need[half:])
        gs = _grads_like(s, bool(n)) if want_s else None
        gt = _grads_like(t, bool(n)) if want_t else None
        sh = ShardSet(s, t, widths=ctx.split, gs=gs, gt=gt)
        g = gloss.reshape(-1).to(torch.float32).contiguous()
        _abi.vjsd_bwd(sh, stats, kl, ctx.beta, g, _abi.new_part(sh.N, sh.S, stats.device))
        out_s = _flat(gs) if want_s else [None] * half
        out_t = _flat(gt) if want_t else [None] * half
        return (None, None, None, *out_s, *out_t)


class _JSDLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, beta, temperature, scale_t2, reduction, mask, split, n_shards, *tensors):
        half = len(tensors) // 2
        s = _unpack(n_shards, tensors[:half])
        t = _unpack(n_shards, tensors[half:])
        sh = ShardSet(s, t, widths=split)
        dev = (s[0] if n_shards else s).device
        N, S = sh.N, sh.S
        opts = _abi.loss_opts(N, temperature, scale_t2, mask, reduction)
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        kl = torch.empty((N, 2), dtype=torch.float32, device=dev)
        rows = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        out = torch.empty((), dtype=torch.float32, device=dev) if reduction != "none" else None
        _abi.vjsd_loss_forward(sh, beta, opts, part, stats, kl, rows, out)
        ctx.args = (beta, temperature, scale_t2, reduction, split, n_shards)
        ctx.save_for_backward(stats, kl, mask, *tensors)
        return rows if out is None else out

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        beta, temperature, scale_t2, reduction, split, n = ctx.args
        stats, kl, mask, *tensors = ctx.saved_tensors
        half = len(tensors) // 2
        s = _unpack(n, tensors[:half])
        t = _unpack(n, tensors[half:])
        need = ctx.needs_input_grad[7:]
        want_s, want_t = any(need[:half]), any(need[half:])
        gs = _grads_like(s, bool(n)) if want_s else None
        gt = _grads_like(t, bool(n)) if want_t else None
        sh = ShardSet(s, t, widths=split, gs=gs, gt=gt)
        opts = _abi.loss_opts(sh.N, temperature, scale_t2, mask, reduction)
        g = gout.reshape(-1).to(torch.float32).contiguous()
        _abi.vjsd_loss_backward(sh, beta, opts, stats, kl, g, _abi.new_part(sh.N, sh.S, stats.device))
        out_s = _flat(gs) if want_s else [None] * half
        out_t = _flat(gt) if want_t else [None] * half
        return (None, None, None, None, None, None, None, *out_s, *out_t)


class _KL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, reverse, split, n_shards, *tensors):
        half = len(tensors) // 2
        s = _unpack(n_shards, tensors[:half])
        t = _unpack(n_shards, tensors[half:])
        sh = ShardSet(s, t, widths=split)
        dev = (s[0] if n_shards else s).device
        N, S = sh.N, sh.S
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        kl = torch.empty((N, 2), dtype=torch.float32, device=dev)
        loss = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        _abi.vkl_fwd(sh, reverse, part, stats, kl, loss)
        ctx.reverse, ctx.split, ctx.n_shards = reverse, split, n_shards
        ctx.save_for_backward(stats, kl, *tensors)
        return loss

    @staticmethod
    @once_differentiable
    def backward(ctx, gloss):
        stats, kl, *tensors = ctx.saved_tensors
        half = len(tensors) // 2
        n = ctx.n_shards
        s = _unpack(n, tensors[:half])
        t = _unpack(n, tensors[half:])
        need = ctx.needs_input_grad[3:]
        want_s, want_t = any(need[:half]), any(need[half:])
        gs = _grads_like(s, bool(n)) if want_s else None
        gt = _grads_like(t, bool(n)) if want_t else None
        sh = ShardSet(s, t, widths=ctx.split, gs=gs, gt=gt)
        g = gloss.reshape(-1).to(torch.float32).contiguous()
        _abi.vkl_bwd(sh, ctx.reverse, stats, kl, g, _abi.new_part(sh.N, sh.S, stats.device))
        out_s = _flat(gs) if want_s else [None] * half
        out_t = _flat(gt) if want_t else [None] * half
        return (None, None, None, *out_s, *out_t)


class _Entropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, split, n_shards, *tensors):
        x = _unpack(n_shards, tensors)
        sh = ShardSet(x, widths=split)
        dev = (x[0] if n_shards else x).device
        N, S = sh.N, sh.S
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        ent = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        _abi.ventropy_fwd(sh, part, stats, ent)
        ctx.split, ctx.n_shards = split, n_shards
        # the backward reads H from its own copy: the caller may overwrite the output
        ctx.save_for_backward(stats, ent.clone(), *tensors)
        return ent

    @staticmethod
    @once_differentiable
    def backward(ctx, gent):
        stats, ent, *tensors = ctx.saved_tensors
        n = ctx.n_shards
        x = _unpack(n, tensors)
        gx = _grads_like(x, bool(n))
        sh = ShardSet(x, widths=ctx.split, gs=gx)
        _abi.ventropy_bwd(sh, stats, ent, gent.reshape(-1).to(torch.float32).contiguous(),
                          _abi.new_part(sh.N, sh.S, stats.device))
        return (None, None, *_flat(gx))


class _Logprobs(torch.autograd.Function):
    @staticmethod
    def forward(ctx, ids, ignore_index, split, n_shards, *tensors):
        x = _unpack(n_shards, tensors)
        sh = ShardSet(x, widths=split)
        dev = (x[0] if n_shards else x).device
        N, S = sh.N, sh.S
        K = ids.shape[-1]
        idv = ids.reshape(N, K).to(torch.int64).contiguous()
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        out = torch.empty((*sh.lead_shape, K), dtype=torch.float32, device=dev)
        err = torch.zeros((1,), dtype=torch.int32, device=dev)
        _abi.vlogprobs_fwd(sh, sh.V, idv, ignore_index, part, stats, out, err)
        # the range check runs every call; it needs this host synchronisation
        if N and K and int(err.item()):
            raise ValueError("logprobs: an index is outside [0, V) and is not ignore_index")
        ctx.ignore_index, ctx.split, ctx.n_shards, ctx.V = ignore_index, split, n_shards, sh.V
        ctx.save_for_backward(stats, idv, *tensors)
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        stats, idv, *tensors = ctx.saved_tensors
        n = ctx.n_shards
        x = _unpack(n, tensors)
        gx = _grads_like(x, bool(n))
        sh = ShardSet(x, widths=ctx.split, gs=gx)
        g = gout.reshape(idv.shape).to(torch.float32).contiguous()
        _abi.vlogprobs_bwd(sh, ctx.V, stats, idv, ctx.ignore_index, g,
                           _abi.new_part(sh.N, sh.S, stats.device))
        return (None, None, None, None, *_flat(gx))


class _TopkKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, ids, tlogp, ignore_index, split, n_shards, *tensors):
        x = _unpack(n_shards, tensors)
        sh = ShardSet(x, widths=split)
        dev = (x[0] if n_shards else x).device
        N, S = sh.N, sh.S
        K = ids.shape[-1]
        idv = ids.reshape(N, K).to(torch.int64).contiguous()
        tl = tlogp.reshape(N, K).to(torch.float32).contiguous()
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        kl = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        err = torch.zeros((1,), dtype=torch.int32, device=dev)
        _abi.vtopk_kl_fwd(sh, sh.V, idv, tl, ignore_index, part, stats, kl, err)
        if N and K and int(err.item()):
            raise ValueError("topk_kl: an index is outside [0, V) and is not ignore_index")
        ctx.ignore_index, ctx.split, ctx.n_shards, ctx.V = ignore_index, split, n_shards, sh.V
        ctx.save_for_backward(stats, idv, tl, *tensors)
        return kl

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        stats, idv, tl, *tensors = ctx.saved_tensors
        n = ctx.n_shards
        x = _unpack(n, tensors)
        gx = _grads_like(x, bool(n))
        sh = ShardSet(x, widths=ctx.split, gs=gx)
        g = gout.reshape(-1).to(torch.float32).contiguous()
        _abi.vtopk_kl_bwd(sh, ctx.V, stats, idv, tl, ctx.ignore_index, g,
                          _abi.new_part(sh.N, sh.S, stats.device))
        return (None, None, None, None, None, *_flat(gx))


class _CrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, labels, ignore_index, reduction, split, n_shards, *tensors):
        x = _unpack(n_shards, tensors)
        sh = ShardSet(x, widths=split)
        dev = (x[0] if n_shards else x).device
        N, S = sh.N, sh.S
        lab = labels.reshape(N).to(torch.int64).contiguous()
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        rows = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        out = torch.empty((), dtype=torch.float32, device=dev) if reduction != "none" else None
        err = torch.zeros((1,), dtype=torch.int32, device=dev)
        _abi.vce_fwd(sh, sh.V, lab, ignore_index, reduction, part, stats, rows, out, err)
        if N and int(err.item()):
            raise ValueError("cross_entropy: a label is outside [0, V) and is not ignore_index")
        ctx.args = (ignore_index, reduction, split, n_shards, sh.V)
        ctx.save_for_backward(stats, lab, *tensors)
        return rows if out is None else out

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        ignore_index, reduction, split, n, V = ctx.args
        stats, lab, *tensors = ctx.saved_tensors
        x = _unpack(n, tensors)
        gx = _grads_like(x, bool(n))
        sh = ShardSet(x, widths=split, gs=gx)
        g = gout.reshape(-1).to(torch.float32).contiguous()
        _abi.vce_bwd(sh, V, stats, lab, ignore_index, reduction, g,
                     _abi.new_part(sh.N, sh.S, stats.device))
        return (None, None, None, None, None, *_flat(gx))


def _as_args(x):
    if isinstance(x, (list, tuple)):
        return len(x), list(x)
    return 0, [x]


def jsd(student, teacher, beta: float = 0.5, *, split=None) -> torch.Tensor:
    """Per-token generalized JSD, fp32 [JSD-PR, Changes].

    ``beta == 0`` is forward KL(teacher || student) and ``beta == 1`` reverse
    KL(student || teacher), as explicit branches.  A teacher that does not require
    grad gets none (the student-only backward).
    """
    beta = float(beta)
    if not (0.0 <= beta <= 1.0):
        raise ValueError("beta must be in [0, 1]")
    ns, s = _as_args(student)
    nt, t = _as_args(teacher)
    if ns != nt or len(s) != len(t):
        raise ValueError("student and teacher must be given the same way (tensor or shard list)")
    return _JSD.apply(beta, None if split is None else tuple(split), ns, *s, *t)


class _JSDLossInForward(torch.autograd.Function):
    """jsd_loss of a reduced (scalar) loss with its gradients computed in the forward, in
    one call (vjsd_loss_forward_backward for a unit upstream gradient); the backward
    scales them by the actual upstream gradient in place, which leaves them untouched
    on the device when it is exactly 1."""

    @staticmethod
    def forward(ctx, beta, temperature, scale_t2, reduction, mask, split, n_shards, *tensors):
        half = len(tensors) // 2
        s = _unpack(n_shards, tensors[:half])
        t = _unpack(n_shards, tensors[half:])
        need = ctx.needs_input_grad[7:]
        want_s, want_t = any(need[:half]), any(need[half:])
        gs = _grads_like(s, bool(n_shards)) if want_s else None
        gt = _grads_like(t, bool(n_shards)) if want_t else None
        sh = ShardSet(s, t, widths=split, gs=gs, gt=gt)
        dev = (s[0] if n_shards else s).device
        N, S = sh.N, sh.S
        opts = _abi.loss_opts(N, temperature, scale_t2, mask, reduction)
        part = _abi.new_part(N, S, dev)
        stats = torch.empty((N, 4), dtype=torch.float64, device=dev)
        kl = torch.empty((N, 2), dtype=torch.float32, device=dev)
        rows = torch.empty(sh.lead_shape, dtype=torch.float32, device=dev)
        out = torch.empty((), dtype=torch.float32, device=dev)
        one = torch.ones(1, dtype=torch.float32, device=dev)
        _abi.vjsd_loss_forward_backward(sh, beta, opts, one, part, stats, kl, rows, out)
        ctx.grads = (_flat(gs) if want_s else [None] * half, _flat(gt) if want_t else [None] * half)
        ctx.used = False
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        if ctx.used:
            raise RuntimeError("jsd_loss(grad_in_forward=True): the backward scales its stored "
                               "gradients in place and can run only once")
        ctx.used = True
        g = gout.reshape(-1)[:1].to(torch.float32).contiguous()
        out_s, out_t = ctx.grads
        ctx.grads = None
        for x in (*out_s, *out_t):
            if x is not None:
                _abi.vlin_scale(x, g)
        return (None, None, None, None, None, None, None, *out_s, *out_t)


def jsd_loss(student, teacher, beta: float = 0.5, *, temperature: float = 1.0,
             scale_t2: bool = False, mask=None, reduction: str = "mean",
             split=None, grad_in_forward: bool = False) -> torch.Tensor:
    """Distillation loss around the per-token JSD, fused into its passes.

    Both logits are divided by ``temperature`` in registers (no fp32 copies); with
    ``scale_t2`` the per-token losses carry T^2.  ``mask`` (bool or uint8, shaped
    like the leading dimensions) drops tokens: their logits are never read and their
    gradients are 0.  ``reduction``: "none" (per-token losses, 0 where dropped),
    "sum", or "mean" over the kept tokens (0 when none is kept).  The pages leave all
    of this to the caller [JSD-PR, Changes]; its teacher-cache caller divides by the
    temperature in fp32 first and keeps the token mean and T^2 scaling
    (DeepSpeedExamples PR #1019).

    ``grad_in_forward`` (a "sum" or "mean" loss only): the forward computes the
    gradients too, in one call with the loss (vjsd_loss_forward_backward, one launch
    per row set for one shard without a mask); the backward multiplies them by the
    upstream gradient in place, a device-side no-op when it is exactly 1 (a plain
    ``loss.backward()``).  The gradients are held from the forward on, and the backward
    can run once.
    """
    beta = float(beta)
    if not (0.0 <= beta <= 1.0):
        raise ValueError("beta must be in [0, 1]")
    temperature = float(temperature)
    if not (temperature > 0.0 and temperature < float("inf")):
        raise ValueError("temperature must be a positive finite number")
    if reduction not in _abi.REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_abi.REDUCTIONS)}")
    ns, s = _as_args(student)
    nt, t = _as_args(teacher)
    if ns != nt or len(s) != len(t):
        raise ValueError("student and teacher must be given the same way (tensor or shard list)")
    m = None
    if mask is not None:
        lead = s[0].shape[:-1]
        if tuple(mask.shape) != tuple(lead):
            raise ValueError(f"mask must have shape {tuple(lead)}, got {tuple(mask.shape)}")
        m = mask.reshape(-1)
        m = m.view(torch.uint8) if m.dtype == torch.bool else m.to(torch.uint8)
        m = m.contiguous()
    fn = _JSDLoss
    if grad_in_forward:
        if reduction == "none":
            raise ValueError("grad_in_forward needs a reduced loss ('sum' or 'mean'): "
                             "per-token upstream gradients are not known in the forward")
        fn = _JSDLossInForward
    return fn.apply(beta, temperature, bool(scale_t2), reduction, m,
                    None if split is None else tuple(split), ns, *s, *t)


def kl_div(student, teacher, reverse: bool = False, *, split=None) -> torch.Tensor:
    """Per-token KL(teacher || student), or KL(student || teacher) with ``reverse``
    [OPS-PR, What]; the forward is a single input pass."""
    ns, s = _as_args(student)
    nt, t = _as_args(teacher)
    if ns != nt or len(s) != len(t):
        raise ValueError("student and teacher must be given the same way (tensor or shard list)")
    return _KL.apply(bool(reverse), None if split is None else tuple(split), ns, *s, *t)


def entropy(logits, *, split=None) -> torch.Tensor:
    """Per-token entropy of softmax(logits) [OPS-PR, What]; single input pass."""
    n, x = _as_args(logits)
    return _Entropy.apply(None if split is None else tuple(split), n, *x)


def topk_kl(student, teacher_topk_ids, teacher_topk_logp, *, ignore_index: int = -100,
            split=None) -> torch.Tensor:
    """Teacher top-k forward KL per token [OPS-PR, What]:
    sum_k exp(t_k) * (t_k - log p_student(id_k)) over the teacher's top-k ids
    ``[..., K]`` (global) and log-probabilities ``[..., K]``.  Slots equal to
    ``ignore_index`` or with t_k = -inf are padding.  The student's log-probabilities
    are gathered and combined inside one kernel; gradients flow to the student
    logits only (the teacher's log-probabilities are data).  An index outside the
    vocabulary raises ValueError after a host synchronisation."""
    if teacher_topk_logp.requires_grad:
        raise ValueError("teacher_topk_logp is data: detach it")
    if teacher_topk_ids.shape != teacher_topk_logp.shape:
        raise ValueError("teacher_topk_ids and teacher_topk_logp must have the same shape")
    n, x = _as_args(student)
    if tuple(teacher_topk_ids.shape[:-1]) != tuple(x[0].shape[:-1]):
        raise ValueError("the top-k tensors must be shaped [..., K] like the logits' leading dims")
    return _TopkKL.apply(teacher_topk_ids, teacher_topk_logp, int(ignore_index),
                         None if split is None else tuple(split), n, *x)


def cross_entropy(logits, labels, *, ignore_index: int = -100, reduction: str = "mean",
                  split=None) -> torch.Tensor:
    """Cross-entropy of integer ``labels`` (shaped like the leading dimensions, global
    ids) over the sharded vocabulary, as ``torch.nn.functional.cross_entropy`` with
    ``ignore_index`` and reduction "none" / "sum" / "mean" (a mean over no labelled
    token is 0).  Rows whose label is ignored are never read (DeepSpeed PR #8309,
    "[AutoTP] vocab-parallel LM head": vocab_parallel_cross_entropy).  A label outside
    the vocabulary raises ValueError after a host synchronisation."""
    if reduction not in _abi.REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_abi.REDUCTIONS)}")
    n, x = _as_args(logits)
    if tuple(labels.shape) != tuple(x[0].shape[:-1]):
        raise ValueError("labels must be shaped like the logits' leading dimensions")
    return _CrossEntropy.apply(labels, int(ignore_index), reduction,
                               None if split is None else tuple(split), n, *x)


def logprobs(logits, index, *, ignore_index: int = -100, split=None) -> torch.Tensor:
    """Log-probabilities of ``index`` (``[...]`` or top-k ``[..., K]``, global ids);
    positions equal to ``ignore_index`` return exactly 0 [OPS-PR, What].  An index
    outside the vocabulary raises ValueError after a host synchronisation."""
    n, x = _as_args(logits)
    single = index.dim() == (x[0].dim() - 1)
    ids = index.unsqueeze(-1) if single else index
    out = _Logprobs.apply(ids, int(ignore_index), None if split is None else tuple(split), n, *x)
    return out.squeeze(-1) if single else out


class _LinearJSD(torch.autograd.Function):
    """Fused-linear loss: the gradients of a reduced loss are formed in the forward pass
    for a unit upstream gradient (the logit blocks exist only there) and scaled by the
    actual one in the backward."""

    @staticmethod
    def forward(ctx, beta, temperature, scale_t2, reduction, mask, chunk, group, hs, ws, ht, wt):
        N, V = hs.shape[0], ws.shape[0]
        dev = hs.device
        want_h = ctx.needs_input_grad[7] and reduction != "none"
        want_w = ctx.needs_input_grad[8] and reduction != "none"
        student = _abi.lin_head(hs, ws, "student")
        teacher = _abi.lin_head(ht, wt, "teacher")
        opts = _abi.loss_opts(N, temperature, scale_t2, mask, reduction)
        C = max(1, min(int(chunk), max(N, 1)))
        nbytes = _abi.vljsd_workspace_bytes(N, V, hs.shape[1], C, group)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
        out = torch.empty((N,) if reduction == "none" else (), dtype=torch.float32, device=dev)
        gh = torch.empty(hs.shape, dtype=hs.dtype, device=dev) if want_h else None
        gw = torch.empty(ws.shape, dtype=ws.dtype, device=dev) if want_w else None
        _abi.vljsd(student, teacher, N, V, beta, opts, C, workspace, out, gh, gw, group=group)
        del workspace
        ctx.save_for_backward(gh, gw)
        ctx.used = False
        return out

    @staticmethod
    @once_differentiable
    def backward(ctx, gout):
        if ctx.used:
            raise RuntimeError("linear_jsd: the backward scales its stored gradients in place "
                               "and can run only once")
        ctx.used = True
        gh, gw = ctx.saved_tensors
        g = gout.reshape(-1)[:1].to(torch.float32).contiguous()
        if gh is not None:
            _abi.vlin_scale(gh, g)
        if gw is not None:
            _abi.vlin_scale(gw, g)
        return (None, None, None, None, None, None, None, gh, gw, None, None)


def linear_jsd(student_hidden, student_head, teacher_hidden, teacher_head, beta: float = 0.5, *,
               temperature: float = 1.0, scale_t2: bool = False, mask=None,
               reduction: str = "mean", chunk: int = 1024, group: int = 0) -> torch.Tensor:
    """Fused-linear distillation loss: ``jsd_loss`` on the logits ``h @ W^T`` of the
    student and the teacher, evaluated ``chunk`` tokens at a time so that the full
    ``[N, V]`` logits never exist (the fused-linear divergence [JSD-PR, Scope and
    limitations] and [OPS-PR, Limitations] leave as future work; [JSD-PR, Motivation]
    describes the tiled LM-head projection it replaces materialised logits with).

    Hidden states ``[N, D]`` or ``[B, T, D]`` and head weights ``[V, D]``, bfloat16,
    with unit column stride; the teacher's width may differ from the student's.  The
    teacher is a constant: pass it without ``requires_grad``.  Gradients flow to the
    student's hidden states and head weight and need ``reduction`` "sum" or "mean";
    "none" returns per-token losses without gradients.  The logit products run on the
    matrix cores in bf16 with fp32 accumulation; the logit gradient is rounded to bf16
    for the two gradient products, as a bf16 model's backward rounds it: the hidden
    gradient is taken chunk by chunk, and for the head gradient the logit gradient is
    kept transposed for ``group`` tokens at a time (whole chunks; 0: as many as fit
    4 GiB).  The default chunk of 1024 tokens keeps the workspace at N=8192, V=151936,
    D=3584 to 5.3 GB (the unfused route holds 7.5 GB of bf16 logits and logit gradient)
    for about the time of 4096-token chunks (9.9 GB).
    """
    beta = float(beta)
    if not (0.0 <= beta <= 1.0):
        raise ValueError("beta must be in [0, 1]")
    temperature = float(temperature)
    if not (temperature > 0.0 and temperature < float("inf")):
        raise ValueError("temperature must be a positive finite number")
    if reduction not in _abi.REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_abi.REDUCTIONS)}")
    if int(chunk) < 1:
        raise ValueError("chunk must be a positive number of tokens")
    if int(group) < 0:
        raise ValueError("group must be a number of tokens (0: automatic)")
    if teacher_hidden.requires_grad or teacher_head.requires_grad:
        raise ValueError("the teacher is a constant: pass teacher tensors without requires_grad "
                         "(detach them)")
    if reduction == "none" and torch.is_grad_enabled() and (
            student_hidden.requires_grad or student_head.requires_grad):
        raise ValueError("gradients of linear_jsd need reduction 'sum' or 'mean'")
    lead = student_hidden.shape[:-1]
    if tuple(teacher_hidden.shape[:-1]) != tuple(lead):
        raise ValueError("student and teacher hidden states must cover the same tokens")
    hs = student_hidden.reshape(-1, student_hidden.shape[-1])
    ht = teacher_hidden.reshape(-1, teacher_hidden.shape[-1])
    m = None
    if mask is not None:
        if tuple(mask.shape) != tuple(lead):
            raise ValueError(f"mask must have shape {tuple(lead)}, got {tuple(mask.shape)}")
        m = mask.reshape(-1)
        m = m.view(torch.uint8) if m.dtype == torch.bool else m.to(torch.uint8)
        m = m.contiguous()
    out = _LinearJSD.apply(beta, temperature, bool(scale_t2), reduction, m, int(chunk), int(group),
                           hs, student_head, ht, teacher_head)
    return out.view(lead) if reduction == "none" else out
