"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

The plain, slow, definition-level reference the GPU library is checked against
(``vjsd_oracle.c``, built with gcc into ``liboracle.so``), plus a pure-Python
brute force for tiny inputs (``oracle.brute``).  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import this package; the product path
never does, and this package imports nothing from the product.

Page keys: [JSD-PR] DeepSpeed PR #8958 "[VocabTP] Add vocabulary-parallel
generalized JSD with Triton kernels"; [OPS-PR] DeepSpeed PR #8791 "Add
vocabulary-parallel logprobs, entropy and KL ops".

Every function takes CPU torch tensors holding the exact stored input values
(float32, float16 or bfloat16; 2-D ``[N, V]`` with unit column stride; float64
for logits already transformed in fp64), evaluates the listed rows in fp64 and
returns numpy float64 arrays packed by position in ``rows``.  ``widths`` splits
the vocabulary into consecutive shards (default: one).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vjsd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at another build of the same source (a planted-mistake
# variant) to show that the pins catch it.
_LIB_OVERRIDE = os.environ.get("VJSD_ORACLE_LIB")
_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3}

_lib = None


def build() -> str:
    """Compile the C oracle with gcc (fp64, IEEE semantics, OpenMP over rows)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-std=gnu11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-Wextra", "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out_dir: str) -> str:
    """The same source under gcc's AddressSanitizer and UndefinedBehaviorSanitizer
    (into out_dir/liboracle_san.so; load it with VJSD_ORACLE_LIB and gcc's libasan
    preloaded).  Checks the checker's own memory and arithmetic safety."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run(["gcc", "-std=gnu11", "-O1", "-g", "-fopenmp", "-fPIC", "-shared", "-Wall",
                    "-Wextra", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-fno-omit-frame-pointer", "-o", lib, _SRC, "-lm"], check=True)
    return lib


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        D = ctypes.c_double
        lib.or_stats.argtypes = [P, I, I64, I64, P, I, P, I64, P, P]
        lib.or_jsd.argtypes = [P, P, I, I64, I64, P, I, D, P, I64, P, P, P, P, P, P]
        lib.or_entropy.argtypes = [P, I, I64, I64, P, I, P, I64, P, P, P]
        lib.or_logprobs.argtypes = [P, I, I64, I64, P, I, P, I64, P, I, I64, P, P, P, P]
        lib.or_num_threads.restype = I
        _lib = lib
    return _lib


def num_threads() -> int:
    """OpenMP threads the oracle runs with."""
    return _load().or_num_threads()


def _mat(x: torch.Tensor):
    if x.device.type != "cpu":
        raise ValueError("oracle inputs must be CPU tensors")
    if x.dim() != 2 or (x.size(1) > 1 and x.stride(1) != 1):
        raise ValueError("oracle inputs must be 2-D with unit column stride")
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype}")
    return x.data_ptr(), _DT[x.dtype], x.stride(0) if x.size(0) > 1 else x.size(1)


def _common(x, widths, rows):
    V = x.size(1)
    w = np.asarray([V] if widths is None else list(widths), dtype=np.int64)
    if w.sum() != V or (w < 0).any():
        raise ValueError("shard widths must be >= 0 and sum to V")
    r = np.arange(x.size(0), dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    if r.size and (r.min() < 0 or r.max() >= x.size(0)):
        raise ValueError("row index out of range")
    return V, np.ascontiguousarray(w), np.ascontiguousarray(r)


def _p(a):
    return None if a is None else a.ctypes.data


def stats(x, widths=None, rows=None):
    """Per-row (max, ln sum exp(x - max)) through the cross-shard merge."""
    ptr, dt, ld = _mat(x)
    V, w, r = _common(x, widths, rows)
    m = np.empty(r.size)
    lz = np.empty(r.size)
    _load().or_stats(ptr, dt, ld, V, _p(w), w.size, _p(r), r.size, _p(m), _p(lz))
    return m, lz


def jsd(s, t, beta, widths=None, rows=None, gout=None, grads=True):
    """Generalized JSD per row; beta 0 / 1 are the forward / reverse KL branches.

    Returns dict(loss, kt, ks, gs, gt) with kt = KL(p_t||M), ks = KL(p_s||M)
    (M = p_s at beta 0, p_t at beta 1), gradients of ``gout[q] * loss[q]``.
    """
    if s.shape != t.shape or s.dtype != t.dtype:
        raise ValueError("student and teacher must match in shape and dtype")
    if _mat(s)[2] != _mat(t)[2]:  # the C side takes one row stride for both
        s, t = s.contiguous(), t.contiguous()
    ps_, dt, ld = _mat(s)
    pt_ = _mat(t)[0]
    V, w, r = _common(s, widths, rows)
    g = None if gout is None else np.ascontiguousarray(gout, dtype=np.float64)
    loss, kt, ks = np.empty(r.size), np.empty(r.size), np.empty(r.size)
    gs = np.empty((r.size, V)) if grads else None
    gt = np.empty((r.size, V)) if grads else None
    _load().or_jsd(ps_, pt_, dt, ld, V, _p(w), w.size, float(beta), _p(r), r.size, _p(g),
                   _p(loss), _p(kt), _p(ks), _p(gs), _p(gt))
    return dict(loss=loss, kt=kt, ks=ks, gs=gs, gt=gt)


def kl_div(s, t, reverse=False, **kw):
    """KL(p_t||p_s), or KL(p_s||p_t) with reverse=True: the beta = 0 / 1 branches."""
    return jsd(s, t, 1.0 if reverse else 0.0, **kw)


def jsd_loss(s, t, beta, temperature=1.0, scale_t2=False, mask=None, reduction="none",
             grad=None, widths=None, grads=True):
    """The distillation loss around the per-token JSD, as a caller writes it.

    The callers of the pages' per-token ops divide both logits by the temperature,
    multiply by T^2 when asked, and average over the tokens a mask keeps ([JSD-PR,
    Changes]: temperature, T^2 scaling, masking and normalisation are the caller's;
    DeepSpeedExamples PR #1019: the teacher-cache route keeps the token mean and the
    T^2 scaling and divides by a temperature other than 1 first).  Here, in fp64:
        l_r   = JSD_beta(softmax(s_r / T), softmax(t_r / T)) * (T^2 if scale_t2)
        rows  = l_r where mask_r, else 0 (masked rows are never evaluated)
        "sum" : sum of l_r over the kept rows
        "mean": that sum / max(kept rows, 1)   (no kept rows: 0)
    ``grad`` is the upstream gradient: [N] for "none", a scalar otherwise.  Returns
    dict(rows, out, kt, ks, gs, gt); gs / gt are d(sum_r grad_r * rows_r)/d(logits)
    for "none", d(grad * out)/d(logits) otherwise; masked rows get exactly 0.
    """
    N = s.shape[0]
    keep = np.ones(N, bool) if mask is None else np.asarray(mask).astype(bool)
    T = float(temperature)
    fac = T * T if scale_t2 else 1.0
    count = int(keep.sum())
    if reduction == "none":
        g = np.zeros(N) if grad is None else np.asarray(grad, np.float64).copy()
    elif reduction == "sum":
        g = np.full(N, 0.0 if grad is None else float(grad))
    elif reduction == "mean":
        g = np.full(N, (0.0 if grad is None else float(grad)) / max(count, 1))
    else:
        raise ValueError(reduction)
    g = np.where(keep, g * fac, 0.0)
    st = s.double() / T  # the caller's division, here exact to fp64
    tt = t.double() / T
    ref = jsd(st, tt, beta, widths=widths, gout=g, grads=grads)
    rows = np.where(keep, ref["loss"] * fac, 0.0)
    out = None
    if reduction != "none":
        tot = rows[keep].sum() if count else 0.0
        out = tot / max(count, 1) if reduction == "mean" else tot
    res = dict(rows=rows, out=out, kt=np.where(keep, ref["kt"], 0.0),
               ks=np.where(keep, ref["ks"], 0.0), gs=None, gt=None)
    if grads:
        # chain rule through x / T; masked rows contribute nothing at all
        res["gs"] = np.where(keep[:, None], ref["gs"] / T, 0.0)
        res["gt"] = np.where(keep[:, None], ref["gt"] / T, 0.0)
    return res


def topk_kl(x, ids, tlogp, ignore_index=-100, widths=None, rows=None, gout=None, grads=True):
    """Teacher top-k forward KL per row, from the student's log-probabilities at the
    teacher's top-k ids ([OPS-PR, What]: the verl forward_kl_topk pattern):
        kl = sum_k exp(t_k) * (t_k - lp_s(id_k))
    over the valid slots: id_k != ignore_index and t_k > -inf (an ignored slot is
    padding; a -inf teacher log-probability has no mass).  A valid slot whose student
    log-probability is -inf makes the row +inf, even when exp(t_k) underflows [OPS-PR,
    Tests]; an undefined student row is NaN with zero gradient [OPS-PR, review].
    ``tlogp`` is data (no gradient); gx is d(gout[q] * kl[q])/dx through the
    log-probabilities' gradient with weights -gout * exp(t_k).
    """
    idv = np.asarray(ids, dtype=np.int64)
    t = np.asarray(tlogp, dtype=np.float64).reshape(idv.shape)
    n = idv.shape[0]
    g = np.ones(n) if gout is None else np.asarray(gout, np.float64).reshape(n)
    valid = (idv != ignore_index) & (t > -np.inf)
    w = np.where(valid, -g[:, None] * np.exp(np.where(valid, t, 0.0)), 0.0)
    lp = logprobs(x, idv, ignore_index, widths=widths, rows=rows, gout=w, grads=grads)
    lps = lp["out"]
    with np.errstate(invalid="ignore"):
        terms = np.where(valid, np.exp(np.where(valid, t, 0.0)) * (t - lps), 0.0)
        terms = np.where(valid & (lps == -np.inf), np.inf, terms)
    kl = terms.sum(axis=1)
    st = stats(x, widths=widths, rows=rows)[0]
    undefined = st == -np.inf
    kl = np.where(undefined, np.nan, kl)
    gx = lp["gx"]
    if grads:
        gx = np.where(undefined[:, None], 0.0, gx)
    return dict(kl=kl, gx=gx)


def cross_entropy(x, labels, ignore_index=-100, reduction="mean", grad=None, widths=None,
                  grads=True):
    """Cross-entropy of integer labels over a sharded vocabulary, the loss a
    vocabulary-parallel causal-LM head installs (DeepSpeed PR #8309, "[AutoTP] vocab-
    parallel LM head": vocab_parallel_cross_entropy), written out with the
    log-probabilities:
        rows_r = -lp(x_r)[label_r], exactly 0 where label_r == ignore_index
        "sum": sum of rows over labelled tokens; "mean": that sum / max(labelled, 1)
    (no labelled token gives 0 with zero gradients).  An undefined row with a label
    is NaN with zero gradient.  ``grad``: [N] for "none", a scalar otherwise.
    Returns dict(rows, out, gx) with gx = d(sum_r grad_r rows_r or grad * out)/dx.
    """
    lab = np.asarray(labels, dtype=np.int64).reshape(-1)
    N = lab.size
    valid = lab != ignore_index
    count = int(valid.sum())
    if reduction == "none":
        g = np.zeros(N) if grad is None else np.asarray(grad, np.float64).reshape(N)
    elif reduction == "sum":
        g = np.full(N, 0.0 if grad is None else float(grad))
    elif reduction == "mean":
        g = np.full(N, (0.0 if grad is None else float(grad)) / max(count, 1))
    else:
        raise ValueError(reduction)
    lp = logprobs(x, lab[:, None], ignore_index, widths=widths, gout=-g[:, None], grads=grads)
    rows = np.where(valid, -lp["out"][:, 0], 0.0)
    out = None
    if reduction != "none":
        tot = rows[valid].sum() if count else 0.0
        out = tot / max(count, 1) if reduction == "mean" else tot
    return dict(rows=rows, out=out, gx=lp["gx"])


def entropy(x, widths=None, rows=None, gout=None, grads=True):
    ptr, dt, ld = _mat(x)
    V, w, r = _common(x, widths, rows)
    g = None if gout is None else np.ascontiguousarray(gout, dtype=np.float64)
    H = np.empty(r.size)
    gx = np.empty((r.size, V)) if grads else None
    _load().or_entropy(ptr, dt, ld, V, _p(w), w.size, _p(r), r.size, _p(g), _p(H), _p(gx))
    return dict(ent=H, gx=gx)


def logprobs(x, ids, ignore_index=-100, widths=None, rows=None, gout=None, grads=True):
    """Log-probabilities of ``ids[q, k]`` (global vocabulary ids) for each listed row.

    ``ids`` has one row of K ids per listed row.  Raises ValueError on an id outside
    [0, V) that is not ``ignore_index``.
    """
    ptr, dt, ld = _mat(x)
    V, w, r = _common(x, widths, rows)
    idv = np.ascontiguousarray(np.asarray(ids, dtype=np.int64).reshape(r.size, -1))
    K = idv.shape[1]
    g = None if gout is None else np.ascontiguousarray(
        np.asarray(gout, np.float64).reshape(r.size, K))
    out = np.empty((r.size, K))
    gx = np.empty((r.size, V)) if grads else None
    if grads and g is None:
        g = np.ones((r.size, K))
    err = ctypes.c_int(0)
    _load().or_logprobs(ptr, dt, ld, V, _p(w), w.size, _p(r), r.size, _p(idv), K,
                        int(ignore_index), _p(g), _p(out), _p(gx), ctypes.byref(err))
    if err.value:
        raise ValueError("logprobs: an id is outside [0, V) and is not ignore_index")
    return dict(out=out, gx=gx)


def linear_jsd(hs, ws, ht, wt, beta, temperature=1.0, scale_t2=False, mask=None,
               reduction="mean", grad=1.0, grads=True, head_grad=True):
    """The distillation loss of ``jsd_loss`` on LM-head projections, in fp64.

    [JSD-PR, Motivation] names a route that evaluates the divergence from tiled
    LM-head projections without materialising the full logits, and [JSD-PR, Scope and
    limitations] / [OPS-PR, Limitations] leave such a fused-linear variant as future
    work: the logits of a row are the products of its hidden state with every row of
    the head weight.  Here, on the exact stored values:
        logits_s = hs @ ws^T   ([N, Ds] x [V, Ds] -> [N, V]),  logits_t = ht @ wt^T
        result   = jsd_loss(logits_s, logits_t, beta, temperature, scale_t2, mask,
                            reduction, grad)
    The teacher is a constant (no gradients).  With G = d(result)/d(logits_s) from
    ``jsd_loss``, the chain rule through the product gives
        gh = G @ ws   ([N, Ds], gradient of the student hidden states)
        gw = G^T @ hs ([V, Ds], gradient of the student head weight)
    Returns dict(out, rows, G, gh, gw) (``out`` None for reduction "none"); with
    ``head_grad`` False the [V, Ds] head gradient is not formed (gw None).
    """
    Hs, Ws = hs.double(), ws.double()
    Ht, Wt = ht.double(), wt.double()
    if Hs.shape[1] != Ws.shape[1] or Ht.shape[1] != Wt.shape[1]:
        raise ValueError("hidden and head widths differ")
    if Hs.shape[0] != Ht.shape[0] or Ws.shape[0] != Wt.shape[0]:
        raise ValueError("student and teacher disagree on tokens or vocabulary")
    ls = (Hs @ Ws.T).contiguous()
    lt = (Ht @ Wt.T).contiguous()
    ref = jsd_loss(ls, lt, beta, temperature=temperature, scale_t2=scale_t2, mask=mask,
                   reduction=reduction, grad=grad, grads=grads)
    res = dict(out=ref["out"], rows=ref["rows"], G=None, gh=None, gw=None)
    if grads:
        res["G"] = ref["gs"]
        G = torch.from_numpy(ref["gs"])
        res["gh"] = (G @ Ws).numpy()
        if head_grad:
            res["gw"] = (G.T @ Hs).numpy()
    return res
