"""ctypes binding of libvjsd's C ABI (``include/vjsd.h``): argument marshalling only.

Each function here has the name of the C entry point it calls and takes torch
tensors for the buffers.  Inputs are described by a :class:`ShardSet`, built from
whole ``[N, V]`` / ``[B, T, V]`` tensors split into column shards, or from one
tensor per shard.  All computation happens in the HIP kernels of libvjsd.so; there
is no other code path, and importing this module fails if the library is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvjsd.so")

VJSD_OK = 0
ERRORS = {-1: "ERR_ARG", -2: "ERR_DTYPE", -3: "ERR_BETA", -4: "ERR_LAYOUT",
          -5: "ERR_EMPTY_SHARD", -6: "ERR_HIP"}
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
ROWC_FLOATS = 16  # per-row constants at the head of the workspace
PART_FLOATS = 8  # per (shard, row) partials after them


class VjsdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"vjsd {ERRORS.get(code, code)}: {msg}")
        self.code = code


class VjsdArgumentError(VjsdError, ValueError):
    pass


class View(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
                ("rows_per_batch", ctypes.c_int64), ("batch_stride", ctypes.c_int64)]


class Shard(ctypes.Structure):
    _fields_ = [("vocab_start", ctypes.c_int64), ("width", ctypes.c_int64),
                ("s", View), ("t", View), ("gs", View), ("gt", View)]


class LossOpts(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_double), ("scale_t2", ctypes.c_int),
                ("mask", ctypes.c_void_p), ("reduction", ctypes.c_int)]


REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    SP = ctypes.POINTER(Shard)
    sig = {
        "vjsd_strerror": ([I], ctypes.c_char_p),
        "vjsd_workspace_bytes": ([I64, I], ctypes.c_size_t),
        "vjsd_stats": ([SP, I, I64, I, I, P, P], I),
        "vjsd_merge": ([P, I, I64, I, P, P], I),
        "vjsd_fwd": ([SP, I, I64, I, P, D, P, P, P, P], I),
        "vjsd_forward": ([SP, I, I64, I, D, P, P, P, P, P], I),
        "vjsd_bwd": ([SP, I, I64, I, P, P, D, P, P, P], I),
        "vkl_fwd": ([SP, I, I64, I, I, P, P, P, P, P], I),
        "vkl_bwd": ([SP, I, I64, I, I, P, P, P, P, P], I),
        "ventropy_fwd": ([SP, I, I64, I, P, P, P, P], I),
        "ventropy_bwd": ([SP, I, I64, I, P, P, P, P, P], I),
        "vlogprobs_fwd": ([SP, I, I64, I, I64, P, I, I64, P, P, P, P, P], I),
        "vlogprobs_bwd": ([SP, I, I64, I, I64, P, P, I, I64, P, P, P], I),
        "vtopk_kl_fwd": ([SP, I, I64, I, I64, P, P, I, I64, P, P, P, P, P], I),
        "vce_fwd": ([SP, I, I64, I, I64, P, I64, I, P, P, P, P, P, P], I),
        "vce_bwd": ([SP, I, I64, I, I64, P, P, I64, I, P, P, P], I),
        "vtopk_kl_bwd": ([SP, I, I64, I, I64, P, P, P, I, I64, P, P, P], I),
        "vjsd_membw_probe": ([P, P, ctypes.c_size_t, I, P], I),
        "vjsd_loss_forward": ([SP, I, I64, I, D, ctypes.POINTER(LossOpts), P, P, P, P, P, P], I),
        "vjsd_loss_backward": ([SP, I, I64, I, D, ctypes.POINTER(LossOpts), P, P, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _check(code: int) -> None:
    if code != VJSD_OK:
        msg = lib.vjsd_strerror(code).decode()
        raise (VjsdError if code == -6 else VjsdArgumentError)(code, msg)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require_gpu(x: torch.Tensor, name: str) -> None:
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _ptr(x: torch.Tensor | None, dtype=None, numel=None, name="buffer"):
    if x is None:
        return None
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {x.dtype}")
    _require_gpu(x, name)
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and x.numel() < numel:
        raise ValueError(f"{name} holds {x.numel()} elements, needs {numel}")
    return x.data_ptr() if x.numel() else None


def _view(x: torch.Tensor | None) -> tuple[View, int]:
    """View of a [N, w] or [B, T, w] tensor with unit column stride; returns (view, N)."""
    if x is None:
        return View(None, 0, 0, 0), -1
    _require_gpu(x, "logits and gradients")
    w = x.shape[-1]
    if x.dim() == 2:
        rs = x.stride(0)
        if w > 1 and x.stride(1) != 1:
            raise ValueError("the vocabulary dimension must have unit stride")
        return View(x.data_ptr() if x.numel() else None, rs, 0, 0), x.shape[0]
    if x.dim() == 3:
        if w > 1 and x.stride(2) != 1:
            raise ValueError("the vocabulary dimension must have unit stride")
        return (View(x.data_ptr() if x.numel() else None, x.stride(1), x.shape[1], x.stride(0)),
                x.shape[0] * x.shape[1])
    raise ValueError("logits must be [N, V] or [B, T, V]")


class ShardSet:
    """The S logical vocabulary shards of one call, as the C ABI sees them.

    ``s``/``t``/``gs``/``gt`` are each either one tensor ``[..., V]`` split by
    ``widths`` into column slices (default: a single shard), or a sequence of
    per-shard tensors ``[..., V_k]``.  ``t``, ``gs`` and ``gt`` may be None.
    """

    def __init__(self, s, t=None, *, widths=None, gs=None, gt=None, vocab_start=0):
        def split(x):
            if x is None:
                return None
            if isinstance(x, (list, tuple)):
                return list(x)
            ws = [x.shape[-1]] if widths is None else list(widths)
            if sum(ws) != x.shape[-1] or any(w < 0 for w in ws):
                raise ValueError("shard widths must be >= 0 and sum to the vocabulary size")
            out, c = [], 0
            for w in ws:
                out.append(x[..., c:c + w])
                c += w
            return out

        ss, ts, gss, gts = split(s), split(t), split(gs), split(gt)
        S = len(ss)
        for other in (ts, gss, gts):
            if other is not None and len(other) != S:
                raise ValueError("all inputs must have the same number of shards")
        dt = ss[0].dtype
        if dt not in DTYPES:
            raise ValueError(f"unsupported logits dtype {dt}")
        for group in (ss, ts, gss, gts):
            for x in group or []:
                if x.dtype != dt:
                    raise ValueError("student, teacher and gradients must share one dtype")
        self.S = S
        self.dtype = dt
        self.dtype_code = DTYPES[dt]
        self.widths = [x.shape[-1] for x in ss]
        self.V = sum(self.widths)
        self.arr = (Shard * S)()
        self.keep = [ss, ts, gss, gts]
        N = None
        start = vocab_start
        for k in range(S):
            vs, n = _view(ss[k])
            vt, nt = _view(ts[k] if ts else None)
            vgs, ng = _view(gss[k] if gss else None)
            vgt, ngt = _view(gts[k] if gts else None)
            for name, x in (("teacher", ts), ("student grad", gss), ("teacher grad", gts)):
                if x is not None and x[k].shape != ss[k].shape:
                    raise ValueError(f"{name} shard {k} shape {tuple(x[k].shape)} != "
                                     f"student shard shape {tuple(ss[k].shape)}")
            N = n if N is None else N
            if n != N:
                raise ValueError("all shards must hold the same rows")
            self.arr[k] = Shard(start, ss[k].shape[-1], vs, vt, vgs, vgt)
            start += ss[k].shape[-1]
        self.N = N
        self.lead_shape = tuple(ss[0].shape[:-1])


def vjsd_strerror(code: int) -> str:
    return lib.vjsd_strerror(code).decode()


def vjsd_workspace_bytes(N: int, S: int) -> int:
    return lib.vjsd_workspace_bytes(N, S)


def vjsd_membw_probe(src: torch.Tensor, dst: torch.Tensor, op: int, stream=None) -> None:
    """Streaming read (op 0) of all of `src`, or copy (op 1) of `src` into `dst`."""
    for x, name in ((src, "src"), (dst, "dst")):
        _require_gpu(x, name)
        if not x.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    nbytes = src.numel() * src.element_size()
    if op == 1 and dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst is smaller than src")
    _check(lib.vjsd_membw_probe(src.data_ptr(), dst.data_ptr(), nbytes, op, _stream(stream)))


def part_floats(N: int, S: int) -> int:
    """Floats of the workspace: vjsd_workspace_bytes(N, S) / 4."""
    return (lib.vjsd_workspace_bytes(N, S) + 3) // 4 if N > 0 and S > 0 else 0


def new_part(N: int, S: int, device) -> torch.Tensor:
    """Workspace of vjsd_workspace_bytes(N, S) bytes."""
    return torch.empty(max(1, part_floats(N, S)), dtype=torch.float32, device=device)


def vjsd_stats(sh: ShardSet, which: int, part, stream=None) -> None:
    _check(lib.vjsd_stats(sh.arr, sh.S, sh.N, sh.dtype_code, which,
                          _ptr(part, torch.float32, part_floats(sh.N, sh.S), "part"),
                          _stream(stream)))


def vjsd_merge(part, S: int, N: int, which: int, stats, stream=None) -> None:
    _check(lib.vjsd_merge(_ptr(part, torch.float32, part_floats(N, S), "part"), S, N, which,
                          _ptr(stats, torch.float64, N * 4, "stats"), _stream(stream)))


def vjsd_fwd(sh: ShardSet, stats, beta: float, part, kl, loss, stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_fwd(sh.arr, sh.S, N, sh.dtype_code, _ptr(stats, torch.float64, N * 4, "stats"),
                        float(beta), _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                        _ptr(kl, torch.float32, N * 2, "kl"), _ptr(loss, torch.float32, N, "loss"),
                        _stream(stream)))


def vjsd_forward(sh: ShardSet, beta: float, part, stats, kl, loss, stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_forward(sh.arr, sh.S, N, sh.dtype_code, float(beta),
                            _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                            _ptr(stats, torch.float64, N * 4, "stats"),
                            _ptr(kl, torch.float32, N * 2, "kl"),
                            _ptr(loss, torch.float32, N, "loss"), _stream(stream)))


def vjsd_bwd(sh: ShardSet, stats, kl, beta: float, grad_loss, part, stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_bwd(sh.arr, sh.S, N, sh.dtype_code, _ptr(stats, torch.float64, N * 4, "stats"),
                        _ptr(kl, torch.float32, N * 2, "kl"), float(beta),
                        _ptr(grad_loss, torch.float32, N, "grad_loss"),
                        _ptr(part, torch.float32, part_floats(N, sh.S), "part"), _stream(stream)))


def loss_opts(N: int, temperature: float = 1.0, scale_t2: bool = False, mask=None,
              reduction: str = "none") -> LossOpts:
    """The C options of the distillation-loss entry points; ``mask`` is a GPU uint8 [N]
    tensor (nonzero = the token counts) or None."""
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    mp = _ptr(mask, torch.uint8, N, "mask") if mask is not None else None
    return LossOpts(float(temperature), int(bool(scale_t2)), mp, REDUCTIONS[reduction])


def vjsd_loss_forward(sh: ShardSet, beta: float, opts: LossOpts, part, stats, kl, rows,
                      out=None, stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_loss_forward(sh.arr, sh.S, N, sh.dtype_code, float(beta), ctypes.byref(opts),
                                 _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                                 _ptr(stats, torch.float64, N * 4, "stats"),
                                 _ptr(kl, torch.float32, N * 2, "kl"),
                                 _ptr(rows, torch.float32, N, "rows"),
                                 _ptr(out, torch.float32, 1, "out"), _stream(stream)))


def vjsd_loss_backward(sh: ShardSet, beta: float, opts: LossOpts, stats, kl, grad, part,
                       stream=None) -> None:
    N = sh.N
    ng = N if opts.reduction == 0 else 1
    _check(lib.vjsd_loss_backward(sh.arr, sh.S, N, sh.dtype_code, float(beta), ctypes.byref(opts),
                                  _ptr(stats, torch.float64, N * 4, "stats"),
                                  _ptr(kl, torch.float32, N * 2, "kl"),
                                  _ptr(grad, torch.float32, ng, "grad"),
                                  _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                                  _stream(stream)))


def vkl_fwd(sh: ShardSet, reverse: bool, part, stats, kl, loss, stream=None) -> None:
    N = sh.N
    _check(lib.vkl_fwd(sh.arr, sh.S, N, sh.dtype_code, int(bool(reverse)),
                       _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                       _ptr(stats, torch.float64, N * 4, "stats"),
                       _ptr(kl, torch.float32, N * 2, "kl"), _ptr(loss, torch.float32, N, "loss"),
                       _stream(stream)))


def vkl_bwd(sh: ShardSet, reverse: bool, stats, kl, grad_loss, part, stream=None) -> None:
    N = sh.N
    _check(lib.vkl_bwd(sh.arr, sh.S, N, sh.dtype_code, int(bool(reverse)),
                       _ptr(stats, torch.float64, N * 4, "stats"),
                       _ptr(kl, torch.float32, N * 2, "kl"),
                       _ptr(grad_loss, torch.float32, N, "grad_loss"),
                       _ptr(part, torch.float32, part_floats(N, sh.S), "part"), _stream(stream)))


def ventropy_fwd(sh: ShardSet, part, stats, ent, stream=None) -> None:
    N = sh.N
    _check(lib.ventropy_fwd(sh.arr, sh.S, N, sh.dtype_code,
                            _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                            _ptr(stats, torch.float64, N * 4, "stats"),
                            _ptr(ent, torch.float32, N, "ent"), _stream(stream)))


def ventropy_bwd(sh: ShardSet, stats, ent, grad, part, stream=None) -> None:
    N = sh.N
    _check(lib.ventropy_bwd(sh.arr, sh.S, N, sh.dtype_code,
                            _ptr(stats, torch.float64, N * 4, "stats"),
                            _ptr(ent, torch.float32, N, "ent"),
                            _ptr(grad, torch.float32, N, "grad"),
                            _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                            _stream(stream)))


def vlogprobs_fwd(sh: ShardSet, vocab_global: int, ids, ignore_index: int, part, stats, out,
                  dev_err, stream=None) -> None:
    N = sh.N
    K = ids.shape[-1] if ids is not None and ids.dim() else 0
    _check(lib.vlogprobs_fwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                             _ptr(ids, torch.int64, N * K, "ids"), K, int(ignore_index),
                             _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                             _ptr(stats, torch.float64, N * 4, "stats"),
                             _ptr(out, torch.float32, N * K, "out"),
                             _ptr(dev_err, torch.int32, 1, "dev_err"), _stream(stream)))


def vce_fwd(sh: ShardSet, vocab_global: int, labels, ignore_index: int, reduction: str, part,
            stats, rows, out, dev_err, stream=None) -> None:
    N = sh.N
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    _check(lib.vce_fwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                       _ptr(labels, torch.int64, N, "labels"), int(ignore_index),
                       REDUCTIONS[reduction],
                       _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                       _ptr(stats, torch.float64, N * 4, "stats"),
                       _ptr(rows, torch.float32, N, "rows"), _ptr(out, torch.float32, 1, "out"),
                       _ptr(dev_err, torch.int32, 1, "dev_err"), _stream(stream)))


def vce_bwd(sh: ShardSet, vocab_global: int, stats, labels, ignore_index: int, reduction: str,
            grad, part, stream=None) -> None:
    N = sh.N
    if reduction not in REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(REDUCTIONS)}")
    _check(lib.vce_bwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                       _ptr(stats, torch.float64, N * 4, "stats"),
                       _ptr(labels, torch.int64, N, "labels"), int(ignore_index),
                       REDUCTIONS[reduction],
                       _ptr(grad, torch.float32, N if reduction == "none" else 1, "grad"),
                       _ptr(part, torch.float32, part_floats(N, sh.S), "part"), _stream(stream)))


def vtopk_kl_fwd(sh: ShardSet, vocab_global: int, ids, tlogp, ignore_index: int, part, stats,
                 kl, dev_err, stream=None) -> None:
    N = sh.N
    K = ids.shape[-1] if ids is not None and ids.dim() else 0
    _check(lib.vtopk_kl_fwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                            _ptr(ids, torch.int64, N * K, "ids"),
                            _ptr(tlogp, torch.float32, N * K, "tlogp"), K, int(ignore_index),
                            _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                            _ptr(stats, torch.float64, N * 4, "stats"),
                            _ptr(kl, torch.float32, N, "kl"),
                            _ptr(dev_err, torch.int32, 1, "dev_err"), _stream(stream)))


def vtopk_kl_bwd(sh: ShardSet, vocab_global: int, stats, ids, tlogp, ignore_index: int, grad,
                 part, stream=None) -> None:
    N = sh.N
    K = ids.shape[-1] if ids is not None and ids.dim() else 0
    _check(lib.vtopk_kl_bwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                            _ptr(stats, torch.float64, N * 4, "stats"),
                            _ptr(ids, torch.int64, N * K, "ids"),
                            _ptr(tlogp, torch.float32, N * K, "tlogp"), K, int(ignore_index),
                            _ptr(grad, torch.float32, N, "grad"),
                            _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                            _stream(stream)))


def vlogprobs_bwd(sh: ShardSet, vocab_global: int, stats, ids, ignore_index: int, grad, part,
                  stream=None) -> None:
    N = sh.N
    K = ids.shape[-1] if ids is not None and ids.dim() else 0
    _check(lib.vlogprobs_bwd(sh.arr, sh.S, N, sh.dtype_code, int(vocab_global),
                             _ptr(stats, torch.float64, N * 4, "stats"),
                             _ptr(ids, torch.int64, N * K, "ids"), K, int(ignore_index),
                             _ptr(grad, torch.float32, N * K, "grad"),
                             _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                             _stream(stream)))
