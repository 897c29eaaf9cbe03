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
# VJSD_LIB points the loader at another build of the same sources (the host-sanitizer
# build that the CPU tests load); by default the in-tree library.
LIB_PATH = os.environ.get("VJSD_LIB") or os.path.join(_HERE, "libvjsd.so")

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


class LinOperand(ctypes.Structure):
    _fields_ = [("p", ctypes.c_void_p), ("ld", ctypes.c_int64), ("dtype", ctypes.c_int),
                ("kmajor", ctypes.c_int)]


class LinHead(ctypes.Structure):
    _fields_ = [("h", ctypes.c_void_p), ("ldh", ctypes.c_int64), ("w", ctypes.c_void_p),
                ("ldw", ctypes.c_int64), ("dim", ctypes.c_int64)]


REDUCTIONS = {"none": 0, "sum": 1, "mean": 2}
LIN_OUT = {"f32": 0, "f32_acc": 1, "bf16": 2}


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
        "vjsd_bwd_noalloc": ([SP, I, I64, I, P, P, D, P, P], I),
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
        "vjsd_forward_backward": ([SP, I, I64, I, D, P, P, P, P, P, P], I),
        "vjsd_loss_forward_backward": ([SP, I, I64, I, D, ctypes.POINTER(LossOpts), P, P, P, P,
                                        P, P, P], I),
        "vlin_gemm": ([I64, I64, I64, LinOperand, LinOperand, P, I64, I, P], I),
        "vljsd_workspace_bytes": ([I64, I64, I64, I64, I64], ctypes.c_size_t),
        "vljsd": ([ctypes.POINTER(LinHead), ctypes.POINTER(LinHead), I64, I64, D,
                   ctypes.POINTER(LossOpts), I64, I64, P, P, P, I64, P, I64, P], I),
        "vlin_scale": ([P, I64, I, P, P], I),
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


def vjsd_bwd_noalloc(sh: ShardSet, stats, kl, beta: float, grad_loss, stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_bwd_noalloc(sh.arr, sh.S, N, sh.dtype_code,
                                _ptr(stats, torch.float64, N * 4, "stats"),
                                _ptr(kl, torch.float32, N * 2, "kl"), float(beta),
                                _ptr(grad_loss, torch.float32, N, "grad_loss"), _stream(stream)))


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


def vjsd_forward_backward(sh: ShardSet, beta: float, grad_loss, part, stats, kl, loss,
                          stream=None) -> None:
    N = sh.N
    _check(lib.vjsd_forward_backward(sh.arr, sh.S, N, sh.dtype_code, float(beta),
                                     _ptr(grad_loss, torch.float32, N, "grad_loss"),
                                     _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                                     _ptr(stats, torch.float64, N * 4, "stats"),
                                     _ptr(kl, torch.float32, N * 2, "kl"),
                                     _ptr(loss, torch.float32, N, "loss"), _stream(stream)))


def vjsd_loss_forward_backward(sh: ShardSet, beta: float, opts: LossOpts, grad, part, stats, kl,
                               rows, out=None, stream=None) -> None:
    N = sh.N
    ng = N if opts.reduction == 0 else 1
    _check(lib.vjsd_loss_forward_backward(sh.arr, sh.S, N, sh.dtype_code, float(beta),
                                          ctypes.byref(opts), _ptr(grad, torch.float32, ng, "grad"),
                                          _ptr(part, torch.float32, part_floats(N, sh.S), "part"),
                                          _ptr(stats, torch.float64, N * 4, "stats"),
                                          _ptr(kl, torch.float32, N * 2, "kl"),
                                          _ptr(rows, torch.float32, N, "rows"),
                                          _ptr(out, torch.float32, 1, "out"), _stream(stream)))


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


# ---- fused linear + JSD ----------------------------------------------------------------

def _matrix(x: torch.Tensor, name: str) -> None:
    _require_gpu(x, name)
    if x.dim() != 2 or (x.shape[1] > 1 and x.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")


def lin_operand(x: torch.Tensor, kmajor: bool, name: str = "operand") -> LinOperand:
    """Operand of vlin_gemm from a 2-D tensor with unit column stride: rows of x are the
    operand's rows (kmajor) or its k index (not kmajor)."""
    _matrix(x, name)
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"{name} must be bfloat16 or float32")
    q = 4 if x.dtype == torch.float32 else 8
    # a single row's stride is never used: any multiple of q covering the row will do
    ld = x.stride(0) if x.shape[0] > 1 else -(-max(x.shape[1], 1) // q) * q
    _whole_rows(x, ld, name)
    return LinOperand(x.data_ptr() if x.numel() else None, ld, DTYPES[x.dtype], int(kmajor))


def _whole_rows(x: torch.Tensor, ld: int, name: str) -> None:
    """The products read whole rows of ld elements: the storage must hold them."""
    if x.numel() == 0:
        return
    have = x.untyped_storage().nbytes() // x.element_size() - x.storage_offset()
    if have < x.shape[0] * ld:
        raise ValueError(f"{name}: the storage must extend over whole rows of {ld} elements "
                         f"(pad the last row, or pass a tensor whose row stride is a multiple "
                         f"of {16 // x.element_size()})")


def vlin_gemm(M: int, N: int, K: int, a: LinOperand, b: LinOperand, c: torch.Tensor,
              out: str = "f32", stream=None) -> None:
    """C[i][j] (+)= sum_k A(i, k) B(j, k) into the 2-D tensor c (row stride >= N)."""
    if out not in LIN_OUT:
        raise ValueError(f"out must be one of {sorted(LIN_OUT)}")
    _matrix(c, "c")
    want = torch.bfloat16 if out == "bf16" else torch.float32
    if c.dtype != want:
        raise ValueError(f"c must be {want} for out={out!r}")
    if c.shape[0] < M or c.shape[1] < N:
        raise ValueError("c is smaller than M x N")
    ldc = c.stride(0) if c.shape[0] > 1 else max(c.shape[1], 1)
    _check(lib.vlin_gemm(M, N, K, a, b, c.data_ptr() if c.numel() else None, ldc, LIN_OUT[out],
                         _stream(stream)))


def lin_head(h: torch.Tensor, w: torch.Tensor, name: str) -> LinHead:
    """One side of the fused-linear loss: hidden [N, dim] and head weight [V, dim], bf16."""
    for x, nm in ((h, f"{name} hidden"), (w, f"{name} head")):
        _matrix(x, nm)
        if x.dtype != torch.bfloat16:
            raise ValueError(f"{nm} must be bfloat16")
    if h.shape[1] != w.shape[1]:
        raise ValueError(f"{name} hidden and head widths differ")
    ldh = h.stride(0) if h.shape[0] > 1 else -(-max(h.shape[1], 1) // 8) * 8
    ldw = w.stride(0) if w.shape[0] > 1 else -(-max(w.shape[1], 1) // 8) * 8
    _whole_rows(h, ldh, f"{name} hidden")
    _whole_rows(w, ldw, f"{name} head")
    return LinHead(h.data_ptr() if h.numel() else None, ldh, w.data_ptr(), ldw, w.shape[1])


def vljsd_workspace_bytes(N: int, V: int, dim_s: int, chunk: int, group: int = 0) -> int:
    return lib.vljsd_workspace_bytes(N, V, dim_s, chunk, group)


def vljsd(student: LinHead, teacher: LinHead, N: int, V: int, beta: float, opts: LossOpts,
          chunk: int, workspace, out, grad_h=None, grad_w=None, stream=None,
          group: int = 0) -> None:
    nout = N if opts.reduction == 0 else 1
    ws = _ptr(workspace, torch.uint8, vljsd_workspace_bytes(N, V, student.dim, chunk, group),
              "workspace")
    gh = gw = None
    ldgh = ldgw = 0
    if grad_h is not None:
        _matrix(grad_h, "grad_h")
        if grad_h.dtype != torch.bfloat16 or grad_h.shape[0] < N:
            raise ValueError("grad_h must be bfloat16 [N, dim_s]")
        gh = grad_h.data_ptr() if grad_h.numel() else None
        ldgh = grad_h.stride(0) if grad_h.shape[0] > 1 else grad_h.shape[1]
    if grad_w is not None:
        _matrix(grad_w, "grad_w")
        if grad_w.dtype != torch.bfloat16 or grad_w.shape[0] < V:
            raise ValueError("grad_w must be bfloat16 [V, dim_s]")
        gw = grad_w.data_ptr()
        ldgw = grad_w.stride(0) if grad_w.shape[0] > 1 else grad_w.shape[1]
    _check(lib.vljsd(ctypes.byref(student), ctypes.byref(teacher), N, V, float(beta),
                     ctypes.byref(opts), int(chunk), int(group), ws,
                     _ptr(out, torch.float32, nout, "out"), gh, ldgh, gw, ldgw, _stream(stream)))


def vlin_scale(x: torch.Tensor, g: torch.Tensor, stream=None) -> None:
    """x *= g[0] in place (x contiguous fp32, fp16 or bf16, g a GPU float32 scalar)."""
    if x.dtype not in DTYPES:
        raise ValueError("x must be float32, float16 or bfloat16")
    _check(lib.vlin_scale(_ptr(x, name="x"), x.numel(), DTYPES[x.dtype],
                          _ptr(g, torch.float32, 1, "g"), _stream(stream)))
