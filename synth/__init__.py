"""Seeded synthetic workloads for the per-token divergence path.

This module only draws inputs; it holds none of the method's arithmetic, and it
is shared by the tests (GPU path and oracle alike), the smoke check and the
benchmark.  Each workload is drawn with a ``torch.Generator`` seeded with
``1000 + index`` on the device it is asked for, in float32, and then rounded to
the storage dtype (round-to-nearest-even), so the oracle and the GPU path see
exactly the same stored values.

The five workloads (shapes after the pages' op-level benchmarks: DeepSpeed PR
#8958 "[VocabTP] Add vocabulary-parallel generalized JSD with Triton kernels",
section Validation, V = 151936; DeepSpeed PR #8791 "Add vocabulary-parallel
logprobs, entropy and KL ops", section Memory, T = 8192 and V_local = 16032):

  tiny        N=64,    V=1000,   fp32: s ~ N(0, 2^2), t = 0.8 s + N(0, 1.5^2)
  tp8_shard   N=8192,  V=16032,  bf16: as tiny
  full_vocab  N=8192,  V=151936, bf16: s0 ~ N(0, 3^2), t = 0.7 s0 + N(0, 2^2) + b,
              s = s0 + b, with the per-column Zipf log-frequency bias
              b_j = -1.1 ln(j + 1)
  robust      N=4096,  V=128256, fp32, shards 60000/0/40000/28256: as tiny, then
              per row 5% of the teacher's columns (6413, without replacement) set to
              -inf, 1% of rows (41) -inf everywhere in both inputs, and +1e4 added
              to 10% of rows (410) in both inputs
  siblings    N=16384, V=128256, fp16 or bf16: as full_vocab, plus K=20 ids per row
              drawn uniformly without replacement, 10% of all ids set to
              ignore_index (-100)

  linear      N=8192, V=151936, Ds=Dt=3584 (a Qwen2.5-7B-sized hidden width), bf16:
              hidden states and LM-head weights for the fused-linear loss (the
              logits h W^T are never drawn).  Student hidden x ~ N(0, 1) with
              feature 0 fixed at 1; head W_s ~ N(0, (3/sqrt(Ds))^2) with column 0
              the Zipf bias b above, so the student logits are about N(0, 3^2) + b
              as in full_vocab.  Teacher hidden y = 0.7 x + N(0, 0.71^2) (feature 0
              again 1), head W_t = 0.7 W_s + N(0, (2/sqrt(Dt))^2) (column 0 = b);
              with Dt != Ds the shared part uses the first min(Ds, Dt) features.

Upstream per-token gradients are U(0.5, 1.5).  Any workload can be drawn at a
reduced (N, V) with the same recipe for tests the oracle must finish quickly.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

IGNORE_INDEX = -100


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    N: int
    V: int
    dtype: torch.dtype
    recipe: str
    widths: tuple = ()
    betas: tuple = (0.5,)
    K: int = 0

    @property
    def seed(self) -> int:
        return 1000 + self.index


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 0, 64, 1000, torch.float32, "gauss2"),
        Workload("tp8_shard", 1, 8192, 16032, torch.bfloat16, "gauss2"),
        Workload("full_vocab", 2, 8192, 151936, torch.bfloat16, "zipf", betas=(0.1, 0.5, 0.9)),
        Workload("robust", 3, 4096, 128256, torch.float32, "robust",
                 widths=(60000, 0, 40000, 28256)),
        Workload("siblings", 4, 16384, 128256, torch.bfloat16, "zipf", betas=(0.0, 1.0), K=20),
    ]
}


@dataclass
class Batch:
    s: torch.Tensor
    t: torch.Tensor
    gout: torch.Tensor               # [N] float32 upstream per-token gradient
    ids: torch.Tensor | None = None  # [N, K] int64 global ids (siblings)
    gids: torch.Tensor | None = None  # [N, K] float32 upstream gradient of logprobs
    rows_masked: torch.Tensor | None = None  # robust: rows that are -inf everywhere
    rows_offset: torch.Tensor | None = None  # robust: rows carrying the +1e4 offset
    meta: dict = field(default_factory=dict)


def zipf_bias(V: int, device, exponent: float = 1.1) -> torch.Tensor:
    """Per-column log-frequency of a Zipf law with rank = column + 1."""
    j = torch.arange(V, device=device, dtype=torch.float64)
    return (-exponent * torch.log1p(j)).to(torch.float32)


def _normal(gen, shape, std, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def draw(name: str, device="cpu", N: int | None = None, V: int | None = None,
         dtype: torch.dtype | None = None, seed: int | None = None) -> Batch:
    """Draw workload ``name`` (optionally at a reduced N, V or another dtype)."""
    w = WORKLOADS[name]
    N = w.N if N is None else N
    V = w.V if V is None else V
    dtype = w.dtype if dtype is None else dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)

    if w.recipe in ("gauss2", "robust"):
        s = _normal(gen, (N, V), 2.0, device)
        t = 0.8 * s + _normal(gen, (N, V), 1.5, device)
    else:  # zipf
        s0 = _normal(gen, (N, V), 3.0, device)
        t = 0.7 * s0 + _normal(gen, (N, V), 2.0, device)
        b = zipf_bias(V, device)
        s = s0 + b
        t += b
        del s0
    batch = Batch(s=s, t=t, gout=None)

    if w.recipe == "robust":
        n_cols = int(round(0.05 * V))
        if n_cols:
            keys = torch.rand((N, V), generator=gen, device=device)
            cols = keys.topk(n_cols, dim=1).indices
            del keys
            t.scatter_(1, cols, float("-inf"))
        n_masked = int(round(0.01 * N))
        n_off = int(round(0.10 * N))
        perm = torch.randperm(N, generator=gen, device=device)
        rows_masked = perm[:n_masked]
        rows_offset = perm[n_masked:n_masked + n_off]
        s[rows_masked] = float("-inf")
        t[rows_masked] = float("-inf")
        s[rows_offset] += 1e4
        t[rows_offset] += 1e4
        batch.rows_masked = rows_masked.sort().values
        batch.rows_offset = rows_offset.sort().values

    batch.s = s.to(dtype)
    batch.t = t.to(dtype)
    del s, t
    batch.gout = torch.rand((N,), generator=gen, device=device) + 0.5

    if w.K:
        K = min(w.K, V)
        ids = torch.randint(0, V, (N, K), generator=gen, device=device)
        for _ in range(1000):  # redraw rows that hold a repeated id
            srt = ids.sort(dim=1).values
            dup = (srt[:, 1:] == srt[:, :-1]).any(dim=1) if K > 1 else srt[:, 0] < 0
            bad = dup.nonzero().flatten()
            if bad.numel() == 0:
                break
            ids[bad] = torch.randint(0, V, (bad.numel(), K), generator=gen, device=device)
        n_ign = int(round(0.10 * N * K))
        pos = torch.randperm(N * K, generator=gen, device=device)[:n_ign]
        ids.view(-1)[pos] = IGNORE_INDEX
        batch.ids = ids
        batch.gids = torch.rand((N, K), generator=gen, device=device) + 0.5
    batch.meta = dict(name=name, N=N, V=V, dtype=str(dtype).replace("torch.", ""))
    return batch


@dataclass
class LinearBatch:
    hs: torch.Tensor  # [N, Ds] student hidden states
    ws: torch.Tensor  # [V, Ds] student LM-head weight
    ht: torch.Tensor  # [N, Dt] teacher hidden states
    wt: torch.Tensor  # [V, Dt] teacher LM-head weight
    meta: dict = field(default_factory=dict)


LINEAR = dict(N=8192, V=151936, Ds=3584, Dt=3584, seed=1005)


def draw_linear(device="cpu", N: int | None = None, V: int | None = None,
                Ds: int | None = None, Dt: int | None = None, seed: int | None = None,
                dtype: torch.dtype = torch.bfloat16) -> LinearBatch:
    """Hidden states and LM-head weights of the fused-linear workload (module doc)."""
    N = LINEAR["N"] if N is None else N
    V = LINEAR["V"] if V is None else V
    Ds = LINEAR["Ds"] if Ds is None else Ds
    Dt = LINEAR["Dt"] if Dt is None else Dt
    gen = torch.Generator(device=device)
    gen.manual_seed(LINEAR["seed"] if seed is None else seed)
    b = zipf_bias(V, device)
    x = _normal(gen, (N, Ds), 1.0, device)
    x[:, 0] = 1.0
    ws = _normal(gen, (V, Ds), 3.0 / Ds ** 0.5, device)
    ws[:, 0] = b
    d = min(Ds, Dt)
    y = _normal(gen, (N, Dt), 0.71, device)
    y[:, :d] += 0.7 * x[:, :d]
    y[:, 0] = 1.0
    wt = _normal(gen, (V, Dt), 2.0 / Dt ** 0.5, device)
    wt[:, :d] += 0.7 * ws[:, :d]
    wt[:, 0] = b
    return LinearBatch(hs=x.to(dtype), ws=ws.to(dtype), ht=y.to(dtype), wt=wt.to(dtype),
                       meta=dict(name="linear", N=N, V=V, Ds=Ds, Dt=Dt,
                                 dtype=str(dtype).replace("torch.", "")))


def default_split(V: int, parts: int) -> list[int]:
    """Even split of V columns into ``parts`` shards, remainder to the first shards
    (101 over two shards gives 51/50, as in DeepSpeed PR #8309's resume example)."""
    q, r = divmod(V, parts)
    return [q + (1 if k < r else 0) for k in range(parts)]


def bytes_of(N: int, V: int, dtype: torch.dtype) -> int:
    return N * V * torch.empty((), dtype=dtype).element_size()


__all__ = ["WORKLOADS", "Workload", "Batch", "draw", "zipf_bias", "default_split",
           "bytes_of", "IGNORE_INDEX", "LinearBatch", "LINEAR", "draw_linear"]
