"""Seeded synthetic inputs for MoE dispatch / combine workloads.

This module only draws inputs: token activations ``x`` (bf16 bit patterns),
routing ``topk_idx`` and routing weights.  It holds none of the dispatch /
combine arithmetic and is shared, unchanged, by the HIP path, the tests and
the CPU oracle so that both sides see bit-identical inputs.

Recipe (one NumPy ``PCG64`` stream per config, split with ``SeedSequence``
into independent sub-streams for x, routing, weights and structure):

* x: fp32 N(0, 1) rounded to bf16 (round-to-nearest-even).  The skewed
  training shape scales 1% of the channels (a seeded choice) by 50 before
  rounding, as outlier channels.
* routing: top-K distinct experts per token by Gumbel-top-K (sampling
  without replacement from the expert popularity p): key_e = log p_e +
  Gumbel(0, 1), the K largest keys in descending order.  Uniform: p = 1/E.
  Zipf(alpha): a seeded permutation pi of the experts, p_{pi[i]} ~ (i+1)^-alpha.
* weights: softmax over K of fp32 N(0, 1) logits per token.

The shapes are DeepSeek-V3-like MoE layers (hidden 7168, 256 experts,
top-8) on 2..64 simulated ranks; no router trace is available, so Zipf
popularity stands in for the skew of a trained router.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

MODE_NORMAL, MODE_LL, MODE_MSG, MODE_RANK = 0, 1, 2, 3
Q_NONE, Q_FP8_F32, Q_FP8_UE8M0 = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    name: str
    R: int
    T: int
    H: int
    E: int
    K: int
    mode: int
    quant: int
    routing: str = "uniform"      # "uniform" | "zipf"
    alpha: float = 0.0
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    align: int = 1
    region_bytes: int = 2 << 20
    epoch: int = 1
    seed: int = 0
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def N(self) -> int:
        return self.R * self.T

    @property
    def L(self) -> int:
        return self.E // self.R

    @property
    def G(self) -> int:
        return self.H // 128

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


SEED_BASE = 20261200

WORKLOADS = {
    "tiny": Workload("tiny", R=2, T=8, H=128, E=8, K=2, mode=MODE_NORMAL, quant=Q_NONE,
                     seed=SEED_BASE + 1),
    "ll_decode": Workload("ll_decode", R=8, T=128, H=7168, E=256, K=8, mode=MODE_LL,
                          quant=Q_FP8_F32, seed=SEED_BASE + 2),
    "normal_prefill": Workload("normal_prefill", R=8, T=4096, H=7168, E=256, K=8,
                               mode=MODE_NORMAL, quant=Q_NONE, routing="zipf", alpha=1.2,
                               seed=SEED_BASE + 3),
    "fp8_train": Workload("fp8_train", R=16, T=8192, H=4096, E=128, K=8, mode=MODE_NORMAL,
                          quant=Q_FP8_UE8M0, routing="zipf", alpha=1.0, outlier_frac=0.01,
                          outlier_scale=50.0, seed=SEED_BASE + 4),
    "messages": Workload("messages", R=64, T=256, H=7168, E=256, K=8, mode=MODE_MSG,
                         quant=Q_FP8_F32, seed=SEED_BASE + 5),
    # the prefill routing in the rank-major (V1) receive layout
    "rank_prefill": Workload("rank_prefill", R=8, T=4096, H=7168, E=256, K=8, mode=MODE_RANK,
                             quant=Q_NONE, routing="zipf", alpha=1.2, seed=SEED_BASE + 3),
}
ORDER = ["tiny", "ll_decode", "normal_prefill", "fp8_train", "messages", "rank_prefill"]


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(4)]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the 16-bit patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gen_x(w: Workload) -> np.ndarray:
    """bf16 bit patterns [R][T][H]."""
    rx, _, _, rs = _streams(w.seed)
    n = w.N
    out = np.empty((n, w.H), np.uint16)
    cols = None
    if w.outlier_frac > 0:
        nout = int(round(w.outlier_frac * w.H))
        cols = rs.choice(w.H, size=nout, replace=False)
    chunk = max(1, (1 << 22) // w.H)
    buf = np.empty((chunk, w.H), np.float32)
    for i in range(0, n, chunk):
        j = min(n, i + chunk)
        a = buf[: j - i]
        rx.standard_normal(out=a, dtype=np.float32)
        if cols is not None:
            a[:, cols] *= np.float32(w.outlier_scale)
        out[i:j] = f32_to_bf16_bits(a)
    out = out.reshape(w.R, w.T, w.H)
    return out


def popularity(w: Workload) -> np.ndarray:
    _, _, _, rs = _streams(w.seed)
    if w.outlier_frac > 0:  # keep the structure stream order fixed
        rs.choice(w.H, size=int(round(w.outlier_frac * w.H)), replace=False)
    if w.routing == "uniform":
        return np.full(w.E, 1.0 / w.E)
    perm = rs.permutation(w.E)
    p = np.empty(w.E)
    p[perm] = (np.arange(1, w.E + 1, dtype=np.float64)) ** (-w.alpha)
    return p / p.sum()


def gen_topk(w: Workload) -> np.ndarray:
    """int32 [R][T][K]: K distinct experts per token (Gumbel-top-K)."""
    _, rr, _, _ = _streams(w.seed)
    logp = np.log(popularity(w))
    out = np.empty((w.N, w.K), np.int32)
    chunk = max(1, (1 << 22) // w.E)
    for i in range(0, w.N, chunk):
        j = min(w.N, i + chunk)
        keys = logp[None, :] + rr.gumbel(size=(j - i, w.E))
        part = np.argpartition(-keys, w.K - 1, axis=1)[:, : w.K]
        pk = np.take_along_axis(keys, part, axis=1)
        order = np.argsort(-pk, axis=1, kind="stable")
        out[i:j] = np.take_along_axis(part, order, axis=1)
    return out.reshape(w.R, w.T, w.K)


def gen_weights(w: Workload) -> np.ndarray:
    """float32 [R][T][K]: softmax over k of N(0,1) logits."""
    _, _, rw, _ = _streams(w.seed)
    z = rw.standard_normal((w.N, w.K), dtype=np.float32)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32).reshape(w.R, w.T, w.K)


def gen_y(w: Workload, rows: int, seed_offset: int = 0) -> np.ndarray:
    """Independent N(0,1) bf16 rows [rows][H], standing in for expert outputs."""
    g = np.random.Generator(np.random.PCG64(w.seed + 7919 * (1 + seed_offset)))
    out = np.empty((rows, w.H), np.uint16)
    chunk = max(1, (1 << 24) // w.H)
    for i in range(0, rows, chunk):
        j = min(rows, i + chunk)
        out[i:j] = f32_to_bf16_bits(g.standard_normal((j - i, w.H), dtype=np.float32))
    return out


def small(name: str = "custom", *, R: int, T: int, H: int, E: int, K: int,
          mode: int = MODE_NORMAL, quant: int = Q_NONE, seed: int = 1, **kw) -> Workload:
    """A small workload with the same recipe, for parity sweeps."""
    return Workload(name, R=R, T=T, H=H, E=E, K=K, mode=mode, quant=quant, seed=seed, **kw)


def masked_topk(w: Workload, topk: np.ndarray, frac: float, dup_frac: float = 0.0,
                seed: int = 99) -> np.ndarray:
    """Edge-case routing: set a fraction of entries to -1 (no expert) and
    copy a fraction of entries from the previous k (duplicate ids)."""
    g = np.random.Generator(np.random.PCG64(w.seed + seed))
    t = topk.copy()
    m = g.random(t.shape) < frac
    t[m] = -1
    if dup_frac > 0 and t.shape[-1] > 1:
        d = g.random(t.shape) < dup_frac
        d[..., 0] = False
        src = np.roll(t, 1, axis=-1)
        t[d] = src[d]
    return t.astype(np.int32)
