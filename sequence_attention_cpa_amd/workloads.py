"""Seeded synthetic workloads for context-parallel attention.

This module only describes shapes and draws random inputs; it holds none of
the attention arithmetic, so both the HIP path and the CPU oracle can be fed
from it.  Shapes follow the pages' workloads: a 64-token toy, the 512-wide
8-head demo model of "Tensor并行与算子拆分", a 7B model (32 heads x 128) at
12k tokens, and one rank's share at 128k (CP=4, 4 heads after TP=8) and 1M
tokens (CP=8) as laid out in "序列与上下文并行" (长上下文的显存账, 工程实践).

Generation recipe (every workload): numpy.random.default_rng(seed) draws Q,
then K, then V as float32 standard normals in global [B, H, L, D] C order;
then, when the workload has outliers, n = round(frac * L) distinct token
indices (Generator.choice without replacement) whose Q and K rows (all heads,
all D) are multiplied by `outlier_mult`; then every tensor is multiplied by
`in_scale`; finally bf16 workloads are rounded to bfloat16 by torch
(round-to-nearest-even).  All multipliers are powers of two, so they are
exact in both float32 and bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    L: int
    N: int
    causal: bool
    dtype: str            # "bf16" or "f32": the element type handed to the kernels
    in_scale: float = 1.0
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    outlier_in_v: bool = False
    seed: int = 0

    @property
    def C(self) -> int:
        """Chunk length L / (2N)."""
        return self.L // (2 * self.N)

    @property
    def Lr(self) -> int:
        """Tokens per rank L / N."""
        return self.L // self.N

    @property
    def n_outliers(self) -> int:
        return int(round(self.outlier_frac * self.L))


WORKLOADS = {
    "tiny": Workload("tiny", B=1, H=2, D=16, L=64, N=4, causal=True, dtype="f32"),
    "demo": Workload("demo", B=16, H=8, D=64, L=128, N=4, causal=False, dtype="bf16",
                     in_scale=0.125),
    "12k": Workload("12k", B=1, H=32, D=128, L=12288, N=4, causal=True, dtype="bf16"),
    "128k": Workload("128k", B=1, H=4, D=128, L=131072, N=4, causal=True, dtype="bf16",
                     outlier_frac=0.01, outlier_mult=8.0),
    # The same share with the outlier rows also applied to V (reported, not gated).
    "128k_qkv": Workload("128k_qkv", B=1, H=4, D=128, L=131072, N=4, causal=True,
                         dtype="bf16", outlier_frac=0.01, outlier_mult=8.0,
                         outlier_in_v=True),
    "1m": Workload("1m", B=1, H=4, D=128, L=1048576, N=8, causal=True, dtype="bf16"),
}


def draw_f32(w: Workload):
    """Q, K, V as float32 numpy arrays [B, H, L, D] plus the sorted outlier
    token indices (int64, possibly empty), before any bf16 rounding."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.H, w.L, w.D)
    Q = rng.standard_normal(shape, dtype=np.float32)
    K = rng.standard_normal(shape, dtype=np.float32)
    V = rng.standard_normal(shape, dtype=np.float32)
    idx = np.zeros(0, dtype=np.int64)
    if w.n_outliers:
        idx = np.sort(rng.choice(w.L, size=w.n_outliers, replace=False)).astype(np.int64)
        mult = np.float32(w.outlier_mult)
        Q[:, :, idx, :] *= mult
        K[:, :, idx, :] *= mult
        if w.outlier_in_v:
            V[:, :, idx, :] *= mult
    if w.in_scale != 1.0:
        s = np.float32(w.in_scale)
        Q *= s
        K *= s
        V *= s
    return Q, K, V, idx


def make_inputs(w: Workload):
    """Q, K, V as CPU torch tensors in the workload's dtype, plus outlier indices.

    bf16 rounding is torch's float32 -> bfloat16 conversion (round to nearest
    even).  The caller moves them to the device and widens them (exactly) to
    float64 for the oracle.
    """
    import torch

    Q, K, V, idx = draw_f32(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = []
    for x in (Q, K, V):
        out.append(torch.from_numpy(x).to(tdt))
    del Q, K, V
    return out[0], out[1], out[2], idx


def make_upstream_grad(w: Workload, seed_offset: int = 1000):
    """dO for a backward pass: standard normal [B, H, L, D] from its own
    generator (seed + seed_offset), in the workload's dtype (bf16 by torch's
    round to nearest even)."""
    import torch

    rng = np.random.default_rng(w.seed + seed_offset)
    g = rng.standard_normal((w.B, w.H, w.L, w.D), dtype=np.float32)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return torch.from_numpy(g).to(tdt)


def sample_rows(w: Workload, rank: int, pos_rank: np.ndarray, n_rows: int,
                outliers: np.ndarray, seed: int = 0) -> np.ndarray:
    """Local row indices of `rank` to check at sizes where every row is too many.

    Picks the first and last row of each of the rank's two chunks, rows at
    128-row tile edges (t mod 128 in {0, 63, 64, 127}) near the chunk ends,
    up to 64 outlier rows that fall in the share, and fills the rest uniformly
    at random (numpy default_rng(seed)).  Returns sorted unique indices.
    """
    C, Lr = w.C, w.Lr
    pick = {0, C - 1, C, Lr - 1}
    for base in (0, C - 128, C, Lr - 128):
        for o in (0, 63, 64, 127):
            t = base + o
            if 0 <= t < Lr:
                pick.add(t)
    if len(outliers):
        where = np.nonzero(np.isin(pos_rank, outliers))[0]
        pick.update(int(t) for t in where[:64])
    rng = np.random.default_rng(seed)
    while len(pick) < min(n_rows, Lr):
        pick.update(int(t) for t in rng.integers(0, Lr, size=n_rows - len(pick)))
    return np.array(sorted(pick), dtype=np.int64)
