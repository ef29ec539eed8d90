"""One pass of the hot path for a set of virtual ranks, built from library calls.

For ranks [rank_lo, rank_hi) of an N-way zigzag split of a [B, H, L, D]
sequence: permute K and V into rank-major order (every rank's K/V is needed by
the ring), permute the ranks' Q, run each rank's ring (N partials, N-1
merges), and scatter the ranks' O and lse back to global token order.  On one
GPU the other ranks' K/V shares are slices of the same buffers, so the ring
needs no communication.

With `fused=True` each rank's ring is one launch (cpa_rank_forward_fused:
the online-softmax state stays in registers across the N blocks) instead of
N partial launches and N-1 merges; bf16 with D = 64 or 128 only.

With `global_layout=True` the whole step is one cpa_share_forward call per
rank: the kernel reads global-order Q/K/V and writes global-order O/lse,
with the zigzag permute folded into its addressing (bf16, D = 64 or 128,
chunks L/(2N) a multiple of 32).

With `rope_base` set, Q and K are rotated at their global positions: on the
way into rank-major order (cpa_zigzag_permute_rope: the rotary embedding is
folded into the permute, so it costs no extra pass over memory), or, in
global-layout mode, by cpa_rope into rotated global-order copies (positions
0 .. L-1) that the ring then reads.

`backward(dO)` runs the ring backward of the ranks after a `step`: dO is
permuted like Q, each rank's cpa_rank_backward writes its dQ and adds its
contributions to every block's dK / dV (rank-major float32 accumulators,
cleared first), and the gradients are scattered back to global order.  In
global-layout mode it is one cpa_share_backward call per rank on the
global-order tensors instead (no permutes).  With RoPE the returned dQ, dK
are gradients with respect to the rotated Q, K.

All buffers are allocated once in the constructor (the backward's on first
use); `step` and `backward` allocate nothing after that.  The global-layout
mode allocates no rank-major buffers: only O, lse and (for the backward) the
global-order gradients and delta.
"""
from __future__ import annotations

from . import (CPA_ROPE_INTERLEAVED, rank_backward, rank_forward, rank_forward_fused,
               rank_forward_workspace, rope, share_backward, share_forward, zigzag_layout,
               zigzag_permute, zigzag_permute_rope)


class SharePipeline:
    def __init__(self, B: int, H: int, L: int, D: int, N: int, causal: bool, dtype, device,
                 rank_lo: int = 0, rank_hi: int | None = None, scale: float = 0.0,
                 fused: bool = False, rope_base: float | None = None,
                 rope_pairing: int = CPA_ROPE_INTERLEAVED, global_layout: bool = False):
        import torch

        self.B, self.H, self.L, self.D, self.N = B, H, L, D, N
        self.causal, self.scale, self.fused = causal, scale, fused
        self.rope_base, self.rope_pairing = rope_base, rope_pairing
        self.global_layout = global_layout
        self.rank_lo = rank_lo
        self.rank_hi = N if rank_hi is None else rank_hi
        nr = self.rank_hi - self.rank_lo
        Lr = L // N
        self.device = device
        self.pos_host = zigzag_layout(L, N)
        self.pos = self.pos_host.to(device)
        if not global_layout:
            self.Kr = torch.empty((N, B, H, Lr, D), dtype=dtype, device=device)
            self.Vr = torch.empty_like(self.Kr)
            self.Qr = torch.empty((nr, B, H, Lr, D), dtype=dtype, device=device)
            self.Or = torch.empty((nr, B, H, Lr, D), dtype=torch.float32, device=device)
            self.lser = torch.empty((nr, B, H, Lr), dtype=torch.float32, device=device)
            ws_bytes = 1 if fused else max(rank_forward_workspace(B, H, L, N, D), 1)
            self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        elif rope_base is not None:
            self.pos_glob = torch.arange(L, dtype=torch.int64, device=device)
            self.Qrot = torch.empty((B, H, L, D), dtype=dtype, device=device)
            self.Krot = torch.empty_like(self.Qrot)
        self.O = torch.zeros((B, H, L, D), dtype=torch.float32, device=device)
        self.lse = torch.full((B, H, L), float("-inf"), dtype=torch.float32, device=device)

    def step(self, Q, K, V):
        """Q, K, V: global [B, H, L, D] on the device.  Returns global (O, lse);
        rows of ranks outside [rank_lo, rank_hi) are left as initialised."""
        N, lo, hi = self.N, self.rank_lo, self.rank_hi
        if self.global_layout:
            if self.rope_base is not None:
                rope(Q, self.pos_glob, self.rope_base, self.rope_pairing, out=self.Qrot)
                rope(K, self.pos_glob, self.rope_base, self.rope_pairing, out=self.Krot)
                Q, K = self.Qrot, self.Krot
            self._inputs = (Q, K, V)
            share_forward(Q, K, V, N, self.causal, self.scale, lo, hi, out=self.O, lse=self.lse)
            return self.O, self.lse
        if self.rope_base is None:
            zigzag_permute(K, self.pos, N, out=self.Kr)
            zigzag_permute(Q, self.pos, N, rank_lo=lo, rank_hi=hi, out=self.Qr)
        else:
            zigzag_permute_rope(K, self.pos, N, self.rope_base, self.rope_pairing, out=self.Kr)
            zigzag_permute_rope(Q, self.pos, N, self.rope_base, self.rope_pairing, rank_lo=lo,
                                rank_hi=hi, out=self.Qr)
        zigzag_permute(V, self.pos, N, out=self.Vr)
        self.ring()
        zigzag_permute(self.Or, self.pos, N, inverse=True, rank_lo=lo, rank_hi=hi, out=self.O)
        zigzag_permute(self.lser, self.pos, N, inverse=True, rank_lo=lo, rank_hi=hi, out=self.lse)
        return self.O, self.lse

    def ring(self):
        """The ring part only (inputs already rank-major)."""
        for k, i in enumerate(range(self.rank_lo, self.rank_hi)):
            if self.fused:
                rank_forward_fused(i, self.N, self.Qr[k], self.Kr, self.Vr, self.pos, self.causal,
                                   self.scale, out=self.Or[k], lse=self.lser[k])
            else:
                rank_forward(i, self.N, self.Qr[k], self.Kr, self.Vr, self.pos, self.causal,
                             self.scale, out=self.Or[k], lse=self.lser[k], workspace=self.ws)

    def backward(self, dO):
        """dO: global [B, H, L, D] (Q's dtype).  Returns global float32 (dQ, dK,
        dV); dQ rows of ranks outside [rank_lo, rank_hi) are left zero, and
        dK, dV hold the contributions of the selected ranks only."""
        import torch

        N, lo, hi = self.N, self.rank_lo, self.rank_hi
        f32 = dict(dtype=torch.float32, device=self.device)
        if not hasattr(self, "dQ"):
            self.dQ = torch.zeros((self.B, self.H, self.L, self.D), **f32)
            self.dK = torch.empty_like(self.dQ)
            self.dV = torch.empty_like(self.dQ)
        if self.global_layout:
            if not hasattr(self, "delta"):
                self.delta = torch.zeros((self.B, self.H, self.L), **f32)
            Q, K, V = self._inputs
            self.dK.zero_()
            self.dV.zero_()
            share_backward(Q, K, V, self.O, dO, self.lse, N, self.causal, self.dK, self.dV,
                           self.scale, lo, hi, dQ=self.dQ, delta=self.delta)
            return self.dQ, self.dK, self.dV
        if not hasattr(self, "dOr"):
            self.dOr = torch.empty_like(self.Qr)
            self.dQr = torch.empty(self.Qr.shape, **f32)
            self.deltar = torch.empty(self.lser.shape, **f32)
            self.dKr = torch.empty(self.Kr.shape, **f32)
            self.dVr = torch.empty(self.Vr.shape, **f32)
        zigzag_permute(dO, self.pos, N, rank_lo=lo, rank_hi=hi, out=self.dOr)
        self.dKr.zero_()
        self.dVr.zero_()
        for k, i in enumerate(range(lo, hi)):
            rank_backward(i, N, self.Qr[k], self.Kr, self.Vr, self.pos, self.Or[k], self.dOr[k],
                          self.lser[k], self.causal, self.dKr, self.dVr, self.scale,
                          dQ=self.dQr[k], delta=self.deltar[k])
        zigzag_permute(self.dQr, self.pos, N, inverse=True, rank_lo=lo, rank_hi=hi, out=self.dQ)
        zigzag_permute(self.dKr, self.pos, N, inverse=True, out=self.dK)
        zigzag_permute(self.dVr, self.pos, N, inverse=True, out=self.dV)
        return self.dQ, self.dK, self.dV
