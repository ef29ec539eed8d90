"""libcpattn: context-parallel ring attention on MI355X (gfx950).

Python names mirror the C ABI (include/cpattn.h) without the `cpa_` prefix.
Tensors supply device memory; the HIP stream is torch's current stream on the
tensors' device.  Nothing is computed here: every call goes to the library.
"""
from __future__ import annotations

import ctypes
import os

from ._lib import (CPA_BF16, CPA_EDTYPE, CPA_EINVAL, CPA_ESHAPE, CPA_F32,  # noqa: F401
                   CPA_ROPE_HALF, CPA_ROPE_INTERLEAVED, CpaError, check, last_error, load,
                   version)

__all__ = ["zigzag_layout", "partial", "merge", "rank_forward_workspace", "rank_forward",
           "rank_forward_noalloc", "rank_forward_fused", "share_forward", "share_backward", "zigzag_permute", "rope",
           "zigzag_permute_rope", "backward_delta", "partial_backward", "rank_backward",
           "check_offsets", "debug_offsets", "last_error", "version", "CpaError", "CPA_ROPE_INTERLEAVED", "CPA_ROPE_HALF"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CPA_BF16
    if t.dtype == torch.float32:
        return CPA_F32
    raise CpaError(CPA_EDTYPE, f"unsupported tensor dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _expect(t, shape, dtypes, name):
    """Reject a tensor whose shape or dtype disagrees with the sizes the C call
    is given: the library sees raw pointers and would read or write past it."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise CpaError(CPA_ESHAPE, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise CpaError(CPA_EDTYPE, f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _need_gpu(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise CpaError(CPA_EINVAL, "tensors must live on the GPU")
        if not t.is_contiguous():
            raise CpaError(CPA_EINVAL, "tensors must be contiguous")


_debug_offsets = os.environ.get("CPA_DEBUG_OFFSETS", "0") not in ("", "0")


def debug_offsets(enable: bool) -> None:
    """Switch the offsets check on or off for every later causal call.

    When on, each call with causal masking first runs check_offsets on its
    position tables and raises CpaError(CPA_EINVAL) naming the first entry
    that does not exceed its predecessor.  The check synchronises the stream
    (it reads the answer back), so it is a debugging aid: off by default, on
    from the start when the environment sets CPA_DEBUG_OFFSETS=1."""
    global _debug_offsets
    _debug_offsets = bool(enable)


def check_offsets(off):
    """Flat index of the first entry of `off` (int64 on the GPU, [n] or
    [rows, n]) that is not the first of its row and does not exceed the entry
    before it; None if every row is strictly increasing.  Synchronises the
    stream to read the answer."""
    torch = _torch()
    if off.dim() == 1:
        rows, n = 1, off.shape[0]
    elif off.dim() == 2:
        rows, n = off.shape
    else:
        raise CpaError(CPA_ESHAPE, f"off must be [n] or [rows, n], got shape {tuple(off.shape)}")
    _expect(off, off.shape, (torch.int64,), "off")
    _need_gpu(off)
    first_bad = torch.empty(1, dtype=torch.int64, device=off.device)
    check(load().cpa_check_offsets(_ptr(off), rows, n, _ptr(first_bad), _stream(off)))
    i = int(first_bad.item())
    return None if i == rows * n else i


def _debug_check(causal, **tables):
    if not (_debug_offsets and causal):
        return
    for name, t in tables.items():
        i = check_offsets(t)
        if i is not None:
            n = t.shape[-1]
            raise CpaError(CPA_EINVAL, f"{name} is not strictly increasing: row {i // n}, entry "
                                       f"{i % n} does not exceed the entry before it")


def _debug_range(pos_all, L):
    """Debug mode only: the permutes index rows by position, so every entry of
    the table must lie in [0, L) (reads the answer back: synchronises)."""
    if not _debug_offsets or pos_all.numel() == 0:
        return
    lo, hi = int(pos_all.min().item()), int(pos_all.max().item())
    if lo < 0 or hi >= L:
        raise CpaError(CPA_EINVAL, f"pos_all has entries outside [0, {L}): min {lo}, max {hi}")


def zigzag_layout(L: int, N: int):
    """int64 CPU tensor [N, L/N] of global token positions per rank (host call)."""
    torch = _torch()
    if N < 1 or L <= 0 or L % (2 * N):
        out = torch.empty(1, dtype=torch.int64)
    else:
        out = torch.empty((N, L // N), dtype=torch.int64)
    check(load().cpa_zigzag_layout(L, N, ctypes.cast(out.data_ptr(), ctypes.POINTER(ctypes.c_int64))))
    return out


def partial(Q, K, V, q_off, k_off, causal: bool, scale: float = 0.0, out=None, lse=None):
    """(O, lse) of Q [B,H,Lq,D] against K/V [B,H,Lk,D] with global positions."""
    torch = _torch()
    B, H, Lq, D = Q.shape
    Lk = K.shape[2]
    if out is None:
        out = torch.empty((B, H, Lq, D), dtype=torch.float32, device=Q.device)
    if lse is None:
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=Q.device)
    dt, f32, i64 = (Q.dtype,), (torch.float32,), (torch.int64,)
    _expect(K, (B, H, Lk, D), dt, "K")
    _expect(V, (B, H, Lk, D), dt, "V")
    _expect(q_off, (Lq,), i64, "q_off")
    _expect(k_off, (Lk,), i64, "k_off")
    _expect(out, (B, H, Lq, D), f32, "out")
    _expect(lse, (B, H, Lq), f32, "lse")
    _need_gpu(Q, K, V, q_off, k_off, out, lse)
    _debug_check(causal, q_off=q_off, k_off=k_off)
    check(load().cpa_partial(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), B, H, Lq, Lk, D,
                             _ptr(q_off), _ptr(k_off), int(bool(causal)), float(scale),
                             _ptr(out), _ptr(lse), _stream(Q)))
    return out, lse


def merge(O_acc, lse_acc, O_new, lse_new):
    """In-place online-softmax merge of (O_new, lse_new) into (O_acc, lse_acc)."""
    torch = _torch()
    f32 = (torch.float32,)
    _expect(O_acc, O_acc.shape, f32, "O_acc")
    _expect(O_new, O_acc.shape, f32, "O_new")
    _expect(lse_acc, O_acc.shape[:-1], f32, "lse_acc")
    _expect(lse_new, O_acc.shape[:-1], f32, "lse_new")
    _need_gpu(O_acc, lse_acc, O_new, lse_new)
    D = O_acc.shape[-1]
    rows = O_acc.numel() // D
    check(load().cpa_merge(_ptr(O_acc), _ptr(lse_acc), _ptr(O_new), _ptr(lse_new), rows, D,
                           _stream(O_acc)))
    return O_acc, lse_acc


def rank_forward_workspace(B: int, H: int, L: int, N: int, D: int) -> int:
    return int(load().cpa_rank_forward_workspace(B, H, L, N, D))


def _check_rank_major(Q_i, K_all, V_all, pos_all, N, out, lse):
    torch = _torch()
    B, H, Lr, D = Q_i.shape
    dt, f32 = (Q_i.dtype,), (torch.float32,)
    _expect(K_all, (N, B, H, Lr, D), dt, "K_all")
    _expect(V_all, (N, B, H, Lr, D), dt, "V_all")
    _expect(pos_all, (N, Lr), (torch.int64,), "pos_all")
    _expect(out, (B, H, Lr, D), f32, "out")
    _expect(lse, (B, H, Lr), f32, "lse")


def rank_forward(i: int, N: int, Q_i, K_all, V_all, pos_all, causal: bool, scale: float = 0.0,
                 out=None, lse=None, workspace=None):
    """Rank i's ring: Q_i [B,H,L/N,D] vs rank-major K_all/V_all [N,B,H,L/N,D]."""
    torch = _torch()
    B, H, Lr, D = Q_i.shape
    L = Lr * N
    if out is None:
        out = torch.empty((B, H, Lr, D), dtype=torch.float32, device=Q_i.device)
    if lse is None:
        lse = torch.empty((B, H, Lr), dtype=torch.float32, device=Q_i.device)
    ws_bytes = rank_forward_workspace(B, H, L, N, D)
    if workspace is None and N > 1:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=Q_i.device)
    _check_rank_major(Q_i, K_all, V_all, pos_all, N, out, lse)
    if workspace is not None and workspace.dtype != torch.uint8:
        raise CpaError(CPA_EDTYPE, f"workspace has dtype {workspace.dtype}, expected torch.uint8")
    _need_gpu(Q_i, K_all, V_all, pos_all, out, lse, workspace)
    _debug_check(causal, pos_all=pos_all)
    check(load().cpa_rank_forward(i, N, _ptr(Q_i), _ptr(K_all), _ptr(V_all), _ptr(pos_all),
                                  _dtype_code(Q_i), B, H, L, D, int(bool(causal)), float(scale),
                                  _ptr(out), _ptr(lse), _ptr(workspace),
                                  0 if workspace is None else workspace.numel(), _stream(Q_i)))
    return out, lse


def rank_forward_noalloc(i: int, N: int, Q_i, K_all, V_all, pos_all, causal: bool,
                         scale: float = 0.0, out=None, lse=None):
    """rank_forward with the partial kept in the library's per-GPU scratch
    instead of a workspace (the C call allocates nothing; out/lse are made
    here only when not given)."""
    torch = _torch()
    B, H, Lr, D = Q_i.shape
    if out is None:
        out = torch.empty((B, H, Lr, D), dtype=torch.float32, device=Q_i.device)
    if lse is None:
        lse = torch.empty((B, H, Lr), dtype=torch.float32, device=Q_i.device)
    _check_rank_major(Q_i, K_all, V_all, pos_all, N, out, lse)
    _need_gpu(Q_i, K_all, V_all, pos_all, out, lse)
    _debug_check(causal, pos_all=pos_all)
    check(load().cpa_rank_forward_noalloc(i, N, _ptr(Q_i), _ptr(K_all), _ptr(V_all),
                                          _ptr(pos_all), _dtype_code(Q_i), B, H, Lr * N, D,
                                          int(bool(causal)), float(scale), _ptr(out), _ptr(lse),
                                          _stream(Q_i)))
    return out, lse


def rank_forward_fused(i: int, N: int, Q_i, K_all, V_all, pos_all, causal: bool,
                       scale: float = 0.0, out=None, lse=None):
    """Rank i's ring in one launch (bf16, D = 64 or 128); same result as rank_forward."""
    torch = _torch()
    B, H, Lr, D = Q_i.shape
    if out is None:
        out = torch.empty((B, H, Lr, D), dtype=torch.float32, device=Q_i.device)
    if lse is None:
        lse = torch.empty((B, H, Lr), dtype=torch.float32, device=Q_i.device)
    _check_rank_major(Q_i, K_all, V_all, pos_all, N, out, lse)
    _need_gpu(Q_i, K_all, V_all, pos_all, out, lse)
    _debug_check(causal, pos_all=pos_all)
    check(load().cpa_rank_forward_fused(i, N, _ptr(Q_i), _ptr(K_all), _ptr(V_all), _ptr(pos_all),
                                        _dtype_code(Q_i), B, H, Lr * N, D, int(bool(causal)),
                                        float(scale), _ptr(out), _ptr(lse), _stream(Q_i)))
    return out, lse


def share_forward(Q, K, V, N: int, causal: bool, scale: float = 0.0, rank_lo: int = 0,
                  rank_hi: int | None = None, out=None, lse=None, precise: bool = False):
    """Rings of ranks [rank_lo, rank_hi) on global-order Q/K/V [B,H,L,D] (bf16):
    O [B,H,L,D] and lse [B,H,L] float32 in global order, the selected ranks'
    rows written (the zigzag permute folded into the kernel's addressing, a
    token's position its global index: no position table).  precise=True
    calls cpa_share_forward_precise (softmax weights as a bf16 pair)."""
    torch = _torch()
    rank_hi = N if rank_hi is None else rank_hi
    B, H, L, D = Q.shape
    if out is None:
        out = torch.zeros((B, H, L, D), dtype=torch.float32, device=Q.device)
    if lse is None:
        lse = torch.full((B, H, L), float("-inf"), dtype=torch.float32, device=Q.device)
    dt, f32 = (Q.dtype,), (torch.float32,)
    _expect(K, (B, H, L, D), dt, "K")
    _expect(V, (B, H, L, D), dt, "V")
    _expect(out, (B, H, L, D), f32, "out")
    _expect(lse, (B, H, L), f32, "lse")
    _need_gpu(Q, K, V, out, lse)
    fn = load().cpa_share_forward_precise if precise else load().cpa_share_forward
    check(fn(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), B, H, L, D, N, rank_lo, rank_hi,
             int(bool(causal)), float(scale), _ptr(out), _ptr(lse), _stream(Q)))
    return out, lse


def share_backward(Q, K, V, O, dO, lse, N: int, causal: bool, dK, dV,
                   scale: float = 0.0, rank_lo: int = 0, rank_hi: int | None = None, dQ=None,
                   delta=None):
    """Ring backward of ranks [rank_lo, rank_hi) on global-order bf16 Q/K/V/dO
    [B,H,L,D] with the forward's global-order O [B,H,L,D] and lse [B,H,L]
    (float32): returns dQ (the selected ranks' rows written) and adds their
    contributions into the global-order float32 accumulators dK, dV."""
    torch = _torch()
    rank_hi = N if rank_hi is None else rank_hi
    B, H, L, D = Q.shape
    if dQ is None:
        dQ = torch.zeros((B, H, L, D), dtype=torch.float32, device=Q.device)
    if delta is None:
        delta = torch.empty((B, H, L), dtype=torch.float32, device=Q.device)
    dt, f32 = (Q.dtype,), (torch.float32,)
    for t, n in ((K, "K"), (V, "V"), (dO, "dO")):
        _expect(t, (B, H, L, D), dt, n)
    for t, n in ((O, "O"), (dQ, "dQ"), (dK, "dK"), (dV, "dV")):
        _expect(t, (B, H, L, D), f32, n)
    _expect(lse, (B, H, L), f32, "lse")
    _expect(delta, (B, H, L), f32, "delta")
    _need_gpu(Q, K, V, O, dO, lse, dK, dV, dQ, delta)
    check(load().cpa_share_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                                    _ptr(lse), _dtype_code(Q), B, H, L, D, N, rank_lo, rank_hi,
                                    int(bool(causal)), float(scale), _ptr(dQ), _ptr(dK), _ptr(dV),
                                    _ptr(delta), _stream(Q)))
    return dQ


def zigzag_permute(src, pos_all, N: int, inverse: bool = False, rank_lo: int = 0,
                   rank_hi: int | None = None, out=None):
    """Global [B,H,L,D] -> rank-major [nr,B,H,L/N,D] (or back with inverse=True)
    for ranks [rank_lo, rank_hi).  A 3-D source/target [B,H,L] is treated as D=1."""
    torch = _torch()
    rank_hi = N if rank_hi is None else rank_hi
    nr = rank_hi - rank_lo
    if inverse:
        squeeze = src.dim() == 4  # [nr,B,H,Lr] for lse
        x = src.unsqueeze(-1) if squeeze else src
        _, B, H, Lr, D = x.shape
        L = Lr * N
        if out is None:
            out = torch.zeros((B, H, L) if squeeze else (B, H, L, D), dtype=src.dtype, device=src.device)
    else:
        squeeze = src.dim() == 3
        x = src.unsqueeze(-1) if squeeze else src
        B, H, L, D = x.shape
        Lr = L // N
        if out is None:
            shape = (nr, B, H, Lr) if squeeze else (nr, B, H, Lr, D)
            out = torch.empty(shape, dtype=src.dtype, device=src.device)
    if inverse:
        # the source must hold exactly the selected ranks: the library reads nr of them
        _expect(src, (nr, B, H, Lr) if squeeze else (nr, B, H, Lr, D), (src.dtype,), "src")
        _expect(out, (B, H, L) if squeeze else (B, H, L, D), (src.dtype,), "out")
    else:
        _expect(out, (nr, B, H, Lr) if squeeze else (nr, B, H, Lr, D), (src.dtype,), "out")
    _expect(pos_all, (N, L // max(N, 1)), (torch.int64,), "pos_all")
    _need_gpu(src, pos_all, out)
    _debug_range(pos_all, L)
    check(load().cpa_zigzag_permute(_ptr(src), _ptr(out), src.element_size(), B, H, L, D,
                                    _ptr(pos_all), N, rank_lo, rank_hi, int(bool(inverse)),
                                    _stream(src)))
    return out


def rope(x, pos, base: float = 10000.0, pairing: int = CPA_ROPE_INTERLEAVED, out=None):
    """Rotary embedding of x [B,H,rows,D] at global positions pos [rows]
    (out=x rotates in place)."""
    torch = _torch()
    B, H, rows, D = x.shape
    if out is None:
        out = torch.empty_like(x)
    _expect(out, x.shape, (x.dtype,), "out")
    _expect(pos, (rows,), (torch.int64,), "pos")
    _need_gpu(x, pos, out)
    check(load().cpa_rope(_ptr(x), _ptr(out), _dtype_code(x), B, H, rows, D, _ptr(pos),
                          float(base), int(pairing), _stream(x)))
    return out


def zigzag_permute_rope(src, pos_all, N: int, base: float = 10000.0,
                        pairing: int = CPA_ROPE_INTERLEAVED, rank_lo: int = 0,
                        rank_hi: int | None = None, out=None):
    """Global [B,H,L,D] -> rank-major [nr,B,H,L/N,D], each row rotated at its
    global position (the forward permute with the rotary embedding folded in)."""
    torch = _torch()
    rank_hi = N if rank_hi is None else rank_hi
    B, H, L, D = src.shape
    if out is None:
        out = torch.empty((rank_hi - rank_lo, B, H, L // N, D), dtype=src.dtype, device=src.device)
    _expect(out, (rank_hi - rank_lo, B, H, L // max(N, 1), D), (src.dtype,), "out")
    _expect(pos_all, (N, L // max(N, 1)), (torch.int64,), "pos_all")
    _need_gpu(src, pos_all, out)
    _debug_range(pos_all, L)
    check(load().cpa_zigzag_permute_rope(_ptr(src), _ptr(out), _dtype_code(src), B, H, L, D,
                                         _ptr(pos_all), N, rank_lo, rank_hi, float(base),
                                         int(pairing), _stream(src)))
    return out


def backward_delta(O, dO, out=None):
    """delta [..., rows] = sum_d dO * O (O float32, dO bf16 or float32)."""
    torch = _torch()
    D = O.shape[-1]
    rows = O.numel() // D
    if out is None:
        out = torch.empty(O.shape[:-1], dtype=torch.float32, device=O.device)
    _expect(O, O.shape, (torch.float32,), "O")
    _expect(dO, O.shape, (torch.bfloat16, torch.float32), "dO")
    _expect(out, O.shape[:-1], (torch.float32,), "out")
    _need_gpu(O, dO, out)
    check(load().cpa_backward_delta(_ptr(O), _ptr(dO), _dtype_code(dO), rows, D, _ptr(out),
                                    _stream(O)))
    return out


def partial_backward(Q, K, V, dO, lse, delta, q_off, k_off, causal: bool, dQ, dK, dV,
                     scale: float = 0.0):
    """Add the gradient contributions of Q [B,H,Lq,D] against K/V [B,H,Lk,D]
    into the float32 accumulators dQ, dK, dV (one ring step of the backward)."""
    torch = _torch()
    B, H, Lq, D = Q.shape
    Lk = K.shape[2]
    dt, f32, i64 = (Q.dtype,), (torch.float32,), (torch.int64,)
    _expect(K, (B, H, Lk, D), dt, "K")
    _expect(V, (B, H, Lk, D), dt, "V")
    _expect(dO, (B, H, Lq, D), dt, "dO")
    _expect(lse, (B, H, Lq), f32, "lse")
    _expect(delta, (B, H, Lq), f32, "delta")
    _expect(q_off, (Lq,), i64, "q_off")
    _expect(k_off, (Lk,), i64, "k_off")
    _expect(dQ, (B, H, Lq, D), f32, "dQ")
    _expect(dK, (B, H, Lk, D), f32, "dK")
    _expect(dV, (B, H, Lk, D), f32, "dV")
    _need_gpu(Q, K, V, dO, lse, delta, q_off, k_off, dQ, dK, dV)
    _debug_check(causal, q_off=q_off, k_off=k_off)
    check(load().cpa_partial_backward(_ptr(Q), _ptr(K), _ptr(V), _ptr(dO), _ptr(lse), _ptr(delta),
                                      _dtype_code(Q), B, H, Lq, Lk, D, _ptr(q_off), _ptr(k_off),
                                      int(bool(causal)), float(scale), _ptr(dQ), _ptr(dK),
                                      _ptr(dV), _stream(Q)))
    return dQ, dK, dV


def rank_backward(i: int, N: int, Q_i, K_all, V_all, pos_all, O_i, dO_i, lse_i, causal: bool,
                  dK_all, dV_all, scale: float = 0.0, dQ=None, delta=None):
    """Rank i's ring backward: returns dQ_i (written) and adds rank i's
    contributions into the rank-major float32 accumulators dK_all, dV_all."""
    torch = _torch()
    B, H, Lr, D = Q_i.shape
    if dQ is None:
        dQ = torch.empty((B, H, Lr, D), dtype=torch.float32, device=Q_i.device)
    if delta is None:
        delta = torch.empty((B, H, Lr), dtype=torch.float32, device=Q_i.device)
    _check_rank_major(Q_i, K_all, V_all, pos_all, N, O_i, lse_i)
    f32 = (torch.float32,)
    _expect(dO_i, (B, H, Lr, D), (Q_i.dtype,), "dO_i")
    _expect(dK_all, (N, B, H, Lr, D), f32, "dK_all")
    _expect(dV_all, (N, B, H, Lr, D), f32, "dV_all")
    _expect(dQ, (B, H, Lr, D), f32, "dQ")
    _expect(delta, (B, H, Lr), f32, "delta")
    _need_gpu(Q_i, K_all, V_all, pos_all, O_i, dO_i, lse_i, dK_all, dV_all, dQ, delta)
    _debug_check(causal, pos_all=pos_all)
    check(load().cpa_rank_backward(i, N, _ptr(Q_i), _ptr(K_all), _ptr(V_all), _ptr(pos_all),
                                   _ptr(O_i), _ptr(dO_i), _ptr(lse_i), _dtype_code(Q_i), B, H,
                                   Lr * N, D, int(bool(causal)), float(scale), _ptr(dQ),
                                   _ptr(dK_all), _ptr(dV_all), _ptr(delta), _stream(Q_i)))
    return dQ
