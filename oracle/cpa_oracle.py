"""CPU fp64 oracle for context-parallel (ring) attention over a zigzag layout.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It shares no
code with the HIP library and imports nothing from it: it works on plain
numpy arrays handed in by the caller.

Every function is the plain definition written out in float64 (numpy), with a
matrix product or an elementwise numpy routine as its only library steps.
Sources (page title, then section):

* "序列与上下文并行" (ai-infra-wiki), section 上下文并行：注意力本身切分 --
  each rank keeps its own Q/K/V segment, the K/V blocks travel a ring, rank i
  forms Q_i against K_j/V_j in the order j = i, i+1, ... and folds each partial
  result into its running result by online softmax; causal imbalance is
  removed by a Z-shaped (zigzag) chunk assignment.  Section 工程实践 adds that
  every rank must know the global offset of its tokens.
* "Tensor并行与算子拆分" (aiknowledge.cn), section 注意力的并行化优化,
  OptimizedTensorParallelAttention.forward -- scores are q.k^T / sqrt(d_k),
  masked entries become -inf, softmax over keys, weights times V.
* "4. 序列并行" (5688vip), section 关键完整代码, and "序列并行：四位书生分读百米长卷"
  (aiqz.cc), section 核心原理 -- the per-rank results, put back in sequence
  order, must equal the result over the whole sequence.

Readings where the pages are silent (each is listed in the design notes):
the zigzag gives rank r chunks r and 2N-1-r of length L/(2N), in ascending
order; a key is visible to a query when its global position is <= the query's;
the scale is 1/sqrt(D); dropout is off; a query row with no visible key gives
O = 0 and lse = -inf; lse is a natural logarithm.

Rotary position embedding (rope, permute_to_ranks_rope) follows the same
page's 工程实践 rule that positions are global, with the frequency schedule of
the sinusoidal table in "Tensor并行与算子拆分" (model code, PositionalEncoding);
the rotation itself is the standard rotary embedding (the pages give no
formula for it).

The backward (backward_block and the functions built on it) is the
derivative of the same attention, written out; the pages state only that CP
is validated on training losses (the same page, 工程实践).

Pins (tests/test_oracle_pins.py): a pure-Python triple loop, torch's
scaled_dot_product_attention in float64, closed forms (uniform scores,
constant V, first causal row), the chunk-then-merge invariant of the pages,
merge algebra, structural invariants and the zigzag balance count; for rope
the pages' sinusoidal table itself, pair-norm preservation, the identity at
position 0, the dependence of q.k on the position difference only, and the
global-versus-local position check; for the backward torch autograd in
float64, central finite differences, the block-by-block ring decomposition,
the zero sum of dK over keys, the sum of dV over keys and constant V.  Every
function below is pinned; none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# Zigzag layout
# ---------------------------------------------------------------------------

def chunk_of_rank(r: int, N: int) -> tuple[int, int]:
    """The two chunk indices (out of 2N) owned by rank r: r and 2N-1-r.

    Reading of the Z-shaped assignment ("序列与上下文并行", 上下文并行 and
    工程实践): pairing an early chunk with the mirrored late chunk gives each
    rank the same amount of causal work.
    """
    return r, 2 * N - 1 - r


def zigzag_layout(L: int, N: int) -> np.ndarray:
    """Global token position of every local token: int64 [N, L/N].

    Row r is chunk r followed by chunk 2N-1-r (both ascending), each chunk
    being C = L/(2N) consecutive positions.
    """
    if N < 1 or L <= 0 or L % (2 * N) != 0:
        raise ValueError(f"zigzag layout needs N >= 1, L > 0, L % 2N == 0 (L={L}, N={N})")
    C = L // (2 * N)
    out = np.empty((N, L // N), dtype=np.int64)
    for r in range(N):
        lo, hi = chunk_of_rank(r, N)
        out[r, :C] = np.arange(lo * C, (lo + 1) * C, dtype=np.int64)
        out[r, C:] = np.arange(hi * C, (hi + 1) * C, dtype=np.int64)
    return out


def contiguous_layout(L: int, N: int) -> np.ndarray:
    """Plain contiguous sharding (rank r holds [rL/N, (r+1)L/N)), the layout of
    the diagram on "序列并行：超长序列训练".  Used only as the unbalanced
    comparator in the balance pin."""
    if N < 1 or L % N != 0:
        raise ValueError("contiguous layout needs L % N == 0")
    return np.arange(L, dtype=np.int64).reshape(N, L // N)


def first_non_increasing(pos) -> int | None:
    """Flat index of the first entry of a position table ([n] or [rows, n])
    that is not the first of its row and does not exceed the entry before it;
    None if every row is strictly increasing.

    Within a rank the Z-shaped assignment gives its early chunk, then its late
    chunk, each in ascending order ("序列与上下文并行", 上下文并行), so every
    row of a zigzag table increases; causal masking by position relies on
    that order.  A plain scan of the rows.
    """
    a = np.asarray(pos, dtype=np.int64)
    if a.ndim == 1:
        a = a.reshape(1, -1)
    rows, n = a.shape
    for r in range(rows):
        for t in range(1, n):
            if a[r, t] <= a[r, t - 1]:
                return r * n + t
    return None


def causal_pairs(q_pos: np.ndarray, k_pos: np.ndarray) -> int:
    """Number of (query, key) pairs with key position <= query position."""
    k_sorted = np.sort(np.asarray(k_pos))
    return int(np.searchsorted(k_sorted, np.asarray(q_pos), side="right").sum())


def ring_order(i: int, N: int) -> list[int]:
    """K/V segments visited by rank i, in order: i, i+1, ..., wrapping mod N
    (the per-card sequences drawn in "序列与上下文并行", 上下文并行)."""
    return [(i + s) % N for s in range(N)]


# ---------------------------------------------------------------------------
# Permutation between the global order and the rank-major zigzag order
# ---------------------------------------------------------------------------

def permute_to_ranks(x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Global [B, H, L, D] -> rank-major [N, B, H, L/N, D]:
    out[r, b, h, t] = x[b, h, pos[r, t]]."""
    return np.stack([x[:, :, pos[r]] for r in range(pos.shape[0])], axis=0)


def permute_from_ranks(y: np.ndarray, pos: np.ndarray, L: int) -> np.ndarray:
    """Inverse of permute_to_ranks: out[b, h, pos[r, t]] = y[r, b, h, t]."""
    N = pos.shape[0]
    out = np.zeros(y.shape[1:3] + (L,) + y.shape[4:], dtype=y.dtype)
    for r in range(N):
        out[:, :, pos[r]] = y[r]
    return out


# ---------------------------------------------------------------------------
# Rotary position embedding at global positions
# ---------------------------------------------------------------------------

ROPE_INTERLEAVED = 0  # pairs (2k, 2k+1)
ROPE_HALF = 1         # pairs (k, k + D/2)


def rope_frequencies(D: int, base: float = 10000.0) -> np.ndarray:
    """theta_k = base^(-2k/D), k = 0 .. D/2-1: the frequency schedule of the
    sinusoidal table in "Tensor并行与算子拆分" (model code, PositionalEncoding:
    the divisor term is exp(-2k ln(10000) / d_model))."""
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * k / D)


def rope_pairs(D: int, pairing: int) -> tuple[np.ndarray, np.ndarray]:
    """Indices (a_k, b_k) of the two elements rotated together by theta_k."""
    k = np.arange(D // 2)
    if pairing == ROPE_INTERLEAVED:
        return 2 * k, 2 * k + 1
    if pairing == ROPE_HALF:
        return k, k + D // 2
    raise ValueError(pairing)


def rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
         pairing: int = ROPE_INTERLEAVED) -> np.ndarray:
    """Rotate every row of x [..., rows, D] by its position: for each pair
    (a_k, b_k) and angle phi = pos * theta_k,
        y[a_k] = x[a_k] cos(phi) - x[b_k] sin(phi)
        y[b_k] = x[a_k] sin(phi) + x[b_k] cos(phi).
    `pos` [rows] are GLOBAL token positions: under CP every rank rotates its
    tokens by their place in the whole sequence, not by their local index
    ("序列与上下文并行", 工程实践: position encodings use the global offset of
    each rank's segment).  Reading: rotary embedding on the pages' sinusoidal
    frequency schedule; float64 throughout."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("rope needs an even head dimension")
    a, b = rope_pairs(D, pairing)
    phi = np.asarray(pos, dtype=np.float64)[:, None] * rope_frequencies(D, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    y = np.empty_like(x)
    y[..., a] = x[..., a] * c - x[..., b] * s
    y[..., b] = x[..., a] * s + x[..., b] * c
    return y


def permute_to_ranks_rope(x: np.ndarray, pos: np.ndarray, base: float = 10000.0,
                          pairing: int = ROPE_INTERLEAVED) -> np.ndarray:
    """Rank-major rows of x, each rotated at its global position:
    out[r, b, h, t] = rope(x[b, h, pos[r, t]], pos[r, t])."""
    return np.stack([rope(x[:, :, pos[r]], pos[r], base, pairing) for r in range(pos.shape[0])],
                    axis=0)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def default_scale(D: int) -> float:
    """Score scale 1/sqrt(d_k) ("Tensor并行与算子拆分", 注意力的并行化优化)."""
    return 1.0 / math.sqrt(D)


def visible(q_pos: np.ndarray, k_pos: np.ndarray, causal: bool) -> np.ndarray:
    """Boolean [Lq, Lk]: may query t see key u?  Causal: key position <= query
    position, both global (reading of the causal boundary; the global-offset
    rule is in "序列与上下文并行", 工程实践)."""
    if not causal:
        return np.ones((len(q_pos), len(k_pos)), dtype=bool)
    return np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]


def _softmax_rows(s: np.ndarray):
    """Row softmax statistics of a score block with -inf for hidden entries.

    Returns (w, m, l): w = exp(s - m) (0 where hidden), m the row max, l the
    row sum of w.  Rows with no finite score keep m = -inf, l = 0, w = 0."""
    m = s.max(axis=1)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(s - m_safe[:, None])
    w[~finite] = 0.0
    l = w.sum(axis=1)
    return w, m, l


def attention_block(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    q_pos: np.ndarray, k_pos: np.ndarray,
                    causal: bool, scale: float | None = None):
    """softmax(q k^T * scale + mask) v for one (batch, head).

    q [Lq, D], k [Lk, D], v [Lk, D] float64; q_pos [Lq], k_pos [Lk] global
    positions.  Returns O [Lq, D] and lse [Lq] (natural log of the row sum of
    exp(scores)).  A row that sees no key gets O = 0 and lse = -inf.
    """
    D = q.shape[1]
    if scale is None:
        scale = default_scale(D)
    s = (q @ k.T) * scale
    s = np.where(visible(q_pos, k_pos, causal), s, NEG_INF)
    w, m, l = _softmax_rows(s)
    O = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.full(q.shape[0], NEG_INF, dtype=np.float64)
    ok = l > 0
    O[ok] = (w[ok] @ v) / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return O, lse


def attention_rows(q_rows: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                   causal: bool, scale: float | None = None, block: int = 256):
    """Full-sequence attention for selected query rows of one (batch, head).

    q_rows [R, D] are the queries at global positions q_pos [R]; k, v [L, D]
    are the whole sequence (key u sits at position u).  Rows are independent,
    so they are evaluated `block` at a time; for causal rows only the keys up
    to the block's last visible position are touched (the rest are masked).
    """
    L = k.shape[0]
    O = np.empty((q_rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.empty(q_rows.shape[0], dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    for a in range(0, q_rows.shape[0], block):
        b = min(a + block, q_rows.shape[0])
        kend = int(q_pos[a:b].max()) + 1 if causal else L
        O[a:b], lse[a:b] = attention_block(q_rows[a:b], k[:kend], v[:kend], q_pos[a:b],
                                           np.arange(kend, dtype=np.int64), causal, scale)
    return O, lse


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, causal: bool,
              scale: float | None = None):
    """Whole-sequence attention, [B, H, L, D] float64 -> O [B, H, L, D], lse [B, H, L]."""
    B, H, L, D = Q.shape
    O = np.empty((B, H, L, V.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, L), dtype=np.float64)
    pos = np.arange(L, dtype=np.int64)
    for b in range(B):
        for h in range(H):
            O[b, h], lse[b, h] = attention_rows(Q[b, h], pos, K[b, h], V[b, h], causal, scale)
    return O, lse


def partial(Qi: np.ndarray, Kj: np.ndarray, Vj: np.ndarray,
            q_off: np.ndarray, k_off: np.ndarray, causal: bool,
            scale: float | None = None):
    """One ring step: rank i's queries against rank j's keys/values.

    Qi [B, H, Lq, D], Kj/Vj [B, H, Lk, D] float64; q_off [Lq], k_off [Lk] global
    positions.  Returns (O [B, H, Lq, D], lse [B, H, Lq]) of the softmax over
    the visible keys of this block only ("序列与上下文并行", 上下文并行: each
    step yields a partial result for the local Q).
    """
    B, H, Lq, _ = Qi.shape
    O = np.empty((B, H, Lq, Vj.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, Lq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            O[b, h], lse[b, h] = attention_block(Qi[b, h], Kj[b, h], Vj[b, h],
                                                 q_off, k_off, causal, scale)
    return O, lse


def merge(O_a: np.ndarray, lse_a: np.ndarray, O_b: np.ndarray, lse_b: np.ndarray):
    """Online-softmax combination of two partial results over disjoint key sets.

    With lse = m + ln(l) and O = (sum_k e^{s_k - m} v_k) / l, the union of the
    two key sets has lse = ln(e^{lse_a} + e^{lse_b}) and O the two O's weighted
    by e^{lse_a - lse} and e^{lse_b - lse} ("序列与上下文并行", 上下文并行: the
    online softmax of FlashAttention folds blocks together).  Evaluated with
    the larger lse factored out.  Two empty partials (-inf, -inf) give O = 0,
    lse = -inf.
    """
    M = np.maximum(lse_a, lse_b)
    empty = ~np.isfinite(M)
    M_safe = np.where(empty, 0.0, M)
    w_a = np.where(np.isfinite(lse_a), np.exp(lse_a - M_safe), 0.0)
    w_b = np.where(np.isfinite(lse_b), np.exp(lse_b - M_safe), 0.0)
    tot = w_a + w_b
    tot_safe = np.where(empty, 1.0, tot)
    O = (w_a[..., None] * O_a + w_b[..., None] * O_b) / tot_safe[..., None]
    O = np.where(empty[..., None], 0.0, O)
    lse = np.where(empty, NEG_INF, M_safe + np.log(tot_safe))
    return O, lse


def rank_forward(i: int, Q_i: np.ndarray, K_ranks: np.ndarray, V_ranks: np.ndarray,
                 pos: np.ndarray, causal: bool, scale: float | None = None):
    """Rank i's whole ring: partials against every rank's K/V in ring order,
    folded by `merge`.

    Q_i [B, H, L/N, D]; K_ranks/V_ranks rank-major [N, B, H, L/N, D]; pos the
    [N, L/N] layout.  Returns (O_i, lse_i) for rank i's local tokens.
    """
    N = pos.shape[0]
    O = lse = None
    for j in ring_order(i, N):
        O_s, lse_s = partial(Q_i, K_ranks[j], V_ranks[j], pos[i], pos[j], causal, scale)
        if O is None:
            O, lse = O_s, lse_s
        else:
            O, lse = merge(O, lse, O_s, lse_s)
    return O, lse


# ---------------------------------------------------------------------------
# Backward: gradients of the attention output
# ---------------------------------------------------------------------------
#
# The pages give no backward; CP exists for training ("序列与上下文并行": the
# numerical check of CP compares training losses, 工程实践), so the gradients
# are needed.  They are the derivative of O = softmax(s) v, s = q k^T * scale
# + mask, for an upstream gradient dO:
#     P = exp(s - lse) on visible pairs, 0 elsewhere   (the forward's weights)
#     dP = dO v^T,  delta_t = sum_u P[t, u] dP[t, u] = sum_d dO[t, d] O[t, d]
#     dS = P * (dP - delta)   (derivative of the softmax)
#     dq = scale * dS k,  dk = scale * dS^T q,  dv = P^T dO.
# Under CP the same formulas hold block by block when P uses the query row's
# FINAL lse over all its keys, so rank i's gradient contributions against
# K/V block j need only (Q_i, dO_i, lse_i, delta_i) and (K_j, V_j).

def backward_delta(O: np.ndarray, dO: np.ndarray) -> np.ndarray:
    """delta [..., rows] = sum over d of dO * O (equal to sum_u P dP)."""
    return np.sum(np.asarray(dO, dtype=np.float64) * np.asarray(O, dtype=np.float64), axis=-1)


def backward_block(q: np.ndarray, k: np.ndarray, v: np.ndarray, dO: np.ndarray,
                   lse: np.ndarray, delta: np.ndarray, q_pos: np.ndarray, k_pos: np.ndarray,
                   causal: bool, scale: float | None = None):
    """Gradient contributions of one query block against one key/value block
    of one (batch, head), given the query rows' final lse and delta.
    Returns (dq [Lq, D], dk [Lk, D], dv [Lk, D]).  Rows with lse = -inf (no
    visible key anywhere) contribute nothing."""
    D = q.shape[1]
    if scale is None:
        scale = default_scale(D)
    s = scale * (q @ k.T)
    fin = np.isfinite(lse)
    ok = visible(q_pos, k_pos, causal) & fin[:, None]
    P = np.zeros_like(s)
    P[ok] = np.exp(s - np.where(fin, lse, 0.0)[:, None])[ok]
    dP = dO @ v.T
    dS = P * (dP - delta[:, None])
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ dO


def backward_rows(q_rows: np.ndarray, q_pos: np.ndarray, k: np.ndarray, v: np.ndarray,
                  dO_rows: np.ndarray, lse_rows: np.ndarray, delta_rows: np.ndarray,
                  causal: bool, scale: float | None = None, block: int = 256):
    """backward_block of selected query rows of one (batch, head) against the
    whole sequence (key u at position u), `block` rows at a time.  Returns dq
    of those rows and their summed contributions to dk, dv [L, D]."""
    L, D = k.shape
    dq = np.empty((q_rows.shape[0], D), dtype=np.float64)
    dk = np.zeros((L, D), dtype=np.float64)
    dv = np.zeros((L, v.shape[1]), dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    for a in range(0, q_rows.shape[0], block):
        b = min(a + block, q_rows.shape[0])
        kend = (int(q_pos[a:b].max()) + 1) if causal else L
        dq[a:b], dk_b, dv_b = backward_block(q_rows[a:b], k[:kend], v[:kend], dO_rows[a:b],
                                             lse_rows[a:b], delta_rows[a:b], q_pos[a:b],
                                             np.arange(kend, dtype=np.int64), causal, scale)
        dk[:kend] += dk_b
        dv[:kend] += dv_b
    return dq, dk, dv


def attention_backward(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                       causal: bool, scale: float | None = None):
    """Gradients of sum(dO * O) with respect to Q, K, V of whole-sequence
    attention, all [B, H, L, D] float64."""
    O, lse = attention(Q, K, V, causal, scale)
    delta = backward_delta(O, dO)
    B, H, L, _ = Q.shape
    pos = np.arange(L, dtype=np.int64)
    dQ, dK, dV = np.empty_like(Q), np.empty_like(K), np.empty_like(V)
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = backward_rows(Q[b, h], pos, K[b, h], V[b, h],
                                                         dO[b, h], lse[b, h], delta[b, h],
                                                         causal, scale)
    return dQ, dK, dV


def partial_backward(Qi: np.ndarray, Kj: np.ndarray, Vj: np.ndarray, dOi: np.ndarray,
                     lse_i: np.ndarray, delta_i: np.ndarray, q_off: np.ndarray,
                     k_off: np.ndarray, causal: bool, scale: float | None = None):
    """One ring step of the backward: rank i's (Q, dO, lse, delta) against
    rank j's K/V, [B, H, rows, D].  Returns (dQ_ij, dK_ij, dV_ij)."""
    B, H, Lq, D = Qi.shape
    Lk = Kj.shape[2]
    dQ = np.empty((B, H, Lq, D))
    dK = np.empty((B, H, Lk, D))
    dV = np.empty((B, H, Lk, Vj.shape[3]))
    for b in range(B):
        for h in range(H):
            dQ[b, h], dK[b, h], dV[b, h] = backward_block(
                Qi[b, h], Kj[b, h], Vj[b, h], dOi[b, h], lse_i[b, h], delta_i[b, h],
                q_off, k_off, causal, scale)
    return dQ, dK, dV


def rank_backward(i: int, Q_i: np.ndarray, K_ranks: np.ndarray, V_ranks: np.ndarray,
                  dO_i: np.ndarray, lse_i: np.ndarray, delta_i: np.ndarray, pos: np.ndarray,
                  causal: bool, scale: float | None = None):
    """Rank i's ring backward: dQ_i summed over every K/V block (in ring
    order), and rank i's contributions to every block's dK, dV (in a
    multi-GPU ring these accumulators travel with K/V and return to their
    owner).  Returns (dQ_i [B, H, L/N, D], dK [N, ...], dV [N, ...])."""
    N = pos.shape[0]
    dQ = np.zeros_like(Q_i)
    dK = np.zeros_like(K_ranks)
    dV = np.zeros_like(V_ranks)
    for j in ring_order(i, N):
        dq, dk, dv = partial_backward(Q_i, K_ranks[j], V_ranks[j], dO_i, lse_i, delta_i,
                                      pos[i], pos[j], causal, scale)
        dQ += dq
        dK[j] += dk
        dV[j] += dv
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# Brute force (pure Python, tiny inputs only)
# ---------------------------------------------------------------------------

def brute_force_attention(Q, K, V, causal: bool, scale: float | None = None):
    """Triple loop over (b, h, query), summing keys one at a time with
    math.exp.  Q, K, V are nested lists or arrays [B][H][L][D]."""
    B, H, L, D = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    O = [[[[0.0] * D for _ in range(L)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * L for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for p in range(L):
                keys = range(p + 1) if causal else range(L)
                scores = []
                for u in keys:
                    dot = 0.0
                    for d in range(D):
                        dot += float(Q[b][h][p][d]) * float(K[b][h][u][d])
                    scores.append(dot * scale)
                m = max(scores)
                ws = [math.exp(x - m) for x in scores]
                tot = sum(ws)
                for d in range(D):
                    acc = 0.0
                    for w, u in zip(ws, keys):
                        acc += w * float(V[b][h][u][d])
                    O[b][h][p][d] = acc / tot
                lse[b][h][p] = m + math.log(tot)
    return np.array(O, dtype=np.float64), np.array(lse, dtype=np.float64)
