"""Pins of the CPU oracle to facts outside itself (CPU only).

Each check_* takes the oracle module so that the planted-mistake test at the
bottom can run every pin against mutated copies of the oracle and show that
each plausible mistake (wrong scale, off-by-one mask, dropped merge term,
wrong sign, wrong chunk pairing, wrong ring direction ...) fails at least one.
"""
import math
import os
import types

import numpy as np
import pytest
import torch

from conftest import read_golden, ROOT
from oracle import cpa_oracle

TOL = 1e-12


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------- layout pins

def check_layout_golden(orc):
    """Tiny worked layout, written by hand from the zigzag reading."""
    rows = read_golden("zigzag_L64_N4.txt")
    got = orc.zigzag_layout(64, 4)
    for r, vals in rows:
        assert got[r].tolist() == vals, (r, got[r].tolist())


def check_layout_permutation(orc):
    """Every layout covers [0, L) exactly once and is two ascending runs of C."""
    for L, N in [(64, 4), (96, 3), (2, 1), (40, 5), (12288, 4), (131072, 4)]:
        pos = orc.zigzag_layout(L, N)
        C = L // (2 * N)
        assert pos.shape == (N, L // N)
        assert np.array_equal(np.sort(pos.ravel()), np.arange(L))
        for r in range(N):
            a, b = pos[r, :C], pos[r, C:]
            assert np.all(np.diff(a) == 1) and np.all(np.diff(b) == 1)
            assert a[0] % C == 0 and b[0] % C == 0 and a[-1] < b[0]


def check_layout_balance(orc):
    """Equal causal work per rank (hand-derived counts), summing to L(L+1)/2."""
    for vals in read_golden("causal_pairs.txt"):
        L, N, want = vals
        pos = orc.zigzag_layout(L, N)
        counts = [orc.causal_pairs(pos[r], np.arange(L)) for r in range(N)]
        assert counts == [want] * N, (L, N, counts)
        assert sum(counts) == L * (L + 1) // 2


def check_ring_order(orc):
    """Ring order prefixes drawn on the page."""
    for card, seq in read_golden("ring_order_diagram.txt"):
        for N in (3, 4, 8):
            assert orc.ring_order(card, N)[: len(seq)] == seq
    for N in (1, 4, 8):
        for i in range(N):
            assert sorted(orc.ring_order(i, N)) == list(range(N))


def check_permute(orc):
    """Gather/scatter between global and rank-major order: the rank-major rows
    are the golden positions, and the inverse undoes it."""
    L, N = 64, 4
    pos = orc.zigzag_layout(L, N)
    x = np.arange(2 * 3 * L * 2, dtype=np.float64).reshape(2, 3, L, 2)
    y = orc.permute_to_ranks(x, pos)
    assert y.shape == (N, 2, 3, L // N, 2)
    for r, vals in read_golden("zigzag_L64_N4.txt"):
        assert np.array_equal(y[r, 1, 2, :, 0], x[1, 2, vals, 0])
    assert np.array_equal(orc.permute_from_ranks(y, pos, L), x)


# ------------------------------------------------------------ attention pins

def check_brute_force(orc):
    """Pure-Python triple loop on tiny random cases."""
    for seed, (B, H, L, D) in enumerate([(1, 1, 1, 1), (1, 2, 5, 3), (2, 1, 16, 4), (1, 1, 7, 2)]):
        Q, K, V = (_rand((B, H, L, D), 3 * seed + t) for t in range(3))
        for causal in (True, False):
            O, lse = orc.attention(Q, K, V, causal)
            Ob, lseb = cpa_oracle.brute_force_attention(Q.tolist(), K.tolist(), V.tolist(), causal)
            assert np.max(np.abs(O - Ob)) <= TOL and np.max(np.abs(lse - lseb)) <= TOL


def _sdpa(Q, K, V, causal):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    O = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    s = torch.matmul(q, k.transpose(-1, -2).contiguous()) / math.sqrt(Q.shape[-1])
    if causal:
        L = Q.shape[2]
        s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    return O.numpy(), torch.logsumexp(s, dim=-1).numpy()


def check_sdpa(orc):
    """torch scaled_dot_product_attention in float64 (its own 1/sqrt(D) scale
    and causal mask) and torch.logsumexp of the scaled scores."""
    cases = [((1, 2, 64, 16), True), ((2, 3, 128, 64), False), ((1, 1, 2048, 128), True),
             ((1, 1, 33, 8), False)]
    for seed, (shape, causal) in enumerate(cases):
        Q, K, V = (_rand(shape, 10 * seed + t) for t in range(3))
        O, lse = orc.attention(Q, K, V, causal)
        Os, lses = _sdpa(Q, K, V, causal)
        assert np.max(np.abs(O - Os)) <= 1e-11, np.max(np.abs(O - Os))
        assert np.max(np.abs(lse - lses)) <= 1e-11


def check_uniform_scores(orc):
    """Q = 0 makes every visible score 0: O_p is the mean of the visible V rows
    and lse_p = ln(#visible keys)."""
    L, D = 40, 8
    V = _rand((1, 1, L, D), 7)
    K = _rand((1, 1, L, D), 8)
    Q = np.zeros((1, 1, L, D))
    O, lse = orc.attention(Q, K, V, True)
    for p in range(L):
        assert np.allclose(O[0, 0, p], V[0, 0, : p + 1].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[0, 0, p] - math.log(p + 1)) <= 1e-13
    O, lse = orc.attention(Q, K, V, False)
    assert np.allclose(O[0, 0], V[0, 0].mean(axis=0), rtol=0, atol=1e-13)
    assert np.allclose(lse, math.log(L), rtol=0, atol=1e-13)


def check_constant_v_and_first_row(orc):
    """Constant V gives O = V; the first causal row sees only key 0, so O_0 = V_0
    and lse_0 = q_0 . k_0 / sqrt(D)."""
    B, H, L, D = 1, 2, 24, 16
    Q, K = _rand((B, H, L, D), 11), _rand((B, H, L, D), 12)
    V = np.full((B, H, L, D), 0.375)
    O, _ = orc.attention(Q, K, V, True)
    assert np.max(np.abs(O - 0.375)) <= 1e-14
    V = _rand((B, H, L, D), 13)
    O, lse = orc.attention(Q, K, V, True)
    for h in range(H):
        assert np.array_equal(O[0, h, 0], V[0, h, 0])
        assert abs(lse[0, h, 0] - Q[0, h, 0] @ K[0, h, 0] / math.sqrt(D)) <= 1e-14


def check_chunk_merge_invariant(orc):
    """The pages' rule: per-rank results, put back in sequence order, equal
    the whole-sequence result -- here for ring partials merged by online
    softmax, every rank, several N, and any ring order."""
    for seed, (B, H, L, D, N, causal) in enumerate(
            [(1, 2, 64, 16, 4, True), (2, 2, 96, 8, 3, True), (1, 1, 32, 4, 1, True),
             (2, 2, 64, 8, 4, False), (1, 1, 80, 8, 5, True)]):
        Q, K, V = (_rand((B, H, L, D), 20 * seed + t) for t in range(3))
        O, lse = orc.attention(Q, K, V, causal)
        pos = orc.zigzag_layout(L, N)
        Qr, Kr, Vr = (orc.permute_to_ranks(x, pos) for x in (Q, K, V))
        Os, lses = [], []
        for i in range(N):
            Oi, lsei = orc.rank_forward(i, Qr[i], Kr, Vr, pos, causal)
            Os.append(Oi)
            lses.append(lsei)
        O2 = orc.permute_from_ranks(np.stack(Os), pos, L)
        lse2 = orc.permute_from_ranks(np.stack(lses)[..., None], pos, L)[..., 0]
        assert np.max(np.abs(O2 - O)) <= TOL and np.max(np.abs(lse2 - lse)) <= TOL
        # a reversed ring order folds the same partials in another order
        i = N - 1
        acc = None
        for j in reversed(range(N)):
            part = orc.partial(Qr[i], Kr[j], Vr[j], pos[i], pos[j], causal)
            acc = part if acc is None else orc.merge(*acc, *part)
        assert np.max(np.abs(acc[0] - Os[i])) <= TOL


def check_partial_empty_rows(orc):
    """Rank 0's first chunk sees nothing of a later rank's keys: O = 0, lse = -inf."""
    L, N, D = 64, 4, 8
    pos = orc.zigzag_layout(L, N)
    C = L // (2 * N)
    Q, K, V = (_rand((1, 1, L // N, D), 30 + t) for t in range(3))
    O, lse = orc.partial(Q, K, V, pos[0], pos[2], True)
    assert np.all(O[0, 0, :C] == 0) and np.all(np.isneginf(lse[0, 0, :C]))
    assert np.all(np.isfinite(lse[0, 0, C:]))


def check_merge_algebra(orc):
    """(0, -inf) is the identity; merge is commutative and associative; two
    empties stay empty without NaN; and merging the partials of two halves of
    a key set equals the softmax over the whole set."""
    rng = np.random.default_rng(40)
    Oa, Ob, Oc = (rng.standard_normal((5, 6)) for _ in range(3))
    la, lb, lc = (rng.standard_normal(5) * 3 for _ in range(3))
    z, zl = np.zeros((5, 6)), np.full(5, -np.inf)
    O, l = orc.merge(Oa, la, z, zl)
    assert np.array_equal(O, Oa) and np.array_equal(l, la)
    O, l = orc.merge(z, zl, Oa, la)
    assert np.max(np.abs(O - Oa)) <= TOL and np.max(np.abs(l - la)) <= TOL
    O1, l1 = orc.merge(Oa, la, Ob, lb)
    O2, l2 = orc.merge(Ob, lb, Oa, la)
    assert np.max(np.abs(O1 - O2)) <= TOL and np.max(np.abs(l1 - l2)) <= TOL
    O3, l3 = orc.merge(*orc.merge(Oa, la, Ob, lb), Oc, lc)
    O4, l4 = orc.merge(Oa, la, *orc.merge(Ob, lb, Oc, lc))
    assert np.max(np.abs(O3 - O4)) <= TOL and np.max(np.abs(l3 - l4)) <= TOL
    O, l = orc.merge(z, zl, z, zl)
    assert np.all(O == 0) and np.all(np.isneginf(l))
    # direct: scores s over 10 keys split 4 + 6
    s = rng.standard_normal((3, 10)) * 4
    v = rng.standard_normal((10, 2))
    def stats(ss, vv):
        w = np.exp(ss)
        return (w @ vv) / w.sum(1, keepdims=True), np.log(w.sum(1))
    O, l = orc.merge(*stats(s[:, :4], v[:4]), *stats(s[:, 4:], v[4:]))
    Of, lf = stats(s, v)
    assert np.max(np.abs(O - Of)) <= TOL and np.max(np.abs(l - lf)) <= TOL


def check_structural(orc):
    """Causal rows ignore every later key; non-causal attention ignores the
    order of the (K, V) rows; one rank reduces to plain attention."""
    B, H, L, D = 1, 1, 48, 8
    Q, K, V = (_rand((B, H, L, D), 50 + t) for t in range(3))
    O, lse = orc.attention(Q, K, V, True)
    p = 20
    K2, V2 = K.copy(), V.copy()
    K2[:, :, p + 1:] += 5.0
    V2[:, :, p + 1:] -= 3.0
    O2, lse2 = orc.attention(Q, K2, V2, True)
    assert np.array_equal(O2[:, :, : p + 1], O[:, :, : p + 1])
    assert np.max(np.abs(O2[:, :, p + 1:] - O[:, :, p + 1:])) > 1e-3
    perm = np.random.default_rng(51).permutation(L)
    On, _ = orc.attention(Q, K, V, False)
    Op, _ = orc.attention(Q, K[:, :, perm], V[:, :, perm], False)
    assert np.max(np.abs(On - Op)) <= TOL
    pos = orc.zigzag_layout(L, 1)
    O1, lse1 = orc.rank_forward(0, orc.permute_to_ranks(Q, pos)[0], orc.permute_to_ranks(K, pos),
                                orc.permute_to_ranks(V, pos), pos, True)
    assert np.max(np.abs(orc.permute_from_ranks(O1[None], pos, L) - O)) <= TOL


def check_sampled_rows(orc):
    """attention_rows on scattered rows equals the whole-sequence rows."""
    L, D = 300, 8
    Q, K, V = (_rand((L, D), 60 + t) for t in range(3))
    O, lse = orc.attention(Q[None, None], K[None, None], V[None, None], True)
    rows = np.array([0, 1, 17, 128, 255, 256, 299])
    Or, lser = orc.attention_rows(Q[rows], rows, K, V, True, block=3)
    assert np.max(np.abs(Or - O[0, 0, rows])) <= TOL and np.max(np.abs(lser - lse[0, 0, rows])) <= TOL


# ------------------------------------------------------------------ rope pins

def _sinusoid_table(p, d):
    """Row p of the sinusoidal position table that "Tensor并行与算子拆分"
    (model code, PositionalEncoding) builds, from its definition: pair k
    (columns 2k and 2k+1) holds the sine and cosine of the angle p * theta_k,
    with the frequency theta_k = 10000^(-2k/d)."""
    angles = [p * 10000.0 ** (-2.0 * k / d) for k in range(d // 2)]
    return [f(a) for a in angles for f in (math.sin, math.cos)]


def check_rope_sinusoid_table(orc):
    """Rotating the unit vector (1, 0) of every pair by position p gives
    (cos, sin) of the pages' table at p: this fixes the frequency schedule,
    the pairing and the direction of the rotation."""
    for d in (2, 8, 16, 128):
        positions = np.array([0, 1, 2, 7, 100, 4095, 131071], dtype=np.int64)
        table = np.array([_sinusoid_table(int(p), d) for p in positions])
        for pairing in (orc.ROPE_INTERLEAVED, orc.ROPE_HALF):
            x = np.zeros((len(positions), d))
            first = np.arange(0, d, 2) if pairing == orc.ROPE_INTERLEAVED else np.arange(d // 2)
            second = first + 1 if pairing == orc.ROPE_INTERLEAVED else first + d // 2
            x[:, first] = 1.0
            y = orc.rope(x, positions, 10000.0, pairing)
            # large angles: allow for the rounding of p * theta (|angle| <= 1.4e5)
            assert np.max(np.abs(y[:, first] - table[:, 1::2])) < 1e-9
            assert np.max(np.abs(y[:, second] - table[:, 0::2])) < 1e-9


def check_rope_norm_and_identity(orc):
    """A rotation keeps every pair's length; position 0 is the identity."""
    x = _rand((3, 40, 64), 11)
    pos = np.arange(1000, 1040, dtype=np.int64)
    for pairing in (orc.ROPE_INTERLEAVED, orc.ROPE_HALF):
        y = orc.rope(x, pos, 10000.0, pairing)
        a, b = orc.rope_pairs(64, pairing)
        assert np.allclose(y[..., a] ** 2 + y[..., b] ** 2, x[..., a] ** 2 + x[..., b] ** 2,
                           rtol=1e-12, atol=1e-12)
        assert not np.allclose(y, x)
        assert np.array_equal(orc.rope(x, np.zeros(40, dtype=np.int64), 10000.0, pairing), x)


def check_rope_relative(orc):
    """q.k after rotation depends on the position difference only, through the
    closed form sum_k [(qa ka + qb kb) cos(dn theta_k) + (qb ka - qa kb) sin(dn theta_k)],
    dn = n - m (rotary embedding's defining property)."""
    D = 32
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    theta = np.array([10000.0 ** (-2.0 * j / D) for j in range(D // 2)])
    for pairing in (orc.ROPE_INTERLEAVED, orc.ROPE_HALF):
        a, b = (np.arange(0, D, 2), np.arange(1, D, 2)) if pairing == orc.ROPE_INTERLEAVED else \
            (np.arange(D // 2), np.arange(D // 2, D))
        for m, n in [(0, 0), (3, 10), (10, 3), (500, 77), (65536, 65535)]:
            qm = orc.rope(q[None], np.array([m]), 10000.0, pairing)[0]
            kn = orc.rope(k[None], np.array([n]), 10000.0, pairing)[0]
            dn = n - m
            want = np.sum((q[a] * k[a] + q[b] * k[b]) * np.cos(dn * theta)
                          + (q[b] * k[a] - q[a] * k[b]) * np.sin(dn * theta))
            assert abs(qm @ kn - want) < 1e-9 * (1 + abs(want)), (pairing, m, n)


def check_rope_global_positions(orc):
    """Rank-major rotated rows equal the globally rotated sequence, gathered by
    the layout; rotating by local indices instead (the offset bug the pages
    warn of) changes every rank but rank 0's first chunk."""
    L, N, D = 64, 4, 16
    x = _rand((2, 3, L, D), 12)
    pos = orc.zigzag_layout(L, N)
    for pairing in (orc.ROPE_INTERLEAVED, orc.ROPE_HALF):
        got = orc.permute_to_ranks_rope(x, pos, 10000.0, pairing)
        want = orc.permute_to_ranks(orc.rope(x, np.arange(L), 10000.0, pairing), pos)
        assert np.allclose(got, want, rtol=0, atol=1e-13)
        local = np.stack([orc.rope(x[:, :, pos[r]], np.arange(L // N), 10000.0, pairing)
                          for r in range(N)])
        C = L // (2 * N)
        assert np.allclose(local[0, :, :, :C], got[0, :, :, :C])
        assert not np.allclose(local[0, :, :, C:], got[0, :, :, C:])
        for r in range(1, N):
            assert not np.allclose(local[r], got[r])


# -------------------------------------------------------------- backward pins

def _sdpa_grads(Q, K, V, dO, causal):
    """torch autograd through scaled_dot_product_attention, float64 on the CPU."""
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def check_backward_autograd(orc):
    """Gradients equal torch autograd of SDPA in float64 (causal and not)."""
    for causal, (B, H, L, D), seed in [(True, (2, 2, 37, 16), 30), (False, (1, 3, 29, 8), 31),
                                       (True, (1, 1, 70, 32), 32)]:
        Q, K, V, dO = (_rand((B, H, L, D), seed + 100 * i) for i in range(4))
        got = orc.attention_backward(Q, K, V, dO, causal)
        want = _sdpa_grads(Q, K, V, dO, causal)
        for g, w, name in zip(got, want, "QKV"):
            assert np.max(np.abs(g - w)) < 1e-11, (causal, name, np.max(np.abs(g - w)))


def check_backward_finite_differences(orc):
    """Central differences of sum(dO * O) at every input entry (tiny case)."""
    B, H, L, D = 1, 1, 5, 3
    Q, K, V, dO = (_rand((B, H, L, D), 40 + i) for i in range(4))

    def loss(Q_, K_, V_):
        return float(np.sum(dO * orc.attention(Q_, K_, V_, True)[0]))

    grads = orc.attention_backward(Q, K, V, dO, True)
    h = 1e-6
    for which, g in enumerate(grads):
        for idx in np.ndindex(Q.shape):
            args = [Q.copy(), K.copy(), V.copy()]
            args[which][idx] += h
            up = loss(*args)
            args[which][idx] -= 2 * h
            down = loss(*args)
            assert abs((up - down) / (2 * h) - g[idx]) < 1e-7, (which, idx)


def check_backward_ring_decomposition(orc):
    """Block-by-block ring backward (final lse and delta per query row) over
    a zigzag layout equals the whole-sequence gradients."""
    B, H, L, D, N = 2, 2, 64, 8, 4
    Q, K, V, dO = (_rand((B, H, L, D), 50 + i) for i in range(4))
    dQ, dK, dV = orc.attention_backward(Q, K, V, dO, True)
    O, lse = orc.attention(Q, K, V, True)
    delta = orc.backward_delta(O, dO)
    pos = orc.zigzag_layout(L, N)
    Qr, Kr, Vr, dOr = (orc.permute_to_ranks(x, pos) for x in (Q, K, V, dO))
    lser = np.stack([lse[:, :, pos[r]] for r in range(N)])
    der = np.stack([delta[:, :, pos[r]] for r in range(N)])
    dQr = np.zeros_like(Qr)
    dKr = np.zeros_like(Kr)
    dVr = np.zeros_like(Vr)
    for i in range(N):
        dq, dk, dv = orc.rank_backward(i, Qr[i], Kr, Vr, dOr[i], lser[i], der[i], pos, True)
        dQr[i] = dq
        dKr += dk
        dVr += dv
    for got, want in ((dQr, dQ), (dKr, dK), (dVr, dV)):
        assert np.max(np.abs(orc.permute_from_ranks(got, pos, L) - want)) < 1e-12


def check_backward_invariants(orc):
    """Adding one vector to every key leaves each softmax row unchanged, so
    dK sums to zero over the keys; softmax rows sum to one, so dV sums to the
    sum of dO over the queries; constant V makes O independent of the scores,
    so dQ = dK = 0."""
    B, H, L, D = 1, 2, 48, 16
    Q, K, V, dO = (_rand((B, H, L, D), 60 + i) for i in range(4))
    for causal in (True, False):
        dQ, dK, dV = orc.attention_backward(Q, K, V, dO, causal)
        assert np.max(np.abs(dK.sum(axis=2))) < 1e-12
        assert np.max(np.abs(dV.sum(axis=2) - dO.sum(axis=2))) < 1e-12
        assert np.max(np.abs(dQ)) > 1e-3
    Vc = np.broadcast_to(_rand((B, H, 1, D), 64), (B, H, L, D)).copy()
    dQ, dK, dV = orc.attention_backward(Q, K, Vc, dO, True)
    assert np.max(np.abs(dQ)) < 1e-12 and np.max(np.abs(dK)) < 1e-12


def check_first_non_increasing(orc):
    """Hand-checked tables: equal neighbours break strict increase, a row may
    restart below the previous row's end, one-entry and empty rows pass, and
    the answer is the smallest flat index; the zigzag tables of the workloads
    increase within every rank; and on small random tables the answer is the
    first True of the row-wise difference test, found by np.nonzero."""
    f = orc.first_non_increasing
    assert f([0, 1, 2, 9]) is None
    assert f([0, 1, 1, 2]) == 2
    assert f([5, 4, 3]) == 1
    assert f([[0, 7], [1, 8]]) is None
    assert f([[0, 7], [8, 8]]) == 3
    assert f([[3], [2], [1]]) is None
    assert f(np.zeros((0,), np.int64)) is None
    assert f([[0, 2, 1, 0], [0, 1, 2, 3]]) == 2
    assert f([[0, 1, 2, 3], [9, 8, 10, 11]]) == 5
    for L, N in [(64, 4), (12288, 4), (131072, 4)]:
        assert f(orc.zigzag_layout(L, N)) is None
    rng = np.random.default_rng(5)
    for _ in range(50):
        a = rng.integers(0, 6, size=(3, 5))
        r, c = np.nonzero(np.diff(a, axis=1) <= 0)
        assert f(a) == (None if len(r) == 0 else int(r[0] * 5 + c[0] + 1))


PINS = [check_layout_golden, check_layout_permutation, check_layout_balance, check_ring_order,
        check_permute, check_brute_force, check_sdpa, check_uniform_scores,
        check_constant_v_and_first_row, check_chunk_merge_invariant, check_partial_empty_rows,
        check_merge_algebra, check_structural, check_sampled_rows, check_rope_sinusoid_table,
        check_rope_norm_and_identity, check_rope_relative, check_rope_global_positions,
        check_backward_autograd, check_backward_finite_differences,
        check_backward_ring_decomposition, check_backward_invariants, check_first_non_increasing]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(cpa_oracle)


def test_layout_rejects_bad_sizes():
    for L, N in [(63, 4), (0, 1), (64, 0), (10, 3)]:
        with pytest.raises(ValueError):
            cpa_oracle.zigzag_layout(L, N)


def test_contiguous_layout_is_unbalanced():
    """The plain contiguous split (the first diagram of "序列并行：超长序列训练")
    gives the last rank far more causal work than the first: max/min =
    (N-1) * 2M / (M+1) + 1 for M = L/N tokens per rank."""
    for L, N in [(64, 4), (131072, 4), (1048576, 8)]:
        pos = cpa_oracle.contiguous_layout(L, N)
        c = [cpa_oracle.causal_pairs(pos[r], np.arange(L)) for r in range(N)]
        M = L // N
        assert c[0] == M * (M + 1) // 2 and c[-1] == (N - 1) * M * M + M * (M + 1) // 2
        assert max(c) / min(c) > 6.6


# ------------------------------------------------------ planted mistakes

MUTANTS = {
    "scale 1/D": ("return 1.0 / math.sqrt(D)", "return 1.0 / D"),
    "mask off by one": ("<= np.asarray(q_pos)[:, None]", "< np.asarray(q_pos)[:, None]"),
    "lse sign": ("lse[ok] = m[ok] + np.log(l[ok])", "lse[ok] = m[ok] - np.log(l[ok])"),
    "V row index": ("O[ok] = (w[ok] @ v) / l[ok, None]", "O[ok] = (w[ok] @ v[::-1]) / l[ok, None]"),
    "transposed scores": ("s = (q @ k.T) * scale", "s = (q @ k.T).T[: q.shape[0], : k.shape[0]] * scale"),
    "merge weight sign": ("np.exp(lse_b - M_safe)", "np.exp(M_safe - lse_b)"),
    "merge dropped term": ("(w_a[..., None] * O_a + w_b[..., None] * O_b)", "(w_a[..., None] * O_a)"),
    "merge lse": ("M_safe + np.log(tot_safe)", "M_safe + np.log(tot_safe) / 2"),
    "chunk pairing": ("return r, 2 * N - 1 - r", "return r, N + r"),
    "chunk offset": ("np.arange(hi * C, (hi + 1) * C", "np.arange(hi * C + 1, (hi + 1) * C + 1"),
    "ring direction": ("(i + s) % N for s in range(N)", "(i - s) % N for s in range(N)"),
    "causal key range": ("kend = int(q_pos[a:b].max()) + 1", "kend = int(q_pos[a:b].max())"),
    "inverse permute": ("out[:, :, pos[r]] = y[r]", "out[:, :, pos[r]] = y[0]"),
    "softmax axis": ("l = w.sum(axis=1)", "l = w.sum(axis=1) * (1 + 1e-9)"),
    "empty row lse": ("lse = np.full(q.shape[0], NEG_INF, dtype=np.float64)",
                      "lse = np.full(q.shape[0], 0.0, dtype=np.float64)"),
    "pair count": ("side=\"right\"", "side=\"left\""),
    "rope sin sign": ("y[..., a] = x[..., a] * c - x[..., b] * s",
                      "y[..., a] = x[..., a] * c + x[..., b] * s"),
    "rope frequency": ("np.power(float(base), -2.0 * k / D)", "np.power(float(base), -1.0 * k / D)"),
    "rope pairing": ("return 2 * k, 2 * k + 1", "return 2 * k + 1, 2 * k"),
    "rope half pairing": ("return k, k + D // 2", "return k, D - 1 - k"),
    "rope local positions": ("rope(x[:, :, pos[r]], pos[r], base, pairing)",
                             "rope(x[:, :, pos[r]], np.arange(pos.shape[1]), base, pairing)"),
    "bwd transposed scores": ("s = scale * (q @ k.T)", "s = scale * (k @ q.T)"),
    "bwd delta sign": ("dS = P * (dP - delta[:, None])", "dS = P * (dP + delta[:, None])"),
    "bwd dropped delta": ("dS = P * (dP - delta[:, None])", "dS = P * dP"),
    "bwd dv transposed": ("P.T @ dO", "P @ dO"),
    "bwd dk scale": ("scale * (dS.T @ q)", "(dS.T @ q)"),
    "bwd dq uses v": ("scale * (dS @ k)", "scale * (dS @ v)"),
    "bwd lse": ("np.exp(s - np.where(fin, lse, 0.0)[:, None])[ok]", "np.exp(s)[ok]"),
    "bwd delta definition": ("np.asarray(dO, dtype=np.float64) * np.asarray(O, dtype=np.float64)",
                             "np.asarray(dO, dtype=np.float64) * np.asarray(dO, dtype=np.float64)"),
    "bwd ring block": ("dK[j] += dk", "dK[i] += dk"),
    "bwd causal key range": ("kend = (int(q_pos[a:b].max()) + 1) if causal",
                             "kend = (int(q_pos[a:b].max())) if causal"),
    "offsets not strict": ("if a[r, t] <= a[r, t - 1]:", "if a[r, t] < a[r, t - 1]:"),
    "offsets across rows": ("for t in range(1, n):", "for t in range(n):"),
    "offsets flat index": ("return r * n + t", "return r * n + t - 1"),
    "rope position offset": ("phi = np.asarray(pos, dtype=np.float64)[:, None]",
                             "phi = (np.asarray(pos, dtype=np.float64)[:, None] + 1)"),
}


def _mutant(old, new):
    path = os.path.join(ROOT, "oracle", "cpa_oracle.py")
    with open(path, encoding="utf-8") as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("cpa_oracle_mutant")
    exec(compile(src.replace(old, new), "cpa_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:  # an assertion or a crash both count as caught
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
