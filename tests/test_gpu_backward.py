"""GPU parity of the backward (cpa_backward_delta, cpa_partial_backward,
cpa_rank_backward and the pipeline's backward) against the fp64 oracle,
through the C ABI."""
import sys

import numpy as np
import pytest
import torch

from oracle import cpa_oracle
from parity_helpers import assert_grad_close, host_map, widen

import sequence_attention_cpa_amd as cpa
from sequence_attention_cpa_amd.pipeline import SharePipeline
from sequence_attention_cpa_amd.workloads import (WORKLOADS, make_inputs, make_upstream_grad,
                                                  sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cpa.load()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def offsets(kind, Lq, Lk, seed):
    if kind == "same":
        return np.arange(Lq, dtype=np.int64), np.arange(Lk, dtype=np.int64)
    if kind == "later_k":  # keys after half the queries: many rows see nothing
        return np.arange(Lq, dtype=np.int64), np.arange(Lq // 2, Lq // 2 + Lk, dtype=np.int64)
    if kind == "earlier_k":
        return np.arange(Lk, Lk + Lq, dtype=np.int64), np.arange(Lk, dtype=np.int64)
    g = np.random.default_rng(seed)
    q = np.cumsum(g.integers(1, 4, size=Lq)).astype(np.int64)
    k = np.cumsum(g.integers(1, 4, size=Lk)).astype(np.int64)
    return q, k


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.bfloat16, 16), (torch.float32, 16),
                                     (torch.float32, 64)])
def test_backward_delta(dtype, D):
    rows = 3 * 1000 + 7
    O = rand((rows, D), torch.float32, 80)
    dO = rand((rows, D), dtype, 81)
    got = cpa.backward_delta(O.to(DEV), dO.to(DEV)).cpu().double().numpy()
    ref = cpa_oracle.backward_delta(widen(O), widen(dO))
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)


PARTIAL_BWD_CASES = [
    # dtype, B, H, Lq, Lk, D, causal, offsets
    (torch.bfloat16, 1, 2, 128, 128, 128, True, "same"),
    (torch.bfloat16, 1, 3, 300, 300, 128, True, "same"),       # ragged q and k tiles
    (torch.bfloat16, 2, 2, 256, 512, 128, True, "later_k"),    # empty rows and skipped tiles
    (torch.bfloat16, 1, 2, 256, 384, 128, True, "earlier_k"),  # no mask at all
    (torch.bfloat16, 1, 2, 200, 333, 128, False, "same"),
    (torch.bfloat16, 2, 2, 192, 130, 64, True, "random"),
    (torch.bfloat16, 1, 2, 517, 259, 128, True, "random"),
    (torch.bfloat16, 1, 2, 96, 80, 16, True, "same"),          # bf16 D=16: fp32 row kernels
    (torch.float32, 1, 2, 100, 77, 16, True, "random"),
    (torch.float32, 1, 2, 64, 96, 64, False, "same"),
]


@pytest.mark.parametrize("case", PARTIAL_BWD_CASES, ids=[str(c[1:]) + str(c[0])[-8:]
                                                         for c in PARTIAL_BWD_CASES])
def test_partial_backward(case):
    """One block: lse/delta are the block's own (it is the whole key set);
    the accumulators start from random values to check that calls add."""
    dtype, B, H, Lq, Lk, D, causal, kind = case
    Q, K, V = (rand((B, H, L, D), dtype, s) for L, s in ((Lq, 82), (Lk, 83), (Lk, 84)))
    dO = rand((B, H, Lq, D), dtype, 85)
    q_off, k_off = offsets(kind, Lq, Lk, 86)
    Q64, K64, V64, dO64 = (widen(x) for x in (Q, K, V, dO))
    O, lse = cpa_oracle.partial(Q64, K64, V64, q_off, k_off, causal)
    delta = cpa_oracle.backward_delta(O, dO64)
    ref = cpa_oracle.partial_backward(Q64, K64, V64, dO64, lse, delta, q_off, k_off, causal)
    base = [rand(x.shape, torch.float32, 90 + n) for n, x in enumerate((Q, K, V))]
    acc = [b.to(DEV) for b in base]
    lse_d = torch.from_numpy(lse).float().to(DEV)
    delta_d = cpa.backward_delta(torch.from_numpy(O).float().to(DEV), dO.to(DEV))
    cpa.partial_backward(Q.to(DEV), K.to(DEV), V.to(DEV), dO.to(DEV), lse_d, delta_d,
                         torch.from_numpy(q_off).to(DEV), torch.from_numpy(k_off).to(DEV), causal,
                         *acc)
    torch.cuda.synchronize()
    for name, a, b, r in zip(("dQ", "dK", "dV"), acc, base, ref):
        got = a.cpu().double().numpy() - b.double().numpy()
        e = assert_grad_close(got, r, dtype == torch.bfloat16, f"{case} {name}")
        say(f"partial bwd {case} {name}: {e[0]:.3e} {e[1]:.3e}")


def run_pipeline(Q, K, V, dO, N, causal, fused, rope=None):
    B, H, L, D = Q.shape
    pipe = SharePipeline(B, H, L, D, N, causal, Q.dtype, DEV, fused=fused == True,
                         rope_base=rope, global_layout=fused == "global")
    pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    dQ, dK, dV = pipe.backward(dO.to(DEV))
    torch.cuda.synchronize()
    return [x.cpu().double().numpy() for x in (dQ, dK, dV)]


RANK_BWD_CASES = [
    # dtype, B, H, L, N, D, causal, fused forward
    (torch.bfloat16, 2, 2, 2048, 4, 128, True, True),
    (torch.bfloat16, 1, 3, 4096, 8, 128, True, True),
    (torch.bfloat16, 2, 2, 1024, 4, 64, True, False),
    (torch.bfloat16, 1, 2, 1536, 4, 128, False, True),
    (torch.bfloat16, 1, 2, 2048, 1, 128, True, True),
    (torch.bfloat16, 1, 2, 256, 16, 128, True, True),   # chunks of 8: every tile masked
    (torch.bfloat16, 2, 2, 2048, 4, 128, True, "global"),  # both passes on global layout
    (torch.bfloat16, 1, 3, 4096, 8, 128, True, "global"),
    (torch.bfloat16, 2, 2, 1024, 4, 64, True, "global"),
    (torch.bfloat16, 1, 2, 1536, 4, 128, False, "global"),  # chunks of 192 rows
    (torch.bfloat16, 1, 2, 2048, 1, 128, True, "global"),
    (torch.bfloat16, 1, 2, 768, 4, 128, True, "global"),   # chunks of 96: tiles straddle chunks
    (torch.bfloat16, 2, 2, 320, 5, 64, True, "global"),    # chunks of 32, partial tiles
    (torch.bfloat16, 1, 1, 4096, 64, 64, True, "global"),  # 64 ranks, one tile per chunk
    (torch.bfloat16, 1, 1, 32768, 4, 128, True, "global"),  # 8192 rows per rank: 8-wave dQ pass
    (torch.bfloat16, 1, 1, 32768, 4, 64, True, True),
    (torch.bfloat16, 1, 1, 32768, 4, 64, True, "global"),  # D = 64, 8-wave dQ on global order
    (torch.bfloat16, 1, 1, 33024, 4, 128, True, "global"),  # 8256 rows per rank: 8-wave dQ, ragged
    (torch.bfloat16, 1, 1, 33000, 4, 128, True, True),     # 8250 rows per rank, chunks of 4125
    (torch.bfloat16, 1, 2, 1000, 4, 128, True, True),   # 250 rows per rank: ragged tiles
    (torch.bfloat16, 2, 3, 1000, 4, 64, True, True),
    (torch.float32, 1, 2, 64, 4, 16, True, False),      # the fp32 tiny shape
    (torch.bfloat16, 1, 2, 128, 4, 16, True, False),    # bf16 D=16 (row kernels)
]


@pytest.mark.parametrize("case", RANK_BWD_CASES, ids=[str(c[1:]) + str(c[0])[-8:]
                                                      for c in RANK_BWD_CASES])
def test_ring_backward_all_ranks(case):
    """Forward then backward of every rank through the pipeline, gradients
    stitched back to global order, against the whole-sequence oracle."""
    dtype, B, H, L, N, D, causal, fused = case
    Q, K, V, dO = (rand((B, H, L, D), dtype, 100 + i) for i in range(4))
    got = run_pipeline(Q, K, V, dO, N, causal, fused)
    ref = cpa_oracle.attention_backward(widen(Q), widen(K), widen(V), widen(dO), causal)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = assert_grad_close(g, r, dtype == torch.bfloat16, f"{case} {name}")
        say(f"ring bwd {case} {name}: {e[0]:.3e} {e[1]:.3e}")


def peaked(shape, seed):
    """bf16 Q or K with every 7th / 5th row scaled by 8: scores in the
    hundreds on those rows, so many softmax rows are dominated by one key."""
    Q = rand(shape, torch.float32, seed)
    K = rand(shape, torch.float32, seed + 1)
    Q[:, :, ::7] *= 8
    K[:, :, ::5] *= 8
    return Q.to(torch.bfloat16), K.to(torch.bfloat16)


@pytest.mark.parametrize("D", [128, 64])
def test_partial_backward_large_logits(D):
    """One causal block with outlier-sized scores: P = exp(s - lse) cancels
    two numbers in the hundreds, and dS is dominated by single keys."""
    B, H, L = 1, 2, 320
    Q, K = peaked((B, H, L, D), 140)
    V, dO = rand((B, H, L, D), torch.bfloat16, 142), rand((B, H, L, D), torch.bfloat16, 143)
    off = np.arange(L, dtype=np.int64)
    Q64, K64, V64, dO64 = (widen(x) for x in (Q, K, V, dO))
    O, lse = cpa_oracle.partial(Q64, K64, V64, off, off, True)
    delta = cpa_oracle.backward_delta(O, dO64)
    ref = cpa_oracle.partial_backward(Q64, K64, V64, dO64, lse, delta, off, off, True)
    acc = [torch.zeros(x.shape, dtype=torch.float32, device=DEV) for x in (Q, K, V)]
    offd = torch.from_numpy(off).to(DEV)
    delta_d = cpa.backward_delta(torch.from_numpy(O).float().to(DEV), dO.to(DEV))
    cpa.partial_backward(Q.to(DEV), K.to(DEV), V.to(DEV), dO.to(DEV),
                         torch.from_numpy(lse).float().to(DEV), delta_d, offd, offd, True, *acc)
    torch.cuda.synchronize()
    for name, a, r in zip(("dQ", "dK", "dV"), acc, ref):
        e = assert_grad_close(a.cpu().double().numpy(), r, True, f"large logits D={D} {name}")
        say(f"partial bwd large logits D={D} {name}: {e[0]:.3e} {e[1]:.3e}")


@pytest.mark.parametrize("mode", [True, "global"])
def test_ring_backward_large_logits(mode):
    """Forward then backward of every rank with outlier-sized scores: the
    backward uses the lse the GPU forward produced (lazy rescale included)."""
    B, H, L, N, D = 1, 2, 2048, 4, 128
    Q, K = peaked((B, H, L, D), 150)
    V, dO = rand((B, H, L, D), torch.bfloat16, 152), rand((B, H, L, D), torch.bfloat16, 153)
    got = run_pipeline(Q, K, V, dO, N, True, mode)
    ref = cpa_oracle.attention_backward(widen(Q), widen(K), widen(V), widen(dO), True)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = assert_grad_close(g, r, True, f"large logits {mode} {name}")
        say(f"ring bwd large logits {mode} {name}: {e[0]:.3e} {e[1]:.3e}")


def oracle_backward_heads(Q, K, V, dO, heads, causal=True):
    """attention_backward of selected (b, h) heads, spread over host threads."""
    def one(bh):
        b, h = bh
        q, k, v, g = (widen(x[b, h]) for x in (Q, K, V, dO))
        pos = np.arange(q.shape[0])
        O, lse = cpa_oracle.attention_rows(q, pos, k, v, causal)
        delta = cpa_oracle.backward_delta(O, g)
        return bh, cpa_oracle.backward_rows(q, pos, k, v, g, lse, delta, causal)
    return dict(host_map(one, heads))


def test_ring_backward_12k_eight_heads_every_row():
    """The 12k workload's shape (L = 12288, N = 4, D = 128) on its first 8
    heads, every gradient entry, on rank-major and on global-order data."""
    w = WORKLOADS["12k"]
    Q, K, V, _ = make_inputs(w)
    dO = make_upstream_grad(w)
    Q, K, V, dO = (x[:, :8].contiguous() for x in (Q, K, V, dO))
    say("12k bwd: GPU")
    got = {mode: run_pipeline(Q, K, V, dO, w.N, w.causal, mode) for mode in (True, "global")}
    say("12k bwd: oracle")
    ref = oracle_backward_heads(Q, K, V, dO, [(0, h) for h in range(8)])
    for mode, g in got.items():
        for n, name in enumerate(("dQ", "dK", "dV")):
            r = np.stack([ref[(0, h)][n] for h in range(8)])[None]
            e = assert_grad_close(g[n], r, True, f"12k {mode} {name}")
            say(f"12k bwd {mode} {name}: {e[0]:.3e} {e[1]:.3e}")


@pytest.mark.parametrize("mode", [True, "global"])
def test_ring_backward_128k_sampled(mode):
    """128k workload, all 4 ranks (forward, ring backward; rank-major or on
    global-order data).  dQ at the
    sampled query rows of rank 0 and rank 3; dK, dV at every key of the last
    512 positions (all queries that see them are in the last 512 rows, so the
    oracle needs only those rows); and two sums that hold at any size: dK sums
    to zero over the keys, dV sums to the sum of dO over the queries."""
    w = WORKLOADS["128k"]
    say("128k bwd: generating")
    Q, K, V, outl = make_inputs(w)
    dO = make_upstream_grad(w)
    pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, DEV, fused=True,
                         global_layout=mode == "global")
    pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    dQ, dK, dV = pipe.backward(dO.to(DEV))
    torch.cuda.synchronize()
    pos = pipe.pos_host.numpy()
    rows = np.unique(np.concatenate([pos[r][sample_rows(w, r, pos[r], 128, outl)] for r in (0, 3)]))
    tail = np.arange(w.L - 512, w.L)
    dQs = dQ[:, :, torch.from_numpy(rows).to(DEV)].cpu().double().numpy()
    dKs = dK[:, :, torch.from_numpy(tail).to(DEV)].cpu().double().numpy()
    dVs = dV[:, :, torch.from_numpy(tail).to(DEV)].cpu().double().numpy()
    sum_dK = dK.double().sum(dim=2).cpu().numpy()
    abs_dK = dK.double().abs().sum(dim=2).cpu().numpy()
    sum_dV = dV.double().sum(dim=2).cpu().numpy()
    del pipe, dQ, dK, dV
    say(f"128k bwd: oracle ({len(rows)} query rows, {len(tail)} keys per head)")

    def one(h):
        q, k, v, g = (widen(x[0, h]) for x in (Q, K, V, dO))
        O, lse = cpa_oracle.attention_rows(q[rows], rows, k, v, True, block=32)
        dq, _, _ = cpa_oracle.backward_rows(q[rows], rows, k, v, g[rows], lse,
                                            cpa_oracle.backward_delta(O, g[rows]), True, block=32)
        Ot, lset = cpa_oracle.attention_rows(q[tail], tail, k, v, True, block=32)
        _, dk, dv = cpa_oracle.backward_rows(q[tail], tail, k, v, g[tail], lset,
                                             cpa_oracle.backward_delta(Ot, g[tail]), True,
                                             block=32)
        return h, dq, dk[tail], dv[tail]
    res = dict((h, (a, b, c)) for h, a, b, c in host_map(one, range(w.H)))
    for n, (name, got) in enumerate((("dQ", dQs), ("dK", dKs), ("dV", dVs))):
        r = np.stack([res[h][n] for h in range(w.H)])[None]
        e = assert_grad_close(got, r, True, f"128k {mode} {name}")
        say(f"128k bwd {mode} {name}: {e[0]:.3e} {e[1]:.3e}")
    sum_dO = dO.double().sum(dim=2).numpy()
    assert np.all(np.abs(sum_dK) <= 1e-3 * abs_dK), float(np.max(np.abs(sum_dK) / abs_dK))
    assert np.all(np.abs(sum_dV - sum_dO) <= 1e-3 * dO.double().abs().sum(dim=2).numpy())


def test_partial_backward_explicit_scale():
    """A caller-given scale reaches P, dQ and dK (not only the default 1/sqrt(D))."""
    B, H, L, D, scale = 1, 2, 160, 128, 0.05
    Q, K, V, dO = (rand((B, H, L, D), torch.bfloat16, 120 + i) for i in range(4))
    off = np.arange(L, dtype=np.int64)
    Q64, K64, V64, dO64 = (widen(x) for x in (Q, K, V, dO))
    O, lse = cpa_oracle.partial(Q64, K64, V64, off, off, True, scale)
    delta = cpa_oracle.backward_delta(O, dO64)
    ref = cpa_oracle.partial_backward(Q64, K64, V64, dO64, lse, delta, off, off, True, scale)
    acc = [torch.zeros(x.shape, device=DEV) for x in (Q, K, V)]
    offd = torch.from_numpy(off).to(DEV)
    cpa.partial_backward(Q.to(DEV), K.to(DEV), V.to(DEV), dO.to(DEV),
                         torch.from_numpy(lse).float().to(DEV),
                         torch.from_numpy(delta).float().to(DEV), offd, offd, True, *acc,
                         scale=scale)
    torch.cuda.synchronize()
    for name, a, r in zip(("dQ", "dK", "dV"), acc, ref):
        assert_grad_close(a.cpu().double().numpy(), r, True, f"scale {name}")


def test_share_backward_rank_subset():
    """cpa_share_backward for ranks [1, 3) only: their dQ rows equal the
    oracle's per-rank ring backward, the other ranks' dQ rows stay untouched,
    and dK / dV hold exactly the two ranks' contributions, in global order."""
    B, H, L, N, D, causal = 1, 2, 2048, 4, 128, True
    Q, K, V, dO = (rand((B, H, L, D), torch.bfloat16, 300 + i) for i in range(4))
    pos = cpa.zigzag_layout(L, N)
    posd = pos.to(DEV)
    Qd, Kd, Vd, dOd = (x.to(DEV) for x in (Q, K, V, dO))
    O, lse = cpa.share_forward(Qd, Kd, Vd, N, causal)
    dK = torch.zeros((B, H, L, D), dtype=torch.float32, device=DEV)
    dV = torch.zeros_like(dK)
    dQ = torch.full((B, H, L, D), 7.0, dtype=torch.float32, device=DEV)
    cpa.share_backward(Qd, Kd, Vd, O, dOd, lse, N, causal, dK, dV, rank_lo=1, rank_hi=3,
                       dQ=dQ)
    torch.cuda.synchronize()
    dQ, dK, dV = (x.cpu().double().numpy() for x in (dQ, dK, dV))
    p = pos.numpy()
    q64, k64, v64, g64 = (widen(x) for x in (Q, K, V, dO))
    O64, lse64 = cpa_oracle.attention(q64, k64, v64, causal)
    delta64 = cpa_oracle.backward_delta(O64, g64)
    K_ranks = np.stack([k64[:, :, p[j]] for j in range(N)])
    V_ranks = np.stack([v64[:, :, p[j]] for j in range(N)])
    dK_ref, dV_ref = np.zeros_like(k64), np.zeros_like(v64)
    for i in (1, 2):
        dq, dk, dv = cpa_oracle.rank_backward(i, q64[:, :, p[i]], K_ranks, V_ranks,
                                              g64[:, :, p[i]], lse64[:, :, p[i]],
                                              delta64[:, :, p[i]], p, causal)
        assert_grad_close(dQ[:, :, p[i]], dq, True, f"rank {i} dQ")
        for j in range(N):
            dK_ref[:, :, p[j]] += dk[j]
            dV_ref[:, :, p[j]] += dv[j]
    assert np.all(dQ[:, :, np.concatenate([p[0], p[3]])] == 7.0), "other ranks' dQ rows changed"
    assert_grad_close(dK, dK_ref, True, "dK of ranks 1-2")
    assert_grad_close(dV, dV_ref, True, "dV of ranks 1-2")


@pytest.mark.parametrize("mode", [True, "global"])
def test_ring_backward_with_rope(mode):
    """With RoPE the pipeline's dQ and dK are gradients with respect to the
    rotated Q and K: against the oracle's backward on inputs rotated at their
    global positions (fp64 rotation, rounded to bf16 as the kernels see them)."""
    B, H, L, N, D = 1, 2, 2048, 4, 128
    Q, K, V, dO = (rand((B, H, L, D), torch.bfloat16, 160 + i) for i in range(4))
    got = run_pipeline(Q, K, V, dO, N, True, mode, rope=10000.0)
    pos = np.arange(L)
    Qr, Kr = (torch.from_numpy(cpa_oracle.rope(widen(x), pos, 10000.0, cpa.CPA_ROPE_INTERLEAVED))
              .to(torch.bfloat16) for x in (Q, K))
    ref = cpa_oracle.attention_backward(widen(Qr), widen(Kr), widen(V), widen(dO), True)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        e = assert_grad_close(g, r, True, f"rope {mode} {name}")
        say(f"ring bwd rope {mode} {name}: {e[0]:.3e} {e[1]:.3e}")
