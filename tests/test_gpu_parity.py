"""GPU parity: every call of libcpattn against the CPU fp64 oracle, through the
C ABI (via the thin ctypes binding), on seeded synthetic inputs."""
import math
import sys

import numpy as np
import pytest
import torch

from oracle import cpa_oracle
from parity_helpers import (assert_bf16_close, assert_f32_close, oracle_rows, widen,
                            check_empty_rows)

import sequence_attention_cpa_amd as cpa
from sequence_attention_cpa_amd.pipeline import SharePipeline
from sequence_attention_cpa_amd.workloads import WORKLOADS, make_inputs, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cpa.load()  # fails loudly if libcpattn.so is missing
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rand(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(dtype)


def increasing_offsets(n, seed, start=0):
    """Strictly increasing global positions with random gaps (not a zigzag)."""
    g = np.random.default_rng(seed)
    return start + np.cumsum(g.integers(1, 4, size=n)).astype(np.int64)


def run_partial(Q, K, V, q_off, k_off, causal, scale=0.0):
    O, lse = cpa.partial(Q.to(DEV), K.to(DEV), V.to(DEV), torch.from_numpy(q_off).to(DEV),
                         torch.from_numpy(k_off).to(DEV), causal, scale)
    torch.cuda.synchronize()
    return O.cpu().double().numpy(), lse.cpu().double().numpy()


def oracle_partial(Q, K, V, q_off, k_off, causal, scale=None):
    return cpa_oracle.partial(widen(Q), widen(K), widen(V), q_off, k_off, causal, scale)


# ----------------------------------------------------------------- partial

PARTIAL_CASES = [
    # B, H, Lq, Lk, D, causal, offsets
    (1, 2, 128, 128, 128, True, "same"),       # one tile, diagonal
    (1, 3, 300, 300, 128, True, "same"),       # ragged: 2 full + 1 partial q tile, ragged k tile
    (2, 2, 256, 512, 128, True, "later_k"),    # keys after queries -> mostly empty
    (1, 2, 256, 512, 128, True, "earlier_k"),  # keys before queries -> all visible, no mask
    (1, 2, 200, 333, 128, False, "same"),      # non-causal, ragged both ways
    (2, 2, 192, 130, 64, True, "random"),      # D=64, random increasing offsets
    (1, 4, 128, 64, 64, False, "same"),
    (1, 2, 517, 259, 128, True, "random"),
]


def make_offsets(kind, Lq, Lk, seed):
    if kind == "same":
        return np.arange(Lq, dtype=np.int64), np.arange(Lk, dtype=np.int64)
    if kind == "later_k":
        return np.arange(Lq, dtype=np.int64), np.arange(Lq // 2, Lq // 2 + Lk, dtype=np.int64)
    if kind == "earlier_k":
        return np.arange(Lk, Lk + Lq, dtype=np.int64), np.arange(Lk, dtype=np.int64)
    q = increasing_offsets(Lq, seed)
    k = increasing_offsets(Lk, seed + 1, start=-20)
    return q, k


@pytest.mark.parametrize("case", PARTIAL_CASES, ids=[str(c) for c in PARTIAL_CASES])
def test_partial_mfma_bf16(case):
    B, H, Lq, Lk, D, causal, kind = case
    say("partial mfma", case)
    Q = rand((B, H, Lq, D), torch.bfloat16, 1)
    K = rand((B, H, Lk, D), torch.bfloat16, 2)
    V = rand((B, H, Lk, D), torch.bfloat16, 3)
    q_off, k_off = make_offsets(kind, Lq, Lk, 4)
    O, lse = run_partial(Q, K, V, q_off, k_off, causal)
    Or, lser = oracle_partial(Q, K, V, q_off, k_off, causal)
    assert_bf16_close(O, lse, Or, lser, str(case))


def test_partial_zigzag_small_chunks_bf16():
    """Chunks of 8 tokens (shorter than a 32-key tile): every K tile mixes
    visible and hidden keys of several chunks, for every (i, j) pair."""
    B, H, L, N, D = 1, 2, 256, 16, 128
    pos = cpa_oracle.zigzag_layout(L, N)
    Q = rand((B, H, L, D), torch.bfloat16, 5)
    K = rand((B, H, L, D), torch.bfloat16, 6)
    V = rand((B, H, L, D), torch.bfloat16, 7)
    for i in (0, 5, 15):
        for j in (0, 3, 15):
            pi, pj = torch.from_numpy(pos[i]), torch.from_numpy(pos[j])
            Qi = Q[:, :, pi]
            Kj, Vj = K[:, :, pj].contiguous(), V[:, :, pj].contiguous()
            O, lse = run_partial(Qi.contiguous(), Kj, Vj, pos[i], pos[j], True)
            Or, lser = oracle_partial(Qi, Kj, Vj, pos[i], pos[j], True)
            assert_bf16_close(O, lse, Or, lser, f"i={i} j={j}")


def test_partial_fully_hidden_rows_are_zero_and_neg_inf():
    B, H, L, N, D = 1, 2, 1024, 4, 128
    pos = cpa_oracle.zigzag_layout(L, N)
    C = L // (2 * N)
    Q = rand((B, H, L // N, D), torch.bfloat16, 8)
    K = rand((B, H, L // N, D), torch.bfloat16, 9)
    O, lse = run_partial(Q, K, K, pos[0], pos[2], True)
    assert np.all(O[:, :, :C] == 0) and np.all(np.isneginf(lse[:, :, :C]))
    Or, lser = oracle_partial(Q, K, K, pos[0], pos[2], True)
    assert_bf16_close(O, lse, Or, lser)


@pytest.mark.parametrize("D", [16, 64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_partial_f32(D, causal):
    """fp32 inputs: fp32 arithmetic end to end, relative error <= 1e-5."""
    B, H, Lq, Lk = 1, 2, 40, 72
    Q = rand((B, H, Lq, D), torch.float32, 10)
    K = rand((B, H, Lk, D), torch.float32, 11)
    V = rand((B, H, Lk, D), torch.float32, 12)
    q_off = np.arange(30, 30 + Lq, dtype=np.int64)
    k_off = np.arange(Lk, dtype=np.int64)
    O, lse = run_partial(Q, K, V, q_off, k_off, causal)
    Or, lser = oracle_partial(Q, K, V, q_off, k_off, causal)
    assert_f32_close(O, lse, Or, lser)


def test_partial_bf16_d16_rowwise():
    Q, K, V = (rand((2, 2, 50, 16), torch.bfloat16, s) for s in (13, 14, 15))
    off = np.arange(50, dtype=np.int64)
    O, lse = run_partial(Q, K, V, off, off, True)
    Or, lser = oracle_partial(Q, K, V, off, off, True)
    assert_bf16_close(O, lse, Or, lser)


def test_partial_explicit_scale():
    Q, K, V = (rand((1, 2, 130, 128), torch.bfloat16, s) for s in (16, 17, 18))
    off = np.arange(130, dtype=np.int64)
    O, lse = run_partial(Q, K, V, off, off, True, scale=0.05)
    Or, lser = oracle_partial(Q, K, V, off, off, True, scale=0.05)
    assert_bf16_close(O, lse, Or, lser)


def test_partial_empty_inputs():
    Q = rand((1, 2, 70, 128), torch.bfloat16, 19)
    K = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16)
    O, lse = run_partial(Q, K, K, np.arange(70, dtype=np.int64), np.zeros(0, dtype=np.int64), True)
    assert np.all(O == 0) and np.all(np.isneginf(lse))
    E = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device=DEV)
    Oe, le = cpa.partial(E, E, E, torch.zeros(0, dtype=torch.int64, device=DEV),
                         torch.zeros(0, dtype=torch.int64, device=DEV), True)
    assert Oe.numel() == 0 and le.numel() == 0


def test_partial_large_logits():
    """Outlier-sized scores (|s| in the hundreds) exercise the running-max rescale."""
    Q = rand((1, 2, 256, 128), torch.float32, 20)
    K = rand((1, 2, 256, 128), torch.float32, 21)
    Q[:, :, ::7] *= 8
    K[:, :, ::5] *= 8
    Q, K = Q.to(torch.bfloat16), K.to(torch.bfloat16)
    V = rand((1, 2, 256, 128), torch.bfloat16, 22)
    off = np.arange(256, dtype=np.int64)
    O, lse = run_partial(Q, K, V, off, off, True)
    Or, lser = oracle_partial(Q, K, V, off, off, True)
    assert_bf16_close(O, lse, Or, lser)


def test_partial_deterministic():
    Q, K, V = (rand((1, 4, 640, 128), torch.bfloat16, s).to(DEV) for s in (23, 24, 25))
    off = torch.arange(640, dtype=torch.int64, device=DEV)
    a = [t.clone() for t in cpa.partial(Q, K, V, off, off, True)]
    b = cpa.partial(Q, K, V, off, off, True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------- merge

def test_merge_vs_oracle():
    rows, D = 3000, 128
    g = torch.Generator().manual_seed(30)
    Oa, Ob = torch.randn(rows, D, generator=g), torch.randn(rows, D, generator=g)
    la, lb = torch.randn(rows, generator=g) * 20, torch.randn(rows, generator=g) * 20
    la[::11] = float("-inf")
    lb[::13] = float("-inf")
    la[::77] = float("-inf")
    lb[::77] = float("-inf")
    Oa[::11] = 0
    Ob[::13] = 0
    Oa[::77] = 0
    Ob[::77] = 0
    Or, lr = cpa_oracle.merge(Oa.double().numpy(), la.double().numpy(), Ob.double().numpy(),
                              lb.double().numpy())
    Od, ld, Obd, lbd = (t.to(DEV) for t in (Oa, la, Ob, lb))
    cpa.merge(Od, ld, Obd, lbd)
    torch.cuda.synchronize()
    assert_f32_close(Od.cpu().double().numpy(), ld.cpu().double().numpy(), Or, lr)


@pytest.mark.parametrize("D", [16, 64])
def test_merge_small_d(D):
    g = torch.Generator().manual_seed(31)
    Oa, Ob = torch.randn(257, D, generator=g), torch.randn(257, D, generator=g)
    la, lb = torch.randn(257, generator=g), torch.randn(257, generator=g)
    Or, lr = cpa_oracle.merge(Oa.double().numpy(), la.double().numpy(), Ob.double().numpy(),
                              lb.double().numpy())
    Od, ld = Oa.to(DEV), la.to(DEV)
    cpa.merge(Od, ld, Ob.to(DEV), lb.to(DEV))
    torch.cuda.synchronize()
    assert_f32_close(Od.cpu().double().numpy(), ld.cpu().double().numpy(), Or, lr)


# ----------------------------------------------------------------- permute

@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64),
                                     (torch.float32, 1), (torch.bfloat16, 4),
                                     (torch.float64, 3)])
@pytest.mark.parametrize("ranks", [(0, 4), (1, 3), (3, 4)])
def test_permute_bit_exact(dtype, D, ranks):
    B, H, L, N = 2, 3, 192, 4
    pos = cpa_oracle.zigzag_layout(L, N)
    x = rand((B, H, L, D), torch.float32, 40).to(dtype)
    lo, hi = ranks
    src = x[..., 0] if D == 1 else x
    pos_d = torch.from_numpy(pos).to(DEV)
    y = cpa.zigzag_permute(src.to(DEV), pos_d, N, rank_lo=lo, rank_hi=hi)
    want = cpa_oracle.permute_to_ranks(x.numpy() if dtype != torch.bfloat16 else x.view(torch.int16).numpy(), pos)[lo:hi]
    got = y.cpu()
    got = got.view(torch.int16).numpy() if dtype == torch.bfloat16 else got.numpy()
    if D == 1:
        want = want[..., 0]
    assert np.array_equal(got, want)
    back = cpa.zigzag_permute(y, pos_d, N, inverse=True, rank_lo=lo, rank_hi=hi)
    torch.cuda.synchronize()
    b = back.cpu()
    rows = np.sort(pos[lo:hi].ravel())
    assert torch.equal(b[:, :, rows], src[:, :, rows])
    other = np.setdiff1d(np.arange(L), rows)
    assert torch.all(b[:, :, other] == 0)


# ------------------------------------------------------------ rank forward

def stitched_all_ranks(w, Q, K, V, fused=False, global_layout=False):
    pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, DEV, fused=fused,
                         global_layout=global_layout)
    O, lse = pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    torch.cuda.synchronize()
    return O.cpu().double().numpy(), lse.cpu().double().numpy()


def test_rank_forward_tiny_f32_all_ranks():
    w = WORKLOADS["tiny"]
    Q, K, V, _ = make_inputs(w)
    O, lse = stitched_all_ranks(w, Q, K, V)
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), w.causal)
    assert_f32_close(O, lse, Or, lr)


def test_rank_forward_demo_bf16_all_ranks():
    w = WORKLOADS["demo"]
    Q, K, V, _ = make_inputs(w)
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), w.causal)
    for fused in (False, True):
        O, lse = stitched_all_ranks(w, Q, K, V, fused)
        assert_bf16_close(O, lse, Or, lr, f"demo fused={fused}")


def test_rank_forward_12k_all_ranks_every_row():
    w = WORKLOADS["12k"]
    say("12k: generating")
    Q, K, V, _ = make_inputs(w)
    say("12k: GPU")
    outs = {f: stitched_all_ranks(w, Q, K, V, f) for f in (False, True)}
    outs["global"] = stitched_all_ranks(w, Q, K, V, True, global_layout=True)
    say("12k: oracle")
    rows = {(b, h): np.arange(w.L) for b in range(w.B) for h in range(w.H)}
    ref = oracle_rows(lambda b, h: widen(Q[b, h]), lambda b, h: widen(K[b, h]),
                      lambda b, h: widen(V[b, h]), rows, w.causal)
    Or = np.stack([np.stack([ref[(b, h)][0] for h in range(w.H)]) for b in range(w.B)])
    lr = np.stack([np.stack([ref[(b, h)][1] for h in range(w.H)]) for b in range(w.B)])
    for f, (O, lse) in outs.items():
        mx, mean = assert_bf16_close(O, lse, Or, lr, f"12k fused={f}")
        say(f"12k fused={f}: max {mx:.3e} mean {mean:.3e}")


def share_check(name, rank, n_rows, block):
    w = WORKLOADS[name]
    say(f"{name}: generating")
    Q, K, V, outl = make_inputs(w)
    Qd, Kd, Vd = Q.to(DEV), K.to(DEV), V.to(DEV)
    results = {}
    pos = None
    modes = (False, True, "global", "precise")
    for fused in modes:
        say(f"{name}: GPU rank {rank} fused={fused}")
        pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, DEV, rank, rank + 1,
                             fused=bool(fused), global_layout=fused in ("global", "precise"))
        if fused == "precise":
            Od, lsed = cpa.share_forward(Qd, Kd, Vd, w.N, w.causal, rank_lo=rank,
                                         rank_hi=rank + 1, precise=True)
        else:
            Od, lsed = pipe.step(Qd, Kd, Vd)
        pos = pipe.pos_host.numpy()
        if "g" not in results:
            t = sample_rows(w, rank, pos[rank], n_rows // (w.B * w.H), outl)
            results["g"] = pos[rank][t]
        gi = torch.from_numpy(results["g"]).to(DEV)
        results[fused] = (Od[:, :, gi].cpu().double().numpy(), lsed[:, :, gi].cpu().double().numpy())
        del pipe, Od, lsed
        torch.cuda.synchronize()
    g = results["g"]
    say(f"{name}: oracle on {len(g)} rows x {w.B * w.H} heads")
    rows = {(b, h): g for b in range(w.B) for h in range(w.H)}
    ref = oracle_rows(lambda b, h: widen(Q[b, h]), lambda b, h: widen(K[b, h]),
                      lambda b, h: widen(V[b, h]), rows, w.causal, block=block)
    Or = np.stack([np.stack([ref[(b, h)][0] for h in range(w.H)]) for b in range(w.B)])
    lr = np.stack([np.stack([ref[(b, h)][1] for h in range(w.H)]) for b in range(w.B)])
    for fused in modes:
        O, lse = results[fused]
        # bf16 weights leave an error in O proportional to V's largest rows;
        # the precise weights do not, so their bounds stay unscaled.
        v_scale = w.outlier_mult if w.outlier_in_v and fused != "precise" else 1.0
        mx, mean = assert_bf16_close(O, lse, Or, lr, f"{name} fused={fused}", v_scale)
        say(f"{name} fused={fused}: max {mx:.3e} mean {mean:.3e}")
        if fused == "precise":
            assert mx <= PRECISE_MAX_ABS and mean <= PRECISE_MEAN_ABS, (mx, mean)


# The precise-weight ring carries each weight to a relative 2^-16 (bf16 hi/lo
# pair), so its O error is that of the fp32 accumulation, far below the bf16
# bounds; its own bounds sit about 3x above the largest errors it showed
# (3.4e-4 max with V rows scaled by 64, 3.0e-4 on the V-outlier share).
PRECISE_MAX_ABS = 1e-3
PRECISE_MEAN_ABS = 1e-4


@pytest.mark.parametrize("rank", [0, 3])
def test_rank_forward_128k_share_sampled(rank):
    share_check("128k", rank, 1024, 32)


def test_rank_forward_128k_outliers_in_v_sampled():
    """The 128k share with the outlier token rows scaled in V as well as in Q
    and K: sampled rows of rank 0, every forward mode.  V's outlier rows are 8
    times larger, and so are the O bounds of the bf16-weight modes; the
    precise-weight ring (cpa_share_forward_precise) meets the unscaled
    bounds."""
    share_check("128k_qkv", 0, 512, 32)


@pytest.mark.timeout(900)
def test_rank_forward_1m_share_sampled():
    share_check("1m", 0, 256, 8)


FUSED_CASES = [
    # B, H, L, N, D, causal
    (2, 2, 2048, 1, 128, True),
    (1, 2, 2048, 2, 128, True),
    (1, 3, 4096, 8, 128, True),
    (2, 2, 1024, 4, 64, True),
    (1, 2, 1536, 4, 128, False),
    (1, 2, 256, 16, 128, True),   # chunks of 8 keys: every tile of every block is masked
    (1, 2, 1000, 4, 128, True),   # 250 rows per rank: ragged query and key tiles
    (2, 3, 1000, 4, 64, True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[str(c) for c in FUSED_CASES])
def test_rank_forward_fused_small_shapes(case):
    """The one-launch ring equals the oracle for every rank, at shapes that span
    several tiles, ragged tails, N = 1 and chunks shorter than a tile."""
    B, H, L, N, D, causal = case
    Q = rand((B, H, L, D), torch.bfloat16, 60)
    K = rand((B, H, L, D), torch.bfloat16, 61)
    V = rand((B, H, L, D), torch.bfloat16, 62)
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), causal)
    pipe = SharePipeline(B, H, L, D, N, causal, Q.dtype, DEV, fused=True)
    O, lse = pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    torch.cuda.synchronize()
    assert_bf16_close(O.cpu().double().numpy(), lse.cpu().double().numpy(), Or, lr, str(case))


@pytest.mark.parametrize("D", [128, 64])
def test_rank_forward_fused_contiguous_split(D):
    """The one-launch ring takes any increasing position table: a contiguous
    split (rank r holds tokens [r L/N, (r+1) L/N), the unbalanced layout the
    zigzag replaces) gives every rank its rows of whole-sequence attention."""
    B, H, L, N = 1, 2, 2048, 4
    Lr = L // N
    Q, K, V = (rand((B, H, L, D), torch.bfloat16, 70 + i) for i in range(3))
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), True)
    pos = torch.arange(L, dtype=torch.int64).reshape(N, Lr).to(DEV)
    Kc = cpa.zigzag_permute(K.to(DEV), pos, N)
    Vc = cpa.zigzag_permute(V.to(DEV), pos, N)
    Qc = cpa.zigzag_permute(Q.to(DEV), pos, N)
    for r in range(N):
        O, lse = cpa.rank_forward_fused(r, N, Qc[r], Kc, Vc, pos, True)
        torch.cuda.synchronize()
        rows = slice(r * Lr, (r + 1) * Lr)
        assert_bf16_close(O.cpu().double().numpy(), lse.cpu().double().numpy(),
                          Or[:, :, rows], lr[:, :, rows], f"contiguous rank {r} D={D}")


SHARE_CASES = [c for c in FUSED_CASES if (c[2] // c[3] // 2) % 32 == 0] + [
    # chunks that are not multiples of the 128-row workgroup: a workgroup's
    # waves straddle the rank's two chunks, and the last one is partial
    (1, 2, 768, 4, 128, True),    # C = 96
    (2, 2, 320, 5, 64, True),     # C = 32, one 64-row workgroup per rank
    (1, 1, 1280, 4, 128, True),   # C = 160
    (1, 1, 4096, 64, 64, True),   # 64 ranks: 64-block rings over 128 chunks of one tile each
]


@pytest.mark.parametrize("case", SHARE_CASES, ids=[str(c) for c in SHARE_CASES])
def test_share_forward_global_layout(case):
    """The global-layout ring (zigzag permute folded into the kernel) equals
    the oracle for every rank; rows are read and written in global order."""
    B, H, L, N, D, causal = case
    Q = rand((B, H, L, D), torch.bfloat16, 63)
    K = rand((B, H, L, D), torch.bfloat16, 64)
    V = rand((B, H, L, D), torch.bfloat16, 65)
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), causal)
    pipe = SharePipeline(B, H, L, D, N, causal, Q.dtype, DEV, fused=True, global_layout=True)
    O, lse = pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    torch.cuda.synchronize()
    assert_bf16_close(O.cpu().double().numpy(), lse.cpu().double().numpy(), Or, lr, str(case))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", list(range(1, 11)))
def test_share_forward_block_lengths(tiles, causal):
    """Chunks of 1 to 10 key tiles (blocks of 2 to 20): the steady loop's
    whole trips over the 8 LDS buffers, its remaining pairs, an unpaired last
    tile and the masked pairs of crossing tiles all meet the oracle."""
    B, H, N, D = 1, 2, 4, 128
    L = 2 * N * 32 * tiles
    Q, K, V = (rand((B, H, L, D), torch.bfloat16, 90 + i) for i in range(3))
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), causal)
    O, lse = cpa.share_forward(Q.to(DEV), K.to(DEV), V.to(DEV), N, causal)
    torch.cuda.synchronize()
    assert_bf16_close(O.cpu().double().numpy(), lse.cpu().double().numpy(), Or, lr,
                      f"C={32 * tiles} causal={causal}")


@pytest.mark.parametrize("case", SHARE_CASES, ids=[str(c) for c in SHARE_CASES])
def test_share_forward_precise(case):
    """The precise-weight ring equals the oracle for every rank, and its O
    error stays small when some V rows are 64 times larger than the rest
    (rows of Q, K and V scaled together, as in the outlier workloads)."""
    B, H, L, N, D, causal = case
    Q = rand((B, H, L, D), torch.bfloat16, 63)
    K = rand((B, H, L, D), torch.bfloat16, 64)
    V = rand((B, H, L, D), torch.float32, 65)
    rows = torch.from_numpy(np.random.default_rng(5).choice(L, size=max(1, L // 50),
                                                             replace=False))
    V[:, :, rows] *= 64.0
    V = V.to(torch.bfloat16)
    Or, lr = cpa_oracle.attention(widen(Q), widen(K), widen(V), causal)
    O, lse = cpa.share_forward(Q.to(DEV), K.to(DEV), V.to(DEV), N, causal, precise=True)
    torch.cuda.synchronize()
    mx, mean = assert_bf16_close(O.cpu().double().numpy(), lse.cpu().double().numpy(), Or, lr,
                                 str(case))
    say(f"precise {case}: max {mx:.3e} mean {mean:.3e}")
    assert mx <= PRECISE_MAX_ABS and mean <= PRECISE_MEAN_ABS, (mx, mean)


def test_share_forward_rank_subset_leaves_other_rows():
    """Only the selected ranks' rows are written."""
    B, H, L, N, D = 1, 2, 2048, 4, 128
    Q, K, V = (rand((B, H, L, D), torch.bfloat16, 66 + i).to(DEV) for i in range(3))
    pos = cpa.zigzag_layout(L, N)
    O = torch.full((B, H, L, D), 7.0, device=DEV)
    lse = torch.full((B, H, L), 7.0, device=DEV)
    cpa.share_forward(Q, K, V, N, True, rank_lo=1, rank_hi=3, out=O, lse=lse)
    torch.cuda.synchronize()
    mine = np.concatenate([pos[1].numpy(), pos[2].numpy()])
    other = np.setdiff1d(np.arange(L), mine)
    assert torch.all(O[:, :, torch.from_numpy(other).to(DEV)] == 7.0)
    assert torch.all(lse[:, :, torch.from_numpy(other).to(DEV)] == 7.0)
    Or, lr = cpa_oracle.attention(widen(Q.cpu()), widen(K.cpu()), widen(V.cpu()), True)
    gi = torch.from_numpy(mine).to(DEV)
    assert_bf16_close(O[:, :, gi].cpu().double().numpy(), lse[:, :, gi].cpu().double().numpy(),
                      Or[:, :, mine], lr[:, :, mine], "ranks 1-2")
