"""GPU check of the position-table precondition (cpa_check_offsets) against the
oracle's plain scan, bit-exact, through the C ABI; and the binding's debug
mode that runs it before causal calls."""
import sys

import numpy as np
import pytest
import torch

from oracle import cpa_oracle

import sequence_attention_cpa_amd as cpa
from sequence_attention_cpa_amd.workloads import WORKLOADS

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


def device_answer(table):
    return cpa.check_offsets(torch.from_numpy(np.ascontiguousarray(table)).to(DEV))


def planted(table, edits):
    t = table.copy()
    for (r, c), v in edits:
        t[r, c] = v
    return t


@pytest.mark.parametrize("name", ["tiny", "demo", "12k", "128k", "1m"])
def test_zigzag_tables_and_planted_breaks(name):
    """Every workload's zigzag table passes; breaks planted at the first and
    last entries of a rank, at the jump from its early to its late chunk, and
    two at once (the smaller index wins) are found where the oracle finds
    them; lowering a rank's first entry below the previous rank's last is no
    break."""
    w = WORKLOADS[name]
    pos = cpa_oracle.zigzag_layout(w.L, w.N)
    N, n = pos.shape
    C = n // 2
    last = N - 1
    cases = {
        "as laid out": [],
        "equal at entry 1": [((0, 1), pos[0, 0])],
        "last entry of the last rank": [((last, n - 1), pos[last, n - 2] - 3)],
        "late chunk starts too low": [((last // 2, C), pos[last // 2, C - 1])],
        "two breaks": [((last, 5), pos[last, 4]), ((last, n - 1), pos[last, 0])],
        "rank restarts low": [((last, 0), -7)],
    }
    for label, edits in cases.items():
        t = planted(pos, edits)
        want = cpa_oracle.first_non_increasing(t)
        say(f"{name} {label}: oracle {want}")
        assert device_answer(t) == want, label
    assert cpa_oracle.first_non_increasing(planted(pos, cases["rank restarts low"])) is None


@pytest.mark.parametrize("rows,n,seed", [(3, 257, 1), (1, 4099, 2), (7, 33, 3), (2, 1, 4)])
def test_random_tables(rows, n, seed):
    """Ragged sizes: increasing rows with random gaps, then a few random
    entries overwritten."""
    rng = np.random.default_rng(seed)
    base = np.cumsum(rng.integers(1, 5, size=(rows, n)), axis=1).astype(np.int64)
    assert device_answer(base) == cpa_oracle.first_non_increasing(base) is None
    for k in range(4):
        t = base.copy()
        for _ in range(k + 1):
            t[rng.integers(rows), rng.integers(n)] = rng.integers(0, 4 * n)
        want = cpa_oracle.first_non_increasing(t)
        assert device_answer(t) == want, (k, want)


def test_one_dimensional_and_empty_tables():
    assert device_answer(np.array([4, 9, 10], dtype=np.int64)) is None
    assert device_answer(np.array([4, 9, 9], dtype=np.int64)) == 2
    assert device_answer(np.zeros((0,), dtype=np.int64)) is None
    assert device_answer(np.zeros((3, 0), dtype=np.int64)) is None


def test_debug_mode_rejects_bad_tables_before_causal_calls():
    """With the debug switch on, a causal call whose table is not strictly
    increasing raises CPA_EINVAL and launches nothing; a good table runs."""
    g = torch.Generator().manual_seed(11)
    B, H, L, D, N = 1, 2, 256, 64, 2
    Q, K, V = (torch.randn((B, H, L, D), generator=g).to(torch.bfloat16).to(DEV) for _ in range(3))
    good = torch.arange(L, dtype=torch.int64, device=DEV)
    bad = good.clone()
    bad[100] = bad[99]
    pos = torch.from_numpy(cpa_oracle.zigzag_layout(L, N)).to(DEV)
    pos_bad = pos.clone()
    pos_bad[1, 70] = pos_bad[1, 69]
    cpa.debug_offsets(True)
    try:
        for kw in (dict(q_off=bad, k_off=good), dict(q_off=good, k_off=bad)):
            with pytest.raises(cpa.CpaError) as e:
                cpa.partial(Q, K, V, causal=True, **kw)
            assert e.value.status == cpa.CPA_EINVAL and "entry 100" in str(e.value)
        cpa.partial(Q, K, V, good, good, causal=True)
        with pytest.raises(cpa.CpaError) as e:
            cpa.rank_forward_fused(1, N, Q[:, :, :L // N].contiguous(),
                                   torch.stack([K[:, :, :L // N], K[:, :, L // N:]]).contiguous(),
                                   torch.stack([V[:, :, :L // N], V[:, :, L // N:]]).contiguous(),
                                   pos_bad, causal=True)
        assert "pos_all" in str(e.value) and "row 1, entry 70" in str(e.value)
        torch.cuda.synchronize()
    finally:
        cpa.debug_offsets(False)


def test_debug_mode_covers_the_ring_and_backward_calls():
    """The rank-major ring, the partial backward, the ring backward and the
    global-layout backward also refuse a bad table before launching."""
    g = torch.Generator().manual_seed(12)
    B, H, L, D, N = 1, 1, 256, 64, 2
    Lr = L // N
    bf = dict(dtype=torch.bfloat16)
    f32 = dict(dtype=torch.float32, device=DEV)
    Q, K, V, dO = (torch.randn((B, H, L, D), generator=g).to(**bf).to(DEV) for _ in range(4))
    Kr, Vr = (torch.randn((N, B, H, Lr, D), generator=g).to(**bf).to(DEV) for _ in range(2))
    Qi, dOi = (torch.randn((B, H, Lr, D), generator=g).to(**bf).to(DEV) for _ in range(2))
    pos = torch.from_numpy(cpa_oracle.zigzag_layout(L, N)).to(DEV)
    bad_pos = pos.clone()
    bad_pos[0, 3] = bad_pos[0, 2]
    bad_off = torch.arange(Lr, dtype=torch.int64, device=DEV)
    bad_off[5] = bad_off[4]
    good_off = torch.arange(Lr, dtype=torch.int64, device=DEV)
    O, lse = torch.zeros((B, H, L, D), **f32), torch.zeros((B, H, L), **f32)
    Oi, lsei = torch.zeros((B, H, Lr, D), **f32), torch.zeros((B, H, Lr), **f32)
    dK, dV, dQ = (torch.zeros((B, H, L, D), **f32) for _ in range(3))
    dKr, dVr = torch.zeros((N, B, H, Lr, D), **f32), torch.zeros((N, B, H, Lr, D), **f32)
    dQi, dKi, dVi = (torch.zeros((B, H, Lr, D), **f32) for _ in range(3))
    calls = {
        "rank_forward_fused": lambda: cpa.rank_forward_fused(0, N, Qi, Kr, Vr, bad_pos, True),
        "partial_backward": lambda: cpa.partial_backward(Qi, Qi, Qi, dOi, lsei, lsei, good_off,
                                                         bad_off, True, dQi, dKi, dVi),
        "rank_backward": lambda: cpa.rank_backward(0, N, Qi, Kr, Vr, bad_pos, Oi, dOi, lsei, True,
                                                   dKr, dVr),
    }
    cpa.debug_offsets(True)
    try:
        for name, call in calls.items():
            with pytest.raises(cpa.CpaError) as e:
                call()
            assert e.value.status == cpa.CPA_EINVAL, name
            say(f"debug offsets, {name}: {e.value}")
        torch.cuda.synchronize()
    finally:
        cpa.debug_offsets(False)
