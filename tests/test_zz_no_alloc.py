"""GPU check of cpa_rank_forward_noalloc, the rank ring that keeps its partial
in the library's own device scratch: its output against cpa_rank_forward's
(the same ring with a caller workspace) on the same inputs, several calls in
a row on one device, each later one smaller than one before it, covering
whole-rank, head-sliced and row-sliced use of the scratch."""
import sys

import numpy as np
import pytest
import torch

import sequence_attention_cpa_amd as cpa

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
# bf16 parity bar of the workloads: max |dO| 1e-2, mean |dO| 1e-3,
# |dlse| <= 1e-3 max(1, |lse|); fp32: 1e-5 relative.
BF16_MAX, BF16_MEAN, LSE_REL = 1e-2, 1e-3, 1e-3


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cpa.load()  # fails loudly if libcpattn.so is missing


def rand(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def call_noalloc(i, N, Q_i, K_all, V_all, pos, causal):
    """Through the binding (C ABI); outputs start as NaN so unwritten rows show."""
    B, H, Lr, D = Q_i.shape
    O = torch.full((B, H, Lr, D), float("nan"), dtype=torch.float32, device=DEV)
    lse = torch.full((B, H, Lr), float("nan"), dtype=torch.float32, device=DEV)
    return cpa.rank_forward_noalloc(i, N, Q_i, K_all, V_all, pos, causal, out=O, lse=lse)


# (dtype, B, H, L, N, D, causal, rank): first a rank whose partial spans four
# head slices of the scratch, then one whose heads are cut into row slices,
# then ranks that fit whole, an fp32 ring and a one-rank ring (no scratch).
CASES = [
    (torch.bfloat16, 1, 32, 12288, 4, 128, True, 1),
    (torch.bfloat16, 1, 1, 262144, 4, 128, True, 0),
    (torch.bfloat16, 2, 2, 1024, 4, 64, True, 3),
    (torch.bfloat16, 1, 2, 4096, 2, 128, False, 1),
    (torch.float32, 1, 2, 64, 4, 16, True, 2),
    (torch.bfloat16, 1, 2, 512, 1, 128, True, 0),
]


def test_noalloc_matches_workspace_ring():
    for k, (dtype, B, H, L, N, D, causal, rank) in enumerate(CASES):
        print(f"noalloc case {k}: {dtype} B={B} H={H} L={L} N={N} D={D} causal={causal} "
              f"rank={rank}", file=sys.stderr, flush=True)
        Lr = L // N
        Q = rand((B, H, Lr, D), dtype, 10 * k + 1).to(DEV)
        K = rand((N, B, H, Lr, D), dtype, 10 * k + 2).to(DEV)
        V = rand((N, B, H, Lr, D), dtype, 10 * k + 3).to(DEV)
        pos = cpa.zigzag_layout(L, N).to(DEV)
        O_ref, l_ref = cpa.rank_forward(rank, N, Q, K, V, pos, causal)
        O, l = call_noalloc(rank, N, Q, K, V, pos, causal)
        torch.cuda.synchronize()
        O, l, O_ref, l_ref = (t.cpu().double().numpy() for t in (O, l, O_ref, l_ref))
        assert np.isfinite(O).all() and np.isfinite(l).all(), f"case {k}: unwritten rows"
        d, dl = np.abs(O - O_ref), np.abs(l - l_ref)
        if dtype == torch.float32:
            assert np.all(d <= 1e-6 + 1e-5 * np.abs(O_ref)), f"case {k}: max |dO| {d.max():.3e}"
            assert np.all(dl <= 1e-6 + 1e-5 * np.abs(l_ref)), f"case {k}: max |dlse| {dl.max():.3e}"
        else:
            assert d.max() <= BF16_MAX, f"case {k}: max |dO| {d.max():.3e}"
            assert d.mean() <= BF16_MEAN, f"case {k}: mean |dO| {d.mean():.3e}"
            assert np.all(dl <= LSE_REL * np.maximum(1.0, np.abs(l_ref))), \
                f"case {k}: max |dlse| {dl.max():.3e}"
