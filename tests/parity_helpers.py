"""Shared helpers of the GPU parity tests: tolerances and a threaded driver
for the oracle (the oracle itself stays single-threaded and plain; rows and
heads are independent, so the tests spread them over host threads)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import cpa_oracle

# bf16 inputs vs the fp64 oracle: max |dO| <= 1e-2 and mean |dO| <= 1e-3 over
# all checked elements; lse within 1e-3 * max(1, |lse|) (fp32 score
# accumulation of large outlier logits); empty rows exactly (0, -inf).
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
LSE_REL = 1e-3
# fp32 inputs: the pages' own check, assert_allclose(rtol=1e-5, atol=1e-6).
F32_RTOL, F32_ATOL = 1e-5, 1e-6


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def widen(t):
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_empty_rows(O, lse, O_ref, lse_ref):
    neg = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), neg), "rows without visible keys differ"
    assert np.all(O[neg] == 0.0), "rows without visible keys must have O = 0"
    assert not np.any(np.isnan(O)) and not np.any(np.isnan(lse))
    return ~neg


def assert_bf16_close(O, lse, O_ref, lse_ref, what=""):
    fin = check_empty_rows(O, lse, O_ref, lse_ref)
    d = np.abs(O - O_ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    assert mx <= BF16_MAX_ABS, f"{what}: max |dO| {mx:.3e} > {BF16_MAX_ABS}"
    assert mean <= BF16_MEAN_ABS, f"{what}: mean |dO| {mean:.3e} > {BF16_MEAN_ABS}"
    dl = np.abs(lse[fin] - lse_ref[fin])
    bound = LSE_REL * np.maximum(1.0, np.abs(lse_ref[fin]))
    assert np.all(dl <= bound), f"{what}: lse off by {float((dl / bound).max()):.2f}x tolerance"
    return mx, mean


def assert_f32_close(O, lse, O_ref, lse_ref):
    fin = check_empty_rows(O, lse, O_ref, lse_ref)
    np.testing.assert_allclose(O, O_ref, rtol=F32_RTOL, atol=F32_ATOL)
    np.testing.assert_allclose(lse[fin], lse_ref[fin], rtol=F32_RTOL, atol=F32_ATOL)


def oracle_rows(Q64, K64, V64, rows_by_bh, causal, scale=None, block=64):
    """Oracle O/lse at global query positions rows_by_bh[(b, h)] for every
    (b, h), heads spread over host threads.  Q64/K64/V64 are callables
    (b, h) -> float64 [L, D] (so huge inputs are widened one head at a time)."""
    def one(bh):
        b, h = bh
        rows = rows_by_bh[bh]
        q = Q64(b, h)[rows]
        return bh, cpa_oracle.attention_rows(q, rows, K64(b, h), V64(b, h), causal, scale,
                                             block=block)
    with ThreadPoolExecutor(host_threads()) as ex:
        return dict(ex.map(one, list(rows_by_bh)))
