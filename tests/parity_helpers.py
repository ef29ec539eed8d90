"""Shared helpers of the GPU parity tests: tolerances and a threaded driver
for the oracle (the oracle itself stays single-threaded and plain; rows and
heads are independent, so the tests spread them over host threads)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from oracle import cpa_oracle

# bf16 inputs vs the fp64 oracle: max |d| <= 1e-2 and mean |d| <= 1e-3 over
# all checked elements, for O and for lse alike (both are outputs of a
# partial); empty rows exactly (0, -inf).  With bf16 weights lse is the log
# of the sum of the rounded weights (the normaliser O uses), which a single
# dominant key moves by up to ln(1 + 2^-9) ~ 2e-3.
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
# fp32 inputs: the pages' own check, assert_allclose(rtol=1e-5, atol=1e-6).
F32_RTOL, F32_ATOL = 1e-5, 1e-6


# Backward, bf16 inputs: P and dS are rounded to bf16 (relative 2^-8) before
# the matrix products, whose sums are fp32, so every gradient entry carries an
# error of a small multiple of 2^-8 times the size of its terms.  Checked
# against the largest entry of the reference gradient (entries near zero
# carry the same absolute error as large ones), norm-wise, and on the mean:
# max |d| <= 7e-3 max|ref|, ||d||_2 <= 5e-3 ||ref||_2, mean |d| <= 5e-3
# mean |ref|.  The kernels measure at most 3.6e-3 and 2.3e-3 on the first
# two over every backward test (large logits included): the gates sit at
# about twice that.  fp32 inputs: |d| <= 1e-5 |ref| + 1e-5 max|ref|
# (dS = P (dP - delta) cancels, so a purely relative bound is too tight).
GRAD_BF16_MAX_REL = 7e-3
GRAD_BF16_NORM_REL = 5e-3
GRAD_BF16_MEAN_REL = 5e-3
GRAD_F32_RTOL = 1e-5
GRAD_F32_ATOL_REL = 1e-5


def assert_grad_close(got, ref, bf16, what=""):
    d = np.abs(got - ref)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    if bf16:
        mx = float(d.max()) / max(scale, 1e-30) if d.size else 0.0
        nrm = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
        mean = float(d.mean() / max(float(np.abs(ref).mean()), 1e-30)) if d.size else 0.0
        print(f"grad {what}: max-rel {mx:.3e} norm-rel {nrm:.3e} mean-rel {mean:.3e}",
              flush=True)
        assert mx <= GRAD_BF16_MAX_REL, f"{what}: max |d| = {mx:.3e} of max|ref| > {GRAD_BF16_MAX_REL}"
        assert nrm <= GRAD_BF16_NORM_REL, f"{what}: norm-wise {nrm:.3e} > {GRAD_BF16_NORM_REL}"
        assert mean <= GRAD_BF16_MEAN_REL, f"{what}: mean-wise {mean:.3e} > {GRAD_BF16_MEAN_REL}"
        return mx, nrm
    bound = GRAD_F32_RTOL * np.abs(ref) + GRAD_F32_ATOL_REL * scale
    worst = float((d / np.maximum(bound, 1e-300)).max()) if d.size else 0.0
    assert np.all(d <= bound), f"{what}: fp32 gradient off by {worst:.2f}x tolerance"
    return worst, 0.0


def host_threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def host_map(fn, items):
    """list(map(fn, items)) over host threads, one BLAS thread per worker: the
    workers already use every core, and a multi-threaded BLAS inside each of
    them oversubscribes the host (measured 45x slower on the 12k oracle)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1), ThreadPoolExecutor(host_threads()) as ex:
        return list(ex.map(fn, items))


def widen(t):
    """Exact widening of a bf16/fp32 tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_empty_rows(O, lse, O_ref, lse_ref):
    neg = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), neg), "rows without visible keys differ"
    assert np.all(O[neg] == 0.0), "rows without visible keys must have O = 0"
    assert not np.any(np.isnan(O)) and not np.any(np.isnan(lse))
    return ~neg


def assert_bf16_close(O, lse, O_ref, lse_ref, what="", v_scale=1.0):
    """v_scale: how much larger than unit scale V's largest rows are.  O is a
    convex combination of V rows, so the error that bf16 weights leave in it
    scales with them; the O bounds are the unit-scale ones times v_scale."""
    fin = check_empty_rows(O, lse, O_ref, lse_ref)
    d = np.abs(O - O_ref)
    mx, mean = float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0
    mx_tol, mean_tol = BF16_MAX_ABS * v_scale, BF16_MEAN_ABS * v_scale
    assert mx <= mx_tol, f"{what}: max |dO| {mx:.3e} > {mx_tol}"
    assert mean <= mean_tol, f"{what}: mean |dO| {mean:.3e} > {mean_tol}"
    dl = np.abs(lse[fin] - lse_ref[fin])
    if dl.size:
        assert dl.max() <= BF16_MAX_ABS, f"{what}: max |dlse| {dl.max():.3e} > {BF16_MAX_ABS}"
        assert dl.mean() <= BF16_MEAN_ABS, f"{what}: mean |dlse| {dl.mean():.3e} > {BF16_MEAN_ABS}"
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
    return dict(host_map(one, list(rows_by_bh)))
