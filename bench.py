"""Benchmark: one rank's share of context-parallel ring attention on one MI355X.

A step is one pass of the whole hot path for the rank: the zigzag layout's
permute of Q/K/V into rank order, the rank's ring over all N K/V blocks with
online-softmax folding, and O and lse back in global token order.  Modes:
  --ring global   (default) one launch (cpa_share_forward): the kernel reads
                  global-order Q/K/V and writes global-order O/lse, the zigzag
                  permute folded into its addressing, the N blocks walked with
                  the online-softmax state in registers;
  --ring fused    explicit permutes to rank-major order, one fused ring launch
                  (cpa_rank_forward_fused), inverse permutes;
  --ring partials explicit permutes, N partial launches and N-1 merges
                  (cpa_rank_forward), inverse permutes.
Inputs are resident in HBM before timing starts.

Metric: causal-useful attention TFLOP/s = 4 * D * B * H * P / t, where P is the
number of (query, key) pairs the rank's queries may see (key position <= query
position), i.e. masked and skipped work is not counted.

Prints ONE JSON line.  `roofline` is for the dominant kernel (the attention
kernel, bf16 MFMA-bound): its useful FLOP per launch over the median duration
of the timed steps' launches, timed with HIP events on the launch stream (in
the default mode a step is that one launch).  `kernels` adds the other launch
forms, the backward, the 12k workload's four ranks, and the bandwidth-bound
kernels (merge, permute, permute+RoPE) against a plain device copy, timed at
the 1M share's sizes so that their working sets exceed the 256 MB MALL.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
share's query rows, on every host core the process may use.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak (no sparsity)
PEAK_HBM_GBS = 8000.0
PMC_FILES = {"global": os.path.join(ROOT, "profiles", "ring_global_128k_pmc.json"),
             "fused": os.path.join(ROOT, "profiles", "ring_fused_128k_pmc.json"),
             "partials": os.path.join(ROOT, "profiles", "partial_attn_128k_pmc.json")}
KERNEL_SRC = os.path.join(ROOT, "sequence_attention_cpa_amd", "csrc", "attn_fwd.hip")


def causal_pairs(q_pos, k_pos):
    import numpy as np
    return int(np.searchsorted(np.sort(k_pos), q_pos, side="right").sum())


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def pmc_traffic(ring, workload):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs, or None when they were taken on a different version of it
    or on another workload (the runs profile the 128k share)."""
    if workload != "128k":
        return None
    try:
        with open(PMC_FILES[ring]) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_sha") != kernel_sha():
        return None
    return d.get("traffic_bytes_per_launch")


def blas_info():
    """numpy's BLAS as threadpoolctl reports it: vendor, library, threads."""
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                return {"vendor": d.get("internal_api"), "library": os.path.basename(
                    d.get("filepath", "")), "threads_default": d.get("num_threads")}
    except Exception:  # pragma: no cover
        pass
    return None


def cpu_baseline(w, Q, K, V, pos_rank, seconds, useful_flop):
    """The oracle, untouched, over a sample of the rank's query rows; rows are
    independent, so host threads each take whole (head, row-block) tasks, one
    BLAS thread each, on every core the process may use."""
    import numpy as np
    import torch
    from concurrent.futures import ThreadPoolExecutor

    from oracle import cpa_oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    cores = max(1, len(os.sched_getaffinity(0)))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    K64 = {bh: K[bh].to(torch.float64).numpy() for bh in heads}
    V64 = {bh: V[bh].to(torch.float64).numpy() for bh in heads}
    rng = np.random.default_rng(0)
    block = 16
    # sample row blocks from the whole share, timing until the budget is spent
    tasks = []
    for _ in range(8192):
        bh = heads[int(rng.integers(len(heads)))]
        t0 = int(rng.integers(0, len(pos_rank) - block + 1))
        tasks.append((bh, pos_rank[t0:t0 + block]))

    def run(task):
        bh, rows = task
        q = Q[bh][torch.from_numpy(rows)].to(torch.float64).numpy()
        cpa_oracle.attention_rows(q, rows, K64[bh], V64[bh], w.causal, block=block)
        return sum(int(p) + 1 for p in rows) if w.causal else len(rows) * w.L

    import contextlib
    ctx = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    pairs = 0
    done_rows = 0
    t_start = time.perf_counter()
    with ctx, ThreadPoolExecutor(cores) as ex:
        i = 0
        while i < len(tasks) and time.perf_counter() - t_start < seconds:
            batch = tasks[i:i + cores]
            pairs += sum(ex.map(run, batch))
            done_rows += block * len(batch)
            i += len(batch)
    el = time.perf_counter() - t_start
    flops = 4.0 * w.D * pairs
    value = flops / el / 1e12
    share_rows = w.B * w.H * len(pos_rank)
    return {"value": value, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done_rows} of the share's {share_rows} query rows ({block}-row blocks, "
                      f"random heads and positions, seed 0), fp64 numpy, {el:.1f} s, "
                      f"{cores} worker threads with 1 BLAS thread each",
            "seconds": round(el, 2), "rows": done_rows,
            "seconds_per_row": round(el / max(done_rows, 1), 6), "blas": blas_info(),
            "extrapolated_full_share_seconds": round(useful_flop / (value * 1e12), 1),
            "extrapolation": "the share's useful FLOP at the sampled rate (extrapolated, "
                             "not measured)"}


def zig_pairs(L, N, ranks):
    """Visible (query, key) pairs of the given ranks' rings under the zigzag
    layout (closed form 2N C^2 + C per head and rank, C = L / 2N)."""
    C = L // (2 * N)
    return len(ranks) * (2 * N * C * C + C)


def small_share(cpa, torch, dev, timed, reps):
    """The 12k workload's shape (B 1, H 32, D 128, L 12288, CP 4), all four
    ranks' rings in one cpa_share_forward call, on device-generated bf16
    N(0,1) inputs."""
    import numpy as np
    B, H, L, D, N = 1, 32, 12288, 128, 4
    g = torch.Generator(device=dev).manual_seed(12)
    Q, K, V = (torch.randn((B, H, L, D), generator=g, device=dev, dtype=torch.float32)
               .to(torch.bfloat16) for _ in range(3))
    O = torch.empty((B, H, L, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, L), dtype=torch.float32, device=dev)
    fn = lambda: cpa.share_forward(Q, K, V, N, True, out=O, lse=lse)  # noqa: E731
    # The clock a launch runs at follows the power drawn over the preceding
    # milliseconds (the backward before this leg runs hotter), so the shape
    # runs back to back for ~50 ms before it is timed, as a training loop at
    # this size would.
    for _ in range(40):
        fn()
    evs = timed(fn, reps)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    flop = 4.0 * D * B * H * zig_pairs(L, N, range(N))
    med = float(np.median(ms))
    return {"workload": "12k: B=1 H=32 D=128 L=12288 CP=4, all 4 ranks, one cpa_share_forward",
            "ms_median": round(med, 4), "ms_min": round(float(ms.min()), 4),
            "TFLOP/s": round(flop / (med * 1e-3) / 1e12, 2), "useful_flop": flop}


def bandwidth(cpa, torch, dev, timed, reps):
    """HBM-bound kernels at the 1M share's sizes (B 1, H 4, D 128, L 2^20,
    CP 8: every working set 0.8-2 GiB, well past the 256 MB MALL), against a
    plain device-to-device copy of the permute's size."""
    import numpy as np
    B, H, L, D, N = 1, 4, 1 << 20, 128, 8
    Lr = L // N
    rows = B * H * Lr
    out = {"sizes": "1M share: B=1 H=4 D=128 L=1048576 CP=8", "mall_free": True,
           "peak_GB/s": PEAK_HBM_GBS}

    def rate(name, fn, nbytes):
        fn()
        evs = timed(fn, reps)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms_median": round(ms, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                     "frac_of_peak": round(gbs / PEAK_HBM_GBS, 3)}

    f32 = dict(dtype=torch.float32, device=dev)
    Oa, On = torch.randn((rows, D), **f32), torch.randn((rows, D), **f32)
    la, ln = torch.randn((rows,), **f32), torch.randn((rows,), **f32)
    # read both partials, write the accumulator (O and lse)
    rate("merge", lambda: cpa.merge(Oa, la, On, ln), rows * (D + 1) * 4 * 3)
    del Oa, On, la, ln
    K = torch.empty((B, H, L, D), dtype=torch.bfloat16, device=dev).normal_()
    Kr = torch.empty((N, B, H, Lr, D), dtype=torch.bfloat16, device=dev)
    pos = cpa.zigzag_layout(L, N).to(dev)
    nb = 2 * K.numel() * K.element_size()  # read K once, write it once
    rate("permute_K", lambda: cpa.zigzag_permute(K, pos, N, out=Kr), nb)
    rate("permute_rope_K", lambda: cpa.zigzag_permute_rope(K, pos, N, 10000.0, out=Kr), nb)
    Kc = torch.empty_like(K)
    rate("device_copy_same_bytes", lambda: Kc.copy_(K), nb)
    c = out["device_copy_same_bytes"]["GB/s"]
    for name in ("merge", "permute_K", "permute_rope_K"):
        out[name]["frac_of_copy"] = round(out[name]["GB/s"] / c, 3)
    del K, Kr, Kc
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="128k")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--ring", choices=("global", "fused", "partials"), default="global",
                    help="global-layout ring launch (default), permutes + fused ring launch, or "
                         "permutes + N partials + N-1 merges")
    ap.add_argument("--backward", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the rank's ring backward (reported under kernels)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extra", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the 12k workload's ranks and the bandwidth-bound kernels at "
                         "1M sizes (reported under kernels)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (virtual ranks on one device); --gpus {args.gpus} "
              "is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sequence_attention_cpa_amd as cpa
    from sequence_attention_cpa_amd.pipeline import SharePipeline
    from sequence_attention_cpa_amd.workloads import WORKLOADS, make_inputs, make_upstream_grad

    cpa.load()
    dev = "cuda:0"
    w = WORKLOADS[args.workload]
    rank = args.rank
    Qh, Kh, Vh, outl = make_inputs(w)
    Q, K, V = Qh.to(dev), Kh.to(dev), Vh.to(dev)
    mfma_ok = w.dtype == "bf16" and w.D in (64, 128)
    global_ok = mfma_ok and (w.C % 32 == 0)
    if args.ring == "global" and not global_ok:
        args.ring = "fused" if mfma_ok else "partials"
    fused = args.ring in ("fused", "global")
    pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, dev, rank, rank + 1,
                         fused=fused, global_layout=args.ring == "global")
    pos = pipe.pos_host.numpy()
    if w.causal:
        pairs = [causal_pairs(pos[rank], pos[j]) for j in range(w.N)]
    else:
        pairs = [w.Lr * w.Lr] * w.N
    useful = 4.0 * w.D * w.B * w.H * sum(pairs)

    stream = torch.cuda.current_stream()
    if args.copy_mib:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the scale between those counters and bytes actually moved.
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        pipe.step(Q, K, V)
    torch.cuda.synchronize()
    evs_step = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs_step[0].record(stream)
    for k in range(args.steps):
        pipe.step(Q, K, V)
        evs_step[k + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    step_ms = np.array([evs_step[k].elapsed_time(evs_step[k + 1]) for k in range(args.steps)])
    ms_step_ev = float(step_ms.mean())

    # Per-kernel timing on the same stream: the global-layout launch, the fused
    # ring launch on rank-major data, the unfused ring's partials (same kernel
    # and arguments as inside cpa_rank_forward), a merge, and the K permute.
    # The rank-major forms need rank-major buffers, which a global-layout
    # pipeline does not hold: a rank-major pipeline provides them.
    rk = pipe if not pipe.global_layout else SharePipeline(
        w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, dev, rank, rank + 1, fused=True)
    zigzag = cpa.zigzag_permute
    zigzag(K, pipe.pos, w.N, out=rk.Kr)
    zigzag(V, pipe.pos, w.N, out=rk.Vr)
    zigzag(Q, pipe.pos, w.N, rank_lo=rank, rank_hi=rank + 1, out=rk.Qr)
    Lr = w.Lr
    tO = torch.empty((w.B, w.H, Lr, w.D), dtype=torch.float32, device=dev)
    tl = torch.empty((w.B, w.H, Lr), dtype=torch.float32, device=dev)
    pos_d = pipe.pos
    reps = max(1, args.steps // 2)

    def timed(fn, n):
        evs = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            evs.append((a, b))
        return evs

    share_evs = []
    if global_ok:
        share_evs = timed(lambda: cpa.share_forward(Q, K, V, w.N, w.causal,
                                                    rank_lo=rank, rank_hi=rank + 1, out=pipe.O,
                                                    lse=pipe.lse), reps)
    # Precise weights (cpa_share_forward_precise) on the same share with the
    # outlier rows scaled in V as well (the 128k_qkv inputs: V's outlier rows
    # times 8, exact in bf16), next to the bf16-weight launch on those inputs.
    qkv = None
    if global_ok and args.extra and len(outl) and w.outlier_mult != 1.0 and not w.outlier_in_v:
        Vx = V.clone()
        Vx[:, :, torch.from_numpy(outl).to(dev)] *= w.outlier_mult
        qkv = {}
        for name, prec in (("bf16_weights", False), ("precise_weights", True)):
            f = lambda: cpa.share_forward(Q, K, Vx, w.N, w.causal, rank_lo=rank,  # noqa: E731
                                          rank_hi=rank + 1, out=pipe.O, lse=pipe.lse,
                                          precise=prec)
            f()
            qkv[name] = timed(f, reps)
        del Vx
    fused_evs, last_evs = [], []
    if mfma_ok:
        fused_evs = timed(lambda: cpa.rank_forward_fused(rank, w.N, rk.Qr[0], rk.Kr, rk.Vr,
                                                         pos_d, w.causal, out=tO, lse=tl), reps)
        # Balance: the last rank's ring does the same causal work under zigzag.
        other = w.N - 1 if rank != w.N - 1 else 0
        Q_other = cpa.zigzag_permute(Q, pos_d, w.N, rank_lo=other, rank_hi=other + 1)[0]
        last_evs = timed(lambda: cpa.rank_forward_fused(other, w.N, Q_other, rk.Kr, rk.Vr,
                                                        pos_d, w.causal, out=tO, lse=tl), reps)
    # Balance without the zigzag: the same one-launch ring on a contiguous split
    # (rank r holds tokens [r L/N, (r+1) L/N)), first and last rank.  Under the
    # causal mask the last rank meets (2N-1) times the first rank's pairs, and a
    # CP step waits for the slowest rank.
    contig = {}
    if mfma_ok and w.causal and w.N > 1:
        pos_c = torch.arange(w.L, dtype=torch.int64, device=dev).reshape(w.N, Lr)
        pos_ch = pos_c.cpu().numpy()
        Kc = zigzag(K, pos_c, w.N)
        Vc = zigzag(V, pos_c, w.N)
        for r in (0, w.N - 1):
            Qc = zigzag(Q, pos_c, w.N, rank_lo=r, rank_hi=r + 1)[0]
            evs = timed(lambda: cpa.rank_forward_fused(r, w.N, Qc, Kc, Vc, pos_c, True, out=tO,
                                                       lse=tl), reps)
            contig[r] = (evs, sum(causal_pairs(pos_ch[r], pos_ch[j]) for j in range(w.N)))
        del Kc, Vc
    part_evs = []
    for _ in range(reps):
        for s in range(w.N):
            j = (rank + s) % w.N
            part_evs += [(j, e) for e in timed(lambda: cpa.partial(
                rk.Qr[0], rk.Kr[j], rk.Vr[j], pos_d[rank], pos_d[j], w.causal, out=tO,
                lse=tl), 1)]
    # Ring backward of the same rank (delta + dQ pass + dK/dV pass), after a
    # forward step so that O and lse are the ring's: on global-order data
    # (cpa_share_backward, the pipeline's backward in the default mode) and on
    # rank-major copies of the same tensors (cpa_rank_backward).
    bwd_evs, gbwd_evs = [], []
    if args.backward:
        pipe.step(Q, K, V)
        dO = make_upstream_grad(w).to(dev)
        pipe.backward(dO)
        if pipe.global_layout:
            gbwd_evs = timed(lambda: cpa.share_backward(
                Q, K, V, pipe.O, dO, pipe.lse, w.N, w.causal, pipe.dK, pipe.dV,
                pipe.scale, rank, rank + 1, dQ=pipe.dQ, delta=pipe.delta), reps)
        zigzag(pipe.O, pos_d, w.N, rank_lo=rank, rank_hi=rank + 1, out=rk.Or)
        zigzag(pipe.lse, pos_d, w.N, rank_lo=rank, rank_hi=rank + 1, out=rk.lser)
        dOr = zigzag(dO, pos_d, w.N, rank_lo=rank, rank_hi=rank + 1)
        f32 = dict(dtype=torch.float32, device=dev)
        dQr = torch.empty((w.B, w.H, Lr, w.D), **f32)
        deltar = torch.empty((w.B, w.H, Lr), **f32)
        dKr = torch.zeros(rk.Kr.shape, **f32)
        dVr = torch.zeros(rk.Vr.shape, **f32)
        bwd_evs = timed(lambda: cpa.rank_backward(rank, w.N, rk.Qr[0], rk.Kr, rk.Vr, pos_d,
                                                  rk.Or[0], dOr[0], rk.lser[0], w.causal,
                                                  dKr, dVr, pipe.scale, dQ=dQr, delta=deltar),
                        reps)
    torch.cuda.synchronize()
    p_ms = np.array([a.elapsed_time(b) for _, (a, b) in part_evs])
    p_flops = np.array([4.0 * w.D * w.B * w.H * pairs[j] for j, _ in part_evs])
    p_avg_ms = float(p_ms.mean())
    f_ms = np.array([a.elapsed_time(b) for a, b in fused_evs]) if fused_evs else None
    o_ms = np.array([a.elapsed_time(b) for a, b in last_evs]) if last_evs else None
    g_ms = np.array([a.elapsed_time(b) for a, b in share_evs]) if share_evs else None

    def stats(x):
        return {"median": round(float(np.median(x)), 4), "min": round(float(np.min(x)), 4),
                "p90": round(float(np.percentile(x, 90)), 4)}
    if args.ring == "global":
        # a step is this one launch: the timed steps' own launch durations
        dom_kernel = (f"attn_fwd_kernel<{w.D}, global layout> (one launch, {w.N} K/V "
                      "blocks)")
        dom_ms = float(np.median(step_ms))
        dom_src = f"median of the {args.steps} timed steps (one launch each)"
        dom_flop = useful
    elif fused:
        dom_kernel = f"attn_fwd_kernel<{w.D}> (one launch, {w.N} K/V blocks)"
        dom_ms = float(np.median(f_ms))
        dom_src = f"median of {len(f_ms)} launches after the timed steps"
        dom_flop = useful
    else:
        dom_kernel = f"attn_fwd_kernel<{w.D}> (one K/V block)"
        dom_ms = float(np.median(p_ms))
        dom_src = f"median of {len(p_ms)} partial launches after the timed steps"
        dom_flop = float(p_flops.mean())
    achieved = dom_flop / (dom_ms * 1e-3) / 1e12
    qkv_report = None
    if qkv:
        qkv_report = {"inputs": f"{w.name} share with the outlier rows scaled in V too "
                                f"(x{w.outlier_mult:g}), rank {rank}"}
        for name, evs in qkv.items():
            ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
            qkv_report[name] = {"ms_median": round(ms, 4),
                                "TFLOP/s": round(useful / (ms * 1e-3) / 1e12, 2)}

    def bwd_report(evs):
        if not evs:
            return None
        b_ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        b_flop = 2.0 * useful  # dV, dP, dQ, dK: 4 products of 2*D per visible pair
        return {"ms": round(b_ms, 4), "TFLOP/s": round(b_flop / (b_ms * 1e-3) / 1e12, 2),
                "useful_flop": b_flop}
    bwd = bwd_report(bwd_evs)
    gbwd = bwd_report(gbwd_evs)
    balance = None
    if contig and o_ms is not None and rank == 0:
        c0, cl = (float(np.median([a.elapsed_time(b) for a, b in contig[r][0]]))
                  for r in (0, w.N - 1))
        z0, zl = float(np.median(f_ms)), float(np.median(o_ms))
        # Per-rank work is linear in the rank under either split, so the mean
        # over ranks is the mean of the first and the last.
        balance = {"contiguous_ms": [round(c0, 4), round(cl, 4)],
                   "contiguous_pairs": [contig[0][1], contig[w.N - 1][1]],
                   "contiguous_step_efficiency": round((c0 + cl) / 2 / max(c0, cl), 3),
                   "zigzag_ms": [round(z0, 4), round(zl, 4)],
                   "zigzag_pairs": [sum(pairs), sum(
                       causal_pairs(pos[w.N - 1], pos[j]) for j in range(w.N))],
                   "zigzag_step_efficiency": round((z0 + zl) / 2 / max(z0, zl), 3)}

    # After the share's own kernels: the 12k shape, then the HBM-bound kernels
    # at 1M sizes (their buffers are freed before the CPU baseline).
    del rk, tO, tl
    small = small_share(cpa, torch, dev, timed, reps) if args.extra else None
    bw = bandwidth(cpa, torch, dev, timed, reps) if args.extra else None

    value = useful / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "causal-useful attention TFLOP/s per GPU at 128k CP=4 share; % bf16 MFMA peak"
        if args.workload == "128k" else f"causal-useful attention TFLOP/s ({args.workload} share)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name} share: rank {rank} of CP={w.N} zigzag, B={w.B} H={w.H} "
                               f"D={w.D} L={w.L}, causal={w.causal}",
                   "B": w.B, "H": w.H, "D": w.D, "L": w.L, "N": w.N, "rank": rank,
                   "causal": w.causal, "useful_flop_per_step": useful,
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": pmc_traffic(args.ring, args.workload), "kernel": dom_kernel,
                     "launch_ms": round(dom_ms, 4), "launch_ms_from": dom_src,
                     "useful_flop_per_launch": dom_flop},
        "kernels": {
            "ring": args.ring,
            "global_ring_ms_stats": stats(g_ms) if g_ms is not None else None,
            "fused_ring_ms": round(float(f_ms.mean()), 4) if f_ms is not None else None,
            "fused_ring_ms_stats": stats(f_ms) if f_ms is not None else None,
            "fused_ring_ms_other_rank": ({"rank": other, **stats(o_ms)}
                                         if o_ms is not None else None),
            "partial_ms": [round(float(x), 4) for x in p_ms[: w.N]],
            "partial_TFLOP/s": round(float(p_flops.mean()) / (p_avg_ms * 1e-3) / 1e12, 2),
            "outliers_in_v": qkv_report,
            "small_share_12k": small,
            "bandwidth": bw,
            "ms_per_step_events": round(ms_step_ev, 4),
            "step_ms_stats": stats(step_ms),
            "balance_first_last_rank": balance,
            "rank_backward": bwd,
            "share_backward": gbwd,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu and rank == 0:
        out["cpu_baseline"] = cpu_baseline(w, Qh, Kh, Vh, pos[rank], args.cpu_seconds, useful)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
