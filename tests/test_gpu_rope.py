"""GPU parity of the rotary embedding at global positions (cpa_rope,
cpa_zigzag_permute_rope) and of the whole path with it, against the fp64
oracle, through the C ABI."""
import sys

import numpy as np
import pytest
import torch

from oracle import cpa_oracle
from parity_helpers import assert_bf16_close, oracle_rows, widen

import sequence_attention_cpa_amd as cpa
from sequence_attention_cpa_amd.pipeline import SharePipeline
from sequence_attention_cpa_amd.workloads import WORKLOADS, make_inputs, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAIRINGS = [cpa.CPA_ROPE_INTERLEAVED, cpa.CPA_ROPE_HALF]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    cpa.load()
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def pair_amplitude(x, pairing):
    """|(x_a, x_b)| of the pair each element belongs to (kept by the rotation)."""
    D = x.shape[-1]
    a, b = cpa_oracle.rope_pairs(D, pairing)
    amp = np.empty_like(x)
    r = np.sqrt(x[..., a] ** 2 + x[..., b] ** 2)
    amp[..., a] = r
    amp[..., b] = r
    return amp


def assert_rope_close(got, ref, x64, pairing, bf16, what):
    """fp32 output: within 2e-6 of the pair amplitude (sin/cos and fma
    rounding).  bf16 output: within half a bf16 ulp of the fp64 value plus the
    same fp32 margin, i.e. the round-to-nearest-even of the exact rotation
    except where the fp32 result sits on a rounding boundary."""
    amp = pair_amplitude(x64, pairing)
    d = np.abs(got - ref)
    bound = 2e-6 * amp
    if bf16:
        mag = np.maximum(np.abs(ref), np.abs(got))
        ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
        bound = bound + 0.5 * ulp
        exact = torch.from_numpy(ref).to(torch.bfloat16).double().numpy() == got
        say(f"{what}: {100 * exact.mean():.4f}% equal to RNE(fp64)")
    worst = float((d / np.maximum(bound, 1e-300)).max()) if d.size else 0.0
    assert np.all(d <= bound), f"{what}: off by {worst:.2f}x tolerance"


@pytest.mark.parametrize("pairing", PAIRINGS)
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 16), (torch.float32, 128),
                                     (torch.bfloat16, 8)])
def test_rope_vs_oracle(dtype, D, pairing):
    """Random rows at random global positions up to 2^22 (large angles), a
    ragged row count, and in-place use."""
    B, H, rows = 2, 3, 1000
    g = torch.Generator().manual_seed(70)
    x = torch.randn((B, H, rows, D), generator=g).to(dtype)
    pos = np.random.default_rng(71).integers(0, 1 << 22, size=rows).astype(np.int64)
    pos[:4] = [0, 1, 131071, 1048575]
    for base in (10000.0, 500000.0):
        ref = cpa_oracle.rope(widen(x), pos, base, pairing)
        xd = x.to(DEV)
        posd = torch.from_numpy(pos).to(DEV)
        y = cpa.rope(xd, posd, base, pairing)
        cpa.rope(xd, posd, base, pairing, out=xd)  # in place
        torch.cuda.synchronize()
        for out, how in ((y, "out of place"), (xd, "in place")):
            assert_rope_close(out.cpu().double().numpy(), ref, widen(x), pairing,
                              dtype == torch.bfloat16, f"D={D} {dtype} {how} base={base}")


@pytest.mark.parametrize("pairing", PAIRINGS)
@pytest.mark.parametrize("dtype,B,H,L,N,D,ranks", [
    (torch.bfloat16, 2, 2, 4096, 4, 128, (0, 4)),
    (torch.bfloat16, 1, 3, 4096, 4, 64, (1, 3)),
    (torch.float32, 1, 2, 64, 4, 16, (0, 4)),
    (torch.bfloat16, 1, 2, 256, 16, 128, (15, 16)),
])
def test_permute_rope_vs_oracle(dtype, B, H, L, N, D, ranks, pairing):
    g = torch.Generator().manual_seed(72)
    x = torch.randn((B, H, L, D), generator=g).to(dtype)
    lo, hi = ranks
    pos = cpa.zigzag_layout(L, N)
    out = cpa.zigzag_permute_rope(x.to(DEV), pos.to(DEV), N, 10000.0, pairing, lo, hi)
    torch.cuda.synchronize()
    pos_np = pos.numpy()
    ref = cpa_oracle.permute_to_ranks_rope(widen(x), pos_np[lo:hi], 10000.0, pairing)
    x_ranks = cpa_oracle.permute_to_ranks(widen(x), pos_np[lo:hi])
    assert_rope_close(out.cpu().double().numpy(), ref, x_ranks, pairing,
                      dtype == torch.bfloat16, f"permute+rope {ranks}")


@pytest.mark.parametrize("pairing", PAIRINGS)
def test_permute_rope_1m_positions_sampled(pairing):
    """The 1M layout (positions up to 2^20 - 1): every rank, sampled rows."""
    L, N, D = 1 << 20, 8, 128
    g = torch.Generator().manual_seed(73)
    x = torch.randn((1, 1, L, D), generator=g).to(torch.bfloat16)
    pos = cpa.zigzag_layout(L, N)
    out = cpa.zigzag_permute_rope(x.to(DEV), pos.to(DEV), N, 10000.0, pairing)
    torch.cuda.synchronize()
    pos_np = pos.numpy()
    Lr = L // N
    rng = np.random.default_rng(74)
    t = np.unique(np.concatenate([[0, Lr // 2 - 1, Lr // 2, Lr - 1], rng.integers(0, Lr, 250)]))
    for r in range(N):
        p = pos_np[r, t]
        x64 = widen(x[0, 0])[p]
        ref = cpa_oracle.rope(x64, p, 10000.0, pairing)
        got = out[r, 0, 0, torch.from_numpy(t).to(DEV)].cpu().double().numpy()
        assert_rope_close(got, ref, x64, pairing, True, f"1M rank {r}")


def rope_oracle_inputs(Q, K, base, pairing):
    """Exact fp64 rotation at global positions, then rounded to the input dtype
    (the attention's inputs are that dtype), then widened."""
    L = Q.shape[2]
    pos = np.arange(L)
    Qr = torch.from_numpy(cpa_oracle.rope(widen(Q), pos, base, pairing)).to(Q.dtype)
    Kr = torch.from_numpy(cpa_oracle.rope(widen(K), pos, base, pairing)).to(K.dtype)
    return Qr, Kr


@pytest.mark.parametrize("pairing", PAIRINGS)
def test_rope_pipeline_12k_every_row(pairing):
    w = WORKLOADS["12k"]
    say("12k rope: generating")
    Q, K, V, _ = make_inputs(w)
    outs = {}
    for fused in (False, True, "global"):
        pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, DEV, fused=bool(fused),
                             rope_base=10000.0, rope_pairing=pairing,
                             global_layout=fused == "global")
        O, lse = pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
        torch.cuda.synchronize()
        outs[fused] = (O.cpu().double().numpy(), lse.cpu().double().numpy())
        del pipe, O, lse
    say("12k rope: oracle")
    Qr, Kr = rope_oracle_inputs(Q, K, 10000.0, pairing)
    rows = {(b, h): np.arange(w.L) for b in range(w.B) for h in range(w.H)}
    ref = oracle_rows(lambda b, h: widen(Qr[b, h]), lambda b, h: widen(Kr[b, h]),
                      lambda b, h: widen(V[b, h]), rows, w.causal)
    Or = np.stack([np.stack([ref[(b, h)][0] for h in range(w.H)]) for b in range(w.B)])
    lr = np.stack([np.stack([ref[(b, h)][1] for h in range(w.H)]) for b in range(w.B)])
    for fused, (O, lse) in outs.items():
        mx, mean = assert_bf16_close(O, lse, Or, lr, f"12k rope fused={fused}")
        say(f"12k rope pairing={pairing} fused={fused}: max {mx:.3e} mean {mean:.3e}")


@pytest.mark.parametrize("mode", ["fused", "global"])
def test_rope_pipeline_128k_share_sampled(mode):
    """128k share (rank 3: positions 49152-65535 and 65536-81919) with RoPE,
    one ring launch on rank-major or global-order data, sampled rows against
    the oracle."""
    w = WORKLOADS["128k"]
    rank = 3
    say(f"128k rope {mode}: generating")
    Q, K, V, outl = make_inputs(w)
    pipe = SharePipeline(w.B, w.H, w.L, w.D, w.N, w.causal, Q.dtype, DEV, rank, rank + 1,
                         fused=True, rope_base=10000.0, global_layout=mode == "global")
    O, lse = pipe.step(Q.to(DEV), K.to(DEV), V.to(DEV))
    pos = pipe.pos_host.numpy()
    t = sample_rows(w, rank, pos[rank], 1024 // (w.B * w.H), outl)
    g = pos[rank][t]
    gi = torch.from_numpy(g).to(DEV)
    O, lse = O[:, :, gi].cpu().double().numpy(), lse[:, :, gi].cpu().double().numpy()
    del pipe
    say("128k rope: oracle")
    Qr, Kr = rope_oracle_inputs(Q, K, 10000.0, cpa.CPA_ROPE_INTERLEAVED)
    rows = {(b, h): g for b in range(w.B) for h in range(w.H)}
    ref = oracle_rows(lambda b, h: widen(Qr[b, h]), lambda b, h: widen(Kr[b, h]),
                      lambda b, h: widen(V[b, h]), rows, w.causal, block=32)
    Or = np.stack([np.stack([ref[(b, h)][0] for h in range(w.H)]) for b in range(w.B)])
    lr = np.stack([np.stack([ref[(b, h)][1] for h in range(w.H)]) for b in range(w.B)])
    mx, mean = assert_bf16_close(O, lse, Or, lr, "128k rope")
    say(f"128k rope: max {mx:.3e} mean {mean:.3e}")
