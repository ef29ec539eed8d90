"""CPU model of the LDS tile schedules of the matrix-core kernels.

The forward's steady loop keeps K and V tiles in NBUF LDS buffers each, copies
K(t + K_AHEAD) and V(t + V_AHEAD) during iteration t, reads K(t+1), V(t-1)
and (for the next iteration's first products) V(t), and meets at a barrier
after every odd iteration; the dQ pass of the backward keeps K/V tile t in
buffer t % 4, copies tile t + 2 during iteration t and meets after every odd
tile; the dK/dV pass keeps Q/dO tile t in buffer t % 2, copies tile t + 1
during iteration t and meets after every tile.  Waves run freely between barriers, so a schedule is safe when, in every
interval between two barriers:
  * each buffer read holds the tile the read expects, copied and waited for
    in an earlier interval (published by a barrier), and
  * no copy writes a buffer that any wave reads in that interval.
The constants are read from the kernel sources, so a change to them that
breaks either rule fails here, on the CPU, before a GPU ever runs it."""
import pathlib
import re

import pytest

CSRC = pathlib.Path(__file__).resolve().parents[1] / "sequence_attention_cpa_amd" / "csrc"


def constant(src, name):
    m = re.search(rf"^constexpr int {name} = (\d+);", src, re.M)
    assert m, f"{name} not found"
    return int(m.group(1))


FWD = (CSRC / "attn_fwd.hip").read_text()
NBUF, K_AHEAD, V_AHEAD = (constant(FWD, n) for n in ("NBUF", "K_AHEAD", "V_AHEAD"))


class Schedule:
    """Copies (interval issued, operand, buffer, tile, interval waited) and
    reads (interval, operand, buffer, tile expected)."""

    def __init__(self):
        self.copies, self.reads, self.interval = [], [], 0

    def copy(self, op, buf, tile):
        self.copies.append([self.interval, op, buf, tile, None])

    def read(self, op, buf, tile):
        self.reads.append((self.interval, op, buf, tile))

    def barrier(self, keep_last=0):
        """Wait for every copy but the last `keep_last` (counters complete in
        order), then meet."""
        pending = [c for c in self.copies if c[4] is None]
        for c in pending[:len(pending) - keep_last]:
            c[4] = self.interval
        self.interval += 1

    def check(self, what):
        for iv, op, buf, tile in self.reads:
            same = [c for c in self.copies if c[1] == op and c[2] == buf and c[0] == iv]
            assert not same, f"{what}: {op} buffer {buf} written while read (interval {iv})"
            before = [c for c in self.copies if c[1] == op and c[2] == buf and c[0] < iv]
            assert before, f"{what}: {op} buffer {buf} read before any copy"
            c = max(before, key=lambda c: c[0])
            assert c[3] == tile, f"{what}: {op} buffer {buf} holds tile {c[3]}, read wants {tile}"
            assert c[4] is not None and c[4] < iv, f"{what}: {op} tile {tile} read before published"


def forward_steady_loop(n_loop):
    """The forward's steady loop over tiles [0, n_loop) of one sweep."""
    last = n_loop - 1
    s = Schedule()
    for j in range(K_AHEAD):
        s.copy("K", j % NBUF, min(j, last))
    for j in range(V_AHEAD):
        s.copy("V", j % NBUF, min(j, last))
    s.copy("V", NBUF - 1, 0)  # the buffer PV(-1) reads: V(0), multiplied by zero weights
    s.barrier()               # wait for every copy, then meet
    s.read("K", 0, 0)         # QK^T of tile 0
    s.read("V", NBUF - 1, 0)  # the first iteration's carried V reads
    t = 0
    iters = []
    while t + 1 < n_loop:
        iters += [(t, False), (t + 1, True)]
        t += 2
    if t < n_loop:
        iters.append((t, False))  # an unpaired last iteration meets no barrier
    for t, bar in iters:
        s.copy("K", (t + K_AHEAD) % NBUF, min(t + K_AHEAD, last))
        s.copy("V", (t + V_AHEAD) % NBUF, min(t + V_AHEAD, last))
        s.read("V", (t + NBUF - 1) % NBUF, max(t - 1, 0))  # PV(t-1)
        s.read("K", (t + 1) % NBUF, min(t + 1, last))      # QK^T(t+1)
        s.read("V", t % NBUF, t)                           # carried: PV(t) of the next iteration
        if bar:
            s.barrier(keep_last=4)  # this pair's 2 K and 2 V copies may stay in flight
    s.read("V", last % NBUF, last)  # PV(last) after the loop
    return s


@pytest.mark.parametrize("n_loop", list(range(1, 41)))
def test_forward_schedule(n_loop):
    forward_steady_loop(n_loop).check(f"forward n_loop={n_loop}")


@pytest.mark.parametrize("change", [("NBUF", -2), ("V_AHEAD", -1), ("K_AHEAD", -1),
                                    ("V_AHEAD", +2), ("K_AHEAD", +3)])
def test_forward_schedule_catches_unsafe_constants(change):
    """The model is not vacuous: a ring two buffers short, or copies issued
    one tile too late or too far ahead, break it."""
    name, delta = change
    g = globals()
    saved = g[name]
    try:
        g[name] = saved + delta
        with pytest.raises(AssertionError):
            for n in range(1, 41):
                forward_steady_loop(n).check(f"{name}{delta:+d}")
    finally:
        g[name] = saved


def dq_pass(T):
    """The dQ pass over T key tiles of one block (four buffers)."""
    s = Schedule()
    s.copy("KV", 0, 0)
    if T > 1:
        s.copy("KV", 1, 1)
    s.barrier()
    iters = []
    t = 0
    while t + 3 < T:
        iters += [(t, 0), (t + 1, 1), (t + 2, 2), (t + 3, 3)]
        t += 4
    if t + 1 < T:
        iters += [(t, 0), (t + 1, 1)]
        t += 2
    if t < T:
        iters.append((t, 0 if t % 4 == 0 else 2))
    for t, p in iters:
        assert p == t % 4
        if t + 2 < T:
            s.copy("KV", (p + 2) % 4, t + 2)
        s.read("KV", p, t)
        if p % 2:
            s.barrier()
    return s


def test_dq_pass_source_matches_the_model():
    """The dQ pass copies tile t + 2 into buffer (P + 2) & 3 and meets after
    odd buffer phases, as modelled."""
    src = (CSRC / "attn_backward.hip").read_text()
    assert "copy_kv(Kbh, Kbh_hi, t + 2, Kl_s + ((P + 2) & 3) * TB);" in src
    assert "if constexpr (P & 1) {" in src
    assert "char k_lds_raw[4 * TB];" in src


@pytest.mark.parametrize("T", list(range(1, 41)))
def test_dq_schedule(T):
    dq_pass(T).check(f"dQ T={T}")


def dkdv_pass(T):
    """The dK/dV pass over T query tiles (two Q/dO buffers)."""
    s = Schedule()
    s.copy("QO", 0, 0)
    s.barrier()
    for t in range(T):
        s.read("QO", t % 2, t)  # the first operand reads, then the copy
        if t + 1 < T:
            s.copy("QO", (t + 1) % 2, t + 1)
        s.barrier()
    return s


def test_dkdv_pass_source_matches_the_model():
    """The dK/dV pass copies tile t + 1 into the other buffer after the first
    operand reads and meets after every tile, as modelled."""
    src = (CSRC / "attn_backward.hip").read_text()
    assert "copy_q(Qbh, Qbh_hi, t + 1, Ql_s + (P ^ 1) * TB);" in src
    assert "char q_lds_raw[2 * TB];" in src
    body = src[src.index("void bwd_dkdv_kernel("):]
    assert body.index("ob[i] = fetch(i);") < body.index("copy_q(Qbh, Qbh_hi, t + 1")


@pytest.mark.parametrize("T", list(range(1, 21)))
def test_dkdv_schedule(T):
    dkdv_pass(T).check(f"dK/dV T={T}")


def test_dkdv_schedule_catches_a_copy_into_the_read_buffer():
    """The model is not vacuous: copying the next tile into the buffer being
    read fails."""
    s = Schedule()
    s.copy("QO", 0, 0)
    s.barrier()
    s.read("QO", 0, 0)
    s.copy("QO", 0, 1)
    s.barrier()
    with pytest.raises(AssertionError):
        s.check("bad dK/dV")
