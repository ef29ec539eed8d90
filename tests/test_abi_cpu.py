"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, computes the zigzag layout bit-exactly, and rejects bad arguments
on the host before any launch (so these calls never reach the HIP runtime)."""
import ctypes
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT
from oracle import cpa_oracle

import sequence_attention_cpa_amd as cpa
from sequence_attention_cpa_amd import _lib

HEADER = os.path.join(ROOT, "include", "cpattn.h")


def header_text():
    """The header's declarations, comments removed."""
    src = open(HEADER, encoding="utf-8").read()
    return re.sub(r"/\*.*?\*/", "", src, flags=re.S)


def header_functions():
    return sorted(set(re.findall(r"\b(cpa_[a-z_]+)\s*\(", header_text())))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libcpattn.so is not built (python -m sequence_attention_cpa_amd.build)")
    return _lib.load()


def test_exports_every_header_symbol(lib):
    names = header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n
    assert cpa.version().startswith("libcpattn")


def test_header_is_plain_c(tmp_path):
    """The header compiles as C99 and links against the library from C."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    prog = tmp_path / "t.c"
    prog.write_text(
        '#include "cpattn.h"\n#include <stdio.h>\n'
        "int main(void){ int64_t out[64]; cpa_status s = cpa_zigzag_layout(64, 4, out);\n"
        ' printf("%d %lld %lld\\n", (int)s, (long long)out[8], (long long)out[16]);\n'
        " return s == CPA_OK && out[8] == 56 && out[16] == 8 ? 0 : 1; }\n")
    exe = tmp_path / "t"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(prog), "-o", str(exe), _lib.LIB_PATH,
                        f"-Wl,-rpath,{os.path.dirname(_lib.LIB_PATH)}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("L,N", [(64, 4), (128, 4), (12288, 4), (131072, 4), (1048576, 8),
                                 (2, 1), (96, 3), (40, 5)])
def test_layout_matches_oracle_bit_exact(lib, L, N):
    got = cpa.zigzag_layout(L, N).numpy()
    assert got.dtype == np.int64
    assert np.array_equal(got, cpa_oracle.zigzag_layout(L, N))


def test_layout_errors(lib):
    with pytest.raises(cpa.CpaError) as e:
        cpa.zigzag_layout(63, 4)
    assert e.value.status == _lib.CPA_ESHAPE and "2N" in str(e.value)
    with pytest.raises(cpa.CpaError) as e:
        cpa.zigzag_layout(64, 0)
    assert e.value.status == _lib.CPA_EINVAL
    assert lib.cpa_zigzag_layout(64, 4, None) == _lib.CPA_EINVAL
    out = (ctypes.c_int64 * 64)()
    assert lib.cpa_zigzag_layout(64, 4, out) == _lib.CPA_OK
    assert cpa.last_error() == ""


# Fake but aligned device addresses: validation must reject before using them.
P = 0x100000


def _partial(lib, **kw):
    a = dict(Q=P, K=P, V=P, dt=_lib.CPA_BF16, B=1, H=2, Lq=64, Lk=64, D=128, q_off=P, k_off=P,
             causal=1, scale=0.0, O=P, lse=P, stream=None)
    a.update(kw)
    return lib.cpa_partial(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["H"], a["Lq"], a["Lk"],
                           a["D"], a["q_off"], a["k_off"], a["causal"], a["scale"], a["O"],
                           a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), _lib.CPA_EDTYPE),
    (dict(D=32), _lib.CPA_EUNSUPPORTED),
    (dict(D=256), _lib.CPA_EUNSUPPORTED),
    (dict(B=0), _lib.CPA_ESHAPE),
    (dict(H=-1), _lib.CPA_ESHAPE),
    (dict(Lq=-1), _lib.CPA_ESHAPE),
    (dict(Lk=(1 << 30) + 1), _lib.CPA_ESHAPE),
    (dict(B=256, H=256), _lib.CPA_ESHAPE),            # B*H above the 65535 grid.y bound
    (dict(Lq=1 << 30, H=64), _lib.CPA_ESHAPE),        # 2^37 work-items in one launch
    (dict(Q=None), _lib.CPA_EINVAL),
    (dict(V=None), _lib.CPA_EINVAL),
    (dict(lse=None), _lib.CPA_EINVAL),
    (dict(q_off=None), _lib.CPA_EINVAL),
    (dict(K=P + 8), _lib.CPA_EINVAL),
    (dict(O=P + 4), _lib.CPA_EINVAL),
    (dict(k_off=P + 4), _lib.CPA_EINVAL),
])
def test_partial_rejects(lib, kw, status):
    assert _partial(lib, **kw) == status
    assert cpa.last_error() != ""


def test_partial_empty_query_block_is_a_no_op(lib):
    """Lq = 0 is valid and enqueues nothing (so it needs no GPU)."""
    assert _partial(lib, Lq=0) == _lib.CPA_OK
    assert _partial(lib, Lq=0, Q=None, O=None, lse=None) == _lib.CPA_OK


def test_merge_rejects(lib):
    assert lib.cpa_merge(P, P, P, P, -1, 128, None) == _lib.CPA_ESHAPE
    assert lib.cpa_merge(P, P, P, P, 10, 8, None) == _lib.CPA_EUNSUPPORTED
    assert lib.cpa_merge(None, P, P, P, 10, 128, None) == _lib.CPA_EINVAL
    assert lib.cpa_merge(P + 4, P, P, P, 10, 128, None) == _lib.CPA_EINVAL
    assert lib.cpa_merge(P, P + 2, P, P, 10, 128, None) == _lib.CPA_EINVAL
    assert lib.cpa_merge(None, None, None, None, 0, 128, None) == _lib.CPA_OK


def test_workspace_size(lib):
    B, H, L, N, D = 1, 4, 131072, 4, 128
    rows = B * H * (L // N)
    want = -(-rows * D * 4 // 256) * 256 + -(-rows * 4 // 256) * 256
    assert cpa.rank_forward_workspace(B, H, L, N, D) == want == 64 * 2**20 + 512 * 2**10
    assert cpa.rank_forward_workspace(1, 1, 63, 4, 16) == 0
    assert cpa.rank_forward_workspace(1, 1, 64, 0, 16) == 0


def _rank(lib, **kw):
    a = dict(i=0, N=4, Q=P, K=P, V=P, pos=P, dt=_lib.CPA_BF16, B=1, H=2, L=256, D=128, causal=1,
             scale=0.0, O=P, lse=P, ws=P, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.cpa_rank_forward(a["i"], a["N"], a["Q"], a["K"], a["V"], a["pos"], a["dt"], a["B"],
                                a["H"], a["L"], a["D"], a["causal"], a["scale"], a["O"], a["lse"],
                                a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(i=4), _lib.CPA_EINVAL),
    (dict(i=-1), _lib.CPA_EINVAL),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(L=260), _lib.CPA_ESHAPE),
    (dict(D=48), _lib.CPA_EUNSUPPORTED),
    (dict(dt=2), _lib.CPA_EDTYPE),
    (dict(pos=None), _lib.CPA_EINVAL),
    (dict(ws=None), _lib.CPA_EINVAL),
    (dict(ws_bytes=1000), _lib.CPA_EINVAL),
    (dict(ws=P + 16), _lib.CPA_EINVAL),
    (dict(Q=P + 2), _lib.CPA_EINVAL),
])
def test_rank_forward_rejects(lib, kw, status):
    assert _rank(lib, **kw) == status
    assert cpa.last_error() != ""


def _noalloc(lib, **kw):
    a = dict(i=0, N=4, Q=P, K=P, V=P, pos=P, dt=_lib.CPA_BF16, B=1, H=2, L=256, D=128, causal=1,
             scale=0.0, O=P, lse=P, stream=None)
    a.update(kw)
    return lib.cpa_rank_forward_noalloc(a["i"], a["N"], a["Q"], a["K"], a["V"], a["pos"], a["dt"],
                                        a["B"], a["H"], a["L"], a["D"], a["causal"], a["scale"],
                                        a["O"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(i=4), _lib.CPA_EINVAL),
    (dict(i=-1), _lib.CPA_EINVAL),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(L=260), _lib.CPA_ESHAPE),
    (dict(D=48), _lib.CPA_EUNSUPPORTED),
    (dict(dt=2), _lib.CPA_EDTYPE),
    (dict(pos=None), _lib.CPA_EINVAL),
    (dict(Q=P + 2), _lib.CPA_EINVAL),
    (dict(O=None), _lib.CPA_EINVAL),
])
def test_rank_forward_noalloc_rejects(lib, kw, status):
    """Host-side checks of the no-allocation ring run before the device scratch
    is looked up, so they need no GPU."""
    assert _noalloc(lib, **kw) == status
    assert cpa.last_error() != ""


def _fused(lib, **kw):
    a = dict(i=0, N=4, Q=P, K=P, V=P, pos=P, dt=_lib.CPA_BF16, B=1, H=2, L=256, D=128, causal=1,
             scale=0.0, O=P, lse=P, stream=None)
    a.update(kw)
    return lib.cpa_rank_forward_fused(a["i"], a["N"], a["Q"], a["K"], a["V"], a["pos"], a["dt"],
                                      a["B"], a["H"], a["L"], a["D"], a["causal"], a["scale"],
                                      a["O"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(i=4), _lib.CPA_EINVAL),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(L=260), _lib.CPA_ESHAPE),
    (dict(dt=_lib.CPA_F32), _lib.CPA_EUNSUPPORTED),
    (dict(D=16), _lib.CPA_EUNSUPPORTED),
    (dict(D=48), _lib.CPA_EUNSUPPORTED),
    (dict(dt=5), _lib.CPA_EDTYPE),
    (dict(pos=None), _lib.CPA_EINVAL),
    (dict(O=P + 4), _lib.CPA_EINVAL),
])
def test_rank_forward_fused_rejects(lib, kw, status):
    assert _fused(lib, **kw) == status
    assert cpa.last_error() != ""


def _perm(lib, **kw):
    a = dict(src=P, dst=P, eb=2, B=1, H=2, L=256, D=128, pos=P, N=4, lo=0, hi=4, inv=0, stream=None)
    a.update(kw)
    return lib.cpa_zigzag_permute(a["src"], a["dst"], a["eb"], a["B"], a["H"], a["L"], a["D"],
                                  a["pos"], a["N"], a["lo"], a["hi"], a["inv"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(eb=3), _lib.CPA_EDTYPE),
    (dict(L=250), _lib.CPA_ESHAPE),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(lo=2, hi=2), _lib.CPA_EINVAL),
    (dict(hi=5), _lib.CPA_EINVAL),
    (dict(lo=-1), _lib.CPA_EINVAL),
    (dict(D=1, eb=2), _lib.CPA_ESHAPE),
    (dict(src=None), _lib.CPA_EINVAL),
    (dict(dst=P + 8), _lib.CPA_EINVAL),
    (dict(pos=P + 4), _lib.CPA_EINVAL),
    (dict(D=0), _lib.CPA_ESHAPE),
])
def test_permute_rejects(lib, kw, status):
    assert _perm(lib, **kw) == status


def test_binding_rejects_cpu_tensors(lib):
    import torch
    x = torch.zeros(1, 2, 64, 16)
    pos = torch.zeros(64, dtype=torch.int64)
    with pytest.raises(cpa.CpaError):
        cpa.partial(x, x, x, pos, pos, True)


def _rope(lib, **kw):
    a = dict(x=P, y=P, dt=_lib.CPA_BF16, B=1, H=2, rows=64, D=128, pos=P, base=10000.0,
             pairing=0, stream=None)
    a.update(kw)
    return lib.cpa_rope(a["x"], a["y"], a["dt"], a["B"], a["H"], a["rows"], a["D"], a["pos"],
                        a["base"], a["pairing"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=9), _lib.CPA_EDTYPE),
    (dict(B=0), _lib.CPA_ESHAPE),
    (dict(rows=-1), _lib.CPA_ESHAPE),
    (dict(D=12), _lib.CPA_EUNSUPPORTED),
    (dict(D=4), _lib.CPA_EUNSUPPORTED),
    (dict(D=520), _lib.CPA_EUNSUPPORTED),
    (dict(base=1.0), _lib.CPA_EINVAL),
    (dict(base=float("nan")), _lib.CPA_EINVAL),
    (dict(base=float("inf")), _lib.CPA_EINVAL),
    (dict(pairing=2), _lib.CPA_EINVAL),
    (dict(pos=None), _lib.CPA_EINVAL),
    (dict(y=None), _lib.CPA_EINVAL),
    (dict(x=P + 8), _lib.CPA_EINVAL),
    (dict(pos=P + 4), _lib.CPA_EINVAL),
])
def test_rope_rejects(lib, kw, status):
    assert _rope(lib, **kw) == status
    assert cpa.last_error() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(off=None), _lib.CPA_EINVAL),
    (dict(first_bad=None), _lib.CPA_EINVAL),
    (dict(off=P + 4), _lib.CPA_EINVAL),
    (dict(first_bad=P + 12), _lib.CPA_EINVAL),
    (dict(rows=-1), _lib.CPA_ESHAPE),
    (dict(n=-5), _lib.CPA_ESHAPE),
    (dict(rows=1 << 40, n=1 << 23), _lib.CPA_ESHAPE),
])
def test_check_offsets_rejects(lib, kw, status):
    a = dict(off=P, rows=4, n=64, first_bad=P + 8192)
    a.update(kw)
    assert lib.cpa_check_offsets(a["off"], a["rows"], a["n"], a["first_bad"], None) == status
    assert cpa.last_error()


def test_debug_offsets_switch(monkeypatch):
    """The binding's offsets check runs only when the switch is on and the
    call is causal, and names the table and entry of the first break."""
    seen = []
    monkeypatch.setattr(cpa, "check_offsets", lambda t: seen.append(t) or t.answer)

    class Table:
        shape = (4, 10)
        answer = None

    bad = Table()
    bad.answer = 23
    cpa.debug_offsets(False)
    cpa._debug_check(True, q_off=bad)
    cpa.debug_offsets(True)
    try:
        cpa._debug_check(False, q_off=bad)
        assert seen == []
        cpa._debug_check(True, q_off=Table(), k_off=Table())
        assert len(seen) == 2
        with pytest.raises(cpa.CpaError) as e:
            cpa._debug_check(True, pos_all=bad)
        assert e.value.status == _lib.CPA_EINVAL and "pos_all" in str(e.value)
        assert "row 2, entry 3" in str(e.value)
    finally:
        cpa.debug_offsets(False)


def test_rope_zero_rows_is_a_no_op(lib):
    assert _rope(lib, rows=0, x=None, y=None, pos=None) == _lib.CPA_OK


def _perm_rope(lib, **kw):
    a = dict(src=P, dst=P + 4096, dt=_lib.CPA_BF16, B=1, H=2, L=256, D=128, pos=P, N=4, lo=0, hi=4,
             base=10000.0, pairing=1, stream=None)
    a.update(kw)
    return lib.cpa_zigzag_permute_rope(a["src"], a["dst"], a["dt"], a["B"], a["H"], a["L"], a["D"],
                                       a["pos"], a["N"], a["lo"], a["hi"], a["base"], a["pairing"],
                                       a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(L=250), _lib.CPA_ESHAPE),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(lo=3, hi=2), _lib.CPA_EINVAL),
    (dict(hi=5), _lib.CPA_EINVAL),
    (dict(D=20), _lib.CPA_EUNSUPPORTED),
    (dict(dt=3), _lib.CPA_EDTYPE),
    (dict(base=0.5), _lib.CPA_EINVAL),
    (dict(pairing=-1), _lib.CPA_EINVAL),
    (dict(src=None), _lib.CPA_EINVAL),
    (dict(dst=P + 8), _lib.CPA_EINVAL),
])
def test_permute_rope_rejects(lib, kw, status):
    assert _perm_rope(lib, **kw) == status
    assert cpa.last_error() != ""


def test_backward_delta_rejects(lib):
    f = lib.cpa_backward_delta
    assert f(P, P, 7, 10, 128, P, None) == _lib.CPA_EDTYPE
    assert f(P, P, _lib.CPA_BF16, -1, 128, P, None) == _lib.CPA_ESHAPE
    assert f(P, P, _lib.CPA_BF16, 10, 32, P, None) == _lib.CPA_EUNSUPPORTED
    assert f(None, P, _lib.CPA_BF16, 10, 128, P, None) == _lib.CPA_EINVAL
    assert f(P, P + 8, _lib.CPA_BF16, 10, 128, P, None) == _lib.CPA_EINVAL
    assert f(None, None, _lib.CPA_BF16, 0, 128, None, None) == _lib.CPA_OK


def _pbwd(lib, **kw):
    a = dict(Q=P, K=P, V=P, dO=P, lse=P, delta=P, dt=_lib.CPA_BF16, B=1, H=2, Lq=64, Lk=64, D=128,
             q_off=P, k_off=P, causal=1, scale=0.0, dQ=P, dK=P, dV=P, stream=None)
    a.update(kw)
    return lib.cpa_partial_backward(a["Q"], a["K"], a["V"], a["dO"], a["lse"], a["delta"], a["dt"],
                                    a["B"], a["H"], a["Lq"], a["Lk"], a["D"], a["q_off"],
                                    a["k_off"], a["causal"], a["scale"], a["dQ"], a["dK"],
                                    a["dV"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dt=4), _lib.CPA_EDTYPE),
    (dict(D=48), _lib.CPA_EUNSUPPORTED),
    (dict(Lq=-2), _lib.CPA_ESHAPE),
    (dict(H=0), _lib.CPA_ESHAPE),
    (dict(B=300, H=300), _lib.CPA_ESHAPE),
    (dict(Lk=1 << 30, H=64), _lib.CPA_ESHAPE),        # dK/dV pass: 2^38 work-items
    (dict(Q=None), _lib.CPA_EINVAL),
    (dict(dO=None), _lib.CPA_EINVAL),
    (dict(delta=None), _lib.CPA_EINVAL),
    (dict(dK=None), _lib.CPA_EINVAL),
    (dict(dV=P + 4), _lib.CPA_EINVAL),
    (dict(dO=P + 2), _lib.CPA_EINVAL),
    (dict(k_off=None), _lib.CPA_EINVAL),
])
def test_partial_backward_rejects(lib, kw, status):
    assert _pbwd(lib, **kw) == status
    assert cpa.last_error() != ""


def test_partial_backward_without_pairs_is_a_no_op(lib):
    assert _pbwd(lib, Lq=0) == _lib.CPA_OK
    assert _pbwd(lib, Lk=0, dK=None, dV=None) == _lib.CPA_OK


def _rbwd(lib, **kw):
    a = dict(i=0, N=4, Q=P, K=P, V=P, pos=P, O=P, dO=P, lse=P, dt=_lib.CPA_BF16, B=1, H=2, L=256,
             D=128, causal=1, scale=0.0, dQ=P, dK=P, dV=P, delta=P, stream=None)
    a.update(kw)
    return lib.cpa_rank_backward(a["i"], a["N"], a["Q"], a["K"], a["V"], a["pos"], a["O"], a["dO"],
                                 a["lse"], a["dt"], a["B"], a["H"], a["L"], a["D"], a["causal"],
                                 a["scale"], a["dQ"], a["dK"], a["dV"], a["delta"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(i=4), _lib.CPA_EINVAL),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(L=260), _lib.CPA_ESHAPE),
    (dict(D=8), _lib.CPA_EUNSUPPORTED),
    (dict(dt=3), _lib.CPA_EDTYPE),
    (dict(pos=None), _lib.CPA_EINVAL),
    (dict(O=None), _lib.CPA_EINVAL),
    (dict(delta=None), _lib.CPA_EINVAL),
    (dict(dK=P + 4), _lib.CPA_EINVAL),
    (dict(lse=None), _lib.CPA_EINVAL),
    (dict(N=1 << 23, L=1 << 31), _lib.CPA_ESHAPE),   # 2^23 blocks: dK/dV launch over 2^32
])
def test_rank_backward_rejects(lib, kw, status):
    assert _rbwd(lib, **kw) == status
    assert cpa.last_error() != ""


def _share(lib, precise=False, **kw):
    a = dict(Q=P, K=P, V=P, dt=_lib.CPA_BF16, B=1, H=2, L=512, D=128, N=4, lo=0, hi=4,
             causal=1, scale=0.0, O=P, lse=P, stream=None)
    a.update(kw)
    fn = lib.cpa_share_forward_precise if precise else lib.cpa_share_forward
    return fn(a["Q"], a["K"], a["V"], a["dt"], a["B"], a["H"], a["L"], a["D"], a["N"], a["lo"],
              a["hi"], a["causal"], a["scale"], a["O"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(L=500), _lib.CPA_ESHAPE),
    (dict(L=128), _lib.CPA_EUNSUPPORTED),      # chunks of 16 keys: not a multiple of 32
    (dict(L=1000), _lib.CPA_EUNSUPPORTED),     # chunk 125: not a multiple of 32
    (dict(dt=_lib.CPA_F32), _lib.CPA_EUNSUPPORTED),
    (dict(D=16), _lib.CPA_EUNSUPPORTED),
    (dict(dt=6), _lib.CPA_EDTYPE),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(lo=2, hi=1), _lib.CPA_EINVAL),
    (dict(V=None), _lib.CPA_EINVAL),
    (dict(B=2, H=32768), _lib.CPA_ESHAPE),
    (dict(L=1 << 30, H=64), _lib.CPA_ESHAPE),        # 2^28 rows per rank x 64 heads
    (dict(O=P + 4), _lib.CPA_EINVAL),
])
@pytest.mark.parametrize("precise", [False, True], ids=["bf16_p", "precise_p"])
def test_share_forward_rejects(lib, kw, status, precise):
    assert _share(lib, precise, **kw) == status
    assert cpa.last_error() != ""


def _share_bwd(lib, **kw):
    a = dict(Q=P, K=P, V=P, O=P, dO=P, lse=P, dt=_lib.CPA_BF16, B=1, H=2, L=512, D=128,
             N=4, lo=0, hi=4, causal=1, scale=0.0, dQ=P, dK=P, dV=P, delta=P, stream=None)
    a.update(kw)
    return lib.cpa_share_backward(a["Q"], a["K"], a["V"], a["O"], a["dO"], a["lse"],
                                  a["dt"], a["B"], a["H"], a["L"], a["D"], a["N"], a["lo"],
                                  a["hi"], a["causal"], a["scale"], a["dQ"], a["dK"], a["dV"],
                                  a["delta"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(L=500), _lib.CPA_ESHAPE),
    (dict(L=128), _lib.CPA_EUNSUPPORTED),      # chunks of 16 rows: not a multiple of 32
    (dict(L=1000), _lib.CPA_EUNSUPPORTED),
    (dict(dt=_lib.CPA_F32), _lib.CPA_EUNSUPPORTED),
    (dict(D=16), _lib.CPA_EUNSUPPORTED),
    (dict(dt=6), _lib.CPA_EDTYPE),
    (dict(N=0), _lib.CPA_EINVAL),
    (dict(lo=3, hi=3), _lib.CPA_EINVAL),
    (dict(hi=5), _lib.CPA_EINVAL),
    (dict(delta=None), _lib.CPA_EINVAL),
    (dict(O=None), _lib.CPA_EINVAL),
    (dict(dK=P + 4), _lib.CPA_EINVAL),
    (dict(lse=P + 2), _lib.CPA_EINVAL),
    (dict(N=1 << 23, L=1 << 29), _lib.CPA_ESHAPE),   # 2^23 blocks x 2 heads x 256 threads
])
def test_share_backward_rejects(lib, kw, status):
    assert _share_bwd(lib, **kw) == status
    assert cpa.last_error() != ""


def test_binding_rejects_mismatched_tensors():
    """The Python layer checks every tensor's shape and dtype against the sizes
    it passes to the library (which sees raw pointers), before any device use:
    these CPU tensors never reach the GPU check."""
    import torch
    bf, f32, i64 = torch.bfloat16, torch.float32, torch.int64
    B, H, L, N, D = 1, 2, 256, 4, 64
    Lr = L // N
    Q = torch.zeros(B, H, L, D, dtype=bf)
    pos = torch.zeros(N, Lr, dtype=i64)
    cases = [
        (lambda: cpa.share_forward(Q, torch.zeros(B, H, L - 64, D, dtype=bf), Q, N, True),
         _lib.CPA_ESHAPE),
        (lambda: cpa.share_forward(Q, torch.zeros(B, H, L, D, dtype=f32), Q, N, True),
         _lib.CPA_EDTYPE),
        (lambda: cpa.share_forward(Q, Q, Q, N, True, lse=torch.zeros(B, H, L - 1)),
         _lib.CPA_ESHAPE),
        (lambda: cpa.partial(Q[:, :, :Lr].contiguous(), Q, Q, pos[0], pos[1], True),
         _lib.CPA_ESHAPE),
        (lambda: cpa.rank_forward_fused(0, N, Q[:, :, :Lr].contiguous(),
                                        torch.zeros(N, B, H, Lr, D, dtype=bf),
                                        torch.zeros(N - 1, B, H, Lr, D, dtype=bf), pos, N, True),
         _lib.CPA_ESHAPE),
        (lambda: cpa.merge(torch.zeros(4, D), torch.zeros(4), torch.zeros(4, D, dtype=bf),
                           torch.zeros(4)), _lib.CPA_EDTYPE),
        (lambda: cpa.zigzag_permute(Q, pos, N, out=torch.zeros(N, B, H, Lr, D, dtype=f32)),
         _lib.CPA_EDTYPE),
        (lambda: cpa.rope(Q, torch.zeros(L - 1, dtype=i64)), _lib.CPA_ESHAPE),
        (lambda: cpa.share_backward(Q, Q, Q, torch.zeros(B, H, L, D), Q,
                                    torch.zeros(B, H, L), N, True, torch.zeros(B, H, L, D),
                                    torch.zeros(B, H, L, D, dtype=bf)), _lib.CPA_EDTYPE),
    ]
    for call, status in cases:
        with pytest.raises(cpa.CpaError) as e:
            call()
        assert e.value.status == status, str(e.value)


def test_inverse_permute_rejects_a_source_of_the_wrong_rank_count():
    """The inverse permute reads rank_hi - rank_lo slices of its source: a
    source holding another number of ranks is refused on the host (these CPU
    tensors never reach the GPU check), so the kernel cannot read past it."""
    import torch
    B, H, L, N, D = 1, 2, 256, 4, 64
    pos = torch.zeros(N, L // N, dtype=torch.int64)
    one_rank = torch.zeros(1, B, H, L // N, D, dtype=torch.bfloat16)
    with pytest.raises(cpa.CpaError) as e:
        cpa.zigzag_permute(one_rank, pos, N, inverse=True)  # default range: all N ranks
    assert e.value.status == _lib.CPA_ESHAPE and "src" in str(e.value)
    with pytest.raises(cpa.CpaError) as e:  # lse-shaped source, 3 ranks for a 2-rank range
        cpa.zigzag_permute(torch.zeros(3, B, H, L // N), pos, N, inverse=True, rank_lo=1,
                           rank_hi=3)
    assert e.value.status == _lib.CPA_ESHAPE


def test_share_calls_take_no_position_table():
    """The global-layout calls address rows through the zigzag closed form and
    take their causal bounds from the same closed form, so they take no table
    that could disagree with it (a contiguous table once gave wrong results
    with CPA_OK)."""
    import inspect
    decl = header_text()
    for name in ("cpa_share_forward", "cpa_share_forward_precise", "cpa_share_backward"):
        i = decl.index(name + "(")
        params = decl[i:decl.index(")", i)]
        assert "pos" not in params and "int64_t" in params, params
    for fn in (cpa.share_forward, cpa.share_backward):
        assert "pos_all" not in inspect.signature(fn).parameters


def test_debug_range_check_of_permute_tables(monkeypatch):
    """Debug mode refuses a permute table with an entry outside [0, L) before
    anything reaches the library (checked here on CPU tensors)."""
    import torch
    import sequence_attention_cpa_amd as m
    monkeypatch.setattr(m, "_debug_offsets", True)
    with pytest.raises(cpa.CpaError) as e:
        m._debug_range(torch.tensor([[0, 5], [6, 64]], dtype=torch.int64), 64)
    assert e.value.status == _lib.CPA_EINVAL and "max 64" in str(e.value)
    with pytest.raises(cpa.CpaError):
        m._debug_range(torch.tensor([[-1, 5]], dtype=torch.int64), 64)
    m._debug_range(torch.tensor([[0, 63]], dtype=torch.int64), 64)


def test_error_text_is_per_thread():
    """Two host threads fail different calls in lockstep: each reads back its
    own message, and a successful call clears it (the header's promise)."""
    import threading

    barrier = threading.Barrier(2)
    seen = {}

    def worker(name, call, want):
        texts = []
        for _ in range(50):
            assert call() != _lib.CPA_OK
            barrier.wait()  # both threads have failed before either reads
            texts.append(cpa.last_error())
            barrier.wait()
        out = (ctypes.c_int64 * 64)()
        assert lib_ok.cpa_zigzag_layout(64, 4, out) == _lib.CPA_OK
        seen[name] = (texts, cpa.last_error(), want)

    lib_ok = _lib.load()
    t1 = threading.Thread(target=worker, args=(
        "layout", lambda: lib_ok.cpa_zigzag_layout(62, 4, (ctypes.c_int64 * 64)()), "2N"))
    t2 = threading.Thread(target=worker, args=(
        "merge", lambda: lib_ok.cpa_merge(P, P, P, P, 10, 48, None), "head_dim"))
    t1.start(); t2.start(); t1.join(); t2.join()
    assert set(seen) == {"layout", "merge"}
    for name, (texts, after, want) in seen.items():
        assert all(want in t for t in texts), f"{name}: {set(texts)}"
        assert after == "", f"{name}: error text not cleared by a successful call"
