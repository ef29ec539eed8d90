"""Child process of tests/test_sanitize_cpu.py: the C-ABI tests, then every
call's success path with large sizes, against the sanitizer build of the
host layer (argv[1]; its kernel launchers are stubs that touch no memory)
instead of libcpattn.so."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
from sequence_attention_cpa_amd import _lib  # noqa: E402

_lib.LIB_PATH = sys.argv[1]
import pytest  # noqa: E402

# the C program of test_header_is_plain_c links the real library; the rest
# call the host layer through ctypes
rc = pytest.main([os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q", "-x",
                  "-s", "-p", "no:cacheprovider", "-k", "not plain_c"])
if rc != 0:
    sys.exit(int(rc))

lib = _lib.load()
P = 1 << 20  # a 256-byte aligned stand-in address: the stub launchers never use it
BF, F32 = _lib.CPA_BF16, _lib.CPA_F32
ws = lib.cpa_rank_forward_workspace(1, 4, 1 << 20, 8, 128)
layout = (ctypes.c_int64 * 64)()
calls = {
    "zigzag_layout": lambda: lib.cpa_zigzag_layout(64, 4, ctypes.cast(layout, _lib._c_i64p)),
    "partial": lambda: lib.cpa_partial(P, P, P, BF, 1, 4, 131072, 131072, 128, P, P, 1, 0.0, P, P,
                                       None),
    "merge": lambda: lib.cpa_merge(P, P, P, P, 1 << 24, 128, None),
    "rank_forward": lambda: lib.cpa_rank_forward(3, 8, P, P, P, P, BF, 1, 4, 1 << 20, 128, 1,
                                                 0.0, P, P, P, ws, None),
    "rank_forward f32": lambda: lib.cpa_rank_forward(1, 4, P, P, P, P, F32, 2, 3, 4096, 16, 1,
                                                     0.0, P, P, P, 1 << 30, None),
    # head slices, then row slices of one head, then N == 1 (no scratch)
    "rank_forward_noalloc heads": lambda: lib.cpa_rank_forward_noalloc(
        1, 4, P, P, P, P, BF, 1, 32, 12288, 128, 1, 0.0, P, P, None),
    "rank_forward_noalloc rows": lambda: lib.cpa_rank_forward_noalloc(
        0, 8, P, P, P, P, BF, 1, 4, 1 << 20, 128, 1, 0.0, P, P, None),
    "rank_forward_noalloc one rank": lambda: lib.cpa_rank_forward_noalloc(
        0, 1, P, P, P, P, F32, 1, 2, 512, 64, 0, 0.0, P, P, None),
    "rank_forward_fused": lambda: lib.cpa_rank_forward_fused(2, 4, P, P, P, P, BF, 1, 4, 131072,
                                                             128, 1, 0.0, P, P, None),
    "share_forward": lambda: lib.cpa_share_forward(P, P, P, BF, 1, 4, 1 << 20, 128, 8, 0, 8, 1,
                                                   0.0, P, P, None),
    "share_forward_precise": lambda: lib.cpa_share_forward_precise(P, P, P, BF, 1, 4, 1 << 20, 128,
                                                                   8, 0, 8, 1, 0.0, P, P, None),
    "zigzag_permute": lambda: lib.cpa_zigzag_permute(P, P, 2, 1, 4, 1 << 20, 128, P, 8, 0, 8, 1,
                                                     None),
    "backward_delta": lambda: lib.cpa_backward_delta(P, P, BF, 1 << 22, 128, P, None),
    "partial_backward": lambda: lib.cpa_partial_backward(P, P, P, P, P, P, BF, 1, 4, 8192, 8192,
                                                         128, P, P, 1, 0.0, P, P, P, None),
    "rank_backward": lambda: lib.cpa_rank_backward(1, 4, P, P, P, P, P, P, P, BF, 1, 4, 131072,
                                                   128, 1, 0.0, P, P, P, P, None),
    "rank_backward f32": lambda: lib.cpa_rank_backward(1, 4, P, P, P, P, P, P, P, F32, 1, 2, 256,
                                                       16, 1, 0.0, P, P, P, P, None),
    "share_backward": lambda: lib.cpa_share_backward(P, P, P, P, P, P, BF, 1, 4, 131072, 128, 4, 0,
                                                     4, 1, 0.0, P, P, P, P, None),
    "rope": lambda: lib.cpa_rope(P, P, BF, 1, 4, 1 << 20, 128, P, 10000.0, 0, None),
    "zigzag_permute_rope": lambda: lib.cpa_zigzag_permute_rope(P, P, BF, 1, 4, 131072, 128, P, 4, 0,
                                                               4, 10000.0, 1, None),
    "check_offsets": lambda: lib.cpa_check_offsets(P, 8, 1 << 17, P, None),
}
bad = {name: st for name, call in calls.items() if (st := call()) != _lib.CPA_OK}
assert not bad, {n: (s, lib.cpa_last_error()) for n, s in bad.items()}
# L = 64, N = 4: chunks of C = 8, rank r holds chunk r then chunk 7 - r
assert list(layout) == [(r if t < 8 else 7 - r) * 8 + t % 8 for r in range(4) for t in range(16)]
print(f"sanitized success paths: {len(calls)} calls OK", flush=True)
