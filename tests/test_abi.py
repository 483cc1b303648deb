"""The C ABI on the CPU: the library loads, exports every declared symbol, and rejects bad arguments.

Only validation paths are exercised here: every call below is invalid, so the
library returns before any HIP call and the (host) output buffers stay untouched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
HEADERS = [HEADER, os.path.join(ROOT, "include", "fa_probe.h")]

fa = pytest.importorskip("exact_tiled_attention_09_amd")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    return fa.lib()


def declared_functions(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_bf16", "fa_fwd_f32", "fa_decode", "fa_decode_split", "fa_decode_combine",
              "fa_decode_workspace_bytes", "fa_decode_num_splits", "fa_status_str", "fa_last_error", "fa_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), f"{n} declared in fa.h but not exported by libfa.so"


def test_status_strings(L):
    assert [fa.status_str(s) for s in range(5)] == ["FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED",
                                                    "FA_ERR_WORKSPACE", "FA_ERR_DEVICE"]
    assert "gfx950" in fa.version()


A = 1 << 20  # fake, 16-byte aligned addresses far apart; never dereferenced on rejected calls


def P(i):
    return ctypes.c_void_p(A * (i + 1))


def fwd(L, q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), B=1, H=1, Nq=8, Nkv=8, d=64, scale=0.125, causal=0, dtype=0):
    return L.fa_fwd(q, k, v, o, lse, B, H, Nq, Nkv, d, scale, causal, None, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(q=ctypes.c_void_p(A + 8)), fa.FA_ERR_INVALID_ARG),
    (dict(lse=ctypes.c_void_p(5 * A + 2)), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(Nkv=1 << 23, d=128), fa.FA_ERR_UNSUPPORTED),            # one head's K past a 32-bit byte range
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=1, Nq=9, Nkv=8), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(o=P(0)), fa.FA_ERR_INVALID_ARG),                       # o aliases q
    (dict(lse=ctypes.c_void_p(3 * A + 64)), fa.FA_ERR_INVALID_ARG),  # lse inside o
    (dict(B=1 << 20, H=1 << 20, Nq=1 << 10), fa.FA_ERR_INVALID_ARG),  # size overflow
])
def test_fwd_rejects(L, kw, status):
    assert fwd(L, **kw) == status
    assert fa.last_error() != ""


def test_rejected_call_leaves_outputs_untouched(L):
    q = np.zeros(8 * 96, np.uint16)
    o = np.full(8 * 96, 7, np.uint16)
    lse = np.full(8, 3.0, np.float32)
    st = L.fa_fwd(q.ctypes.data_as(ctypes.c_void_p), q.ctypes.data_as(ctypes.c_void_p),
                  q.ctypes.data_as(ctypes.c_void_p), o.ctypes.data_as(ctypes.c_void_p),
                  lse.ctypes.data_as(ctypes.c_void_p), 1, 1, 8, 8, 96, 0.1, 0, None, 0)
    assert st == fa.FA_ERR_UNSUPPORTED
    assert (o == 7).all() and (lse == 3.0).all()
    assert "d=96" in fa.last_error()


def test_typed_wrappers_validate(L):
    assert L.fa_fwd_bf16(P(0), P(1), P(2), P(3), P(4), 1, 1, 8, 8, 80, 0.1, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert L.fa_fwd_f32(P(0), P(1), P(2), None, P(4), 1, 1, 8, 8, 64, 0.1, 0, None) == fa.FA_ERR_INVALID_ARG


def test_decode_workspace_arithmetic(L):
    # O_s [B,H,S,d] + lse_s [B,H,S], fp32
    assert fa.fa_decode_workspace_bytes(64, 32, 8192, 128, 16) == 64 * 32 * 16 * 129 * 4
    assert fa.fa_decode_workspace_bytes(2, 3, 100, 64, 7) == 2 * 3 * 7 * 65 * 4
    assert fa.fa_decode_workspace_bytes(2, 3, 100, 96, 7) == 0  # unsupported d
    assert fa.fa_decode_workspace_bytes(2, 3, 100, 64, 101) == 0  # more splits than keys
    s = fa.fa_decode_num_splits(1, 1, 100000, 128, 0)
    assert 1 <= s <= 100000
    assert fa.fa_decode_num_splits(64, 32, 8192, 128, 0) >= 1
    assert fa.fa_decode_num_splits(1, 1, 10, 64, 0) == 1
    assert fa.fa_decode_num_splits(4, 4, 1000, 64, 3) == 3
    # split counts for fa_fwd_split: ~512 work-groups, splits of at least 512 keys
    assert fa.fa_fwd_split_num_splits(1, 32, 1000, 8192, 128) == 2     # 256 query tiles of a chunk
    assert fa.fa_fwd_split_num_splits(1, 32, 8192, 8192, 128) == 1     # 2048 query tiles already
    assert fa.fa_fwd_split_num_splits(1, 1, 128, 100000, 64) == 196    # capped by 512-key splits
    assert fa.fa_fwd_split_num_splits(1, 1, 1, 300, 128) == 1
    assert fa.fa_fwd_split_num_splits(1, 1, 1, 300, 96) == 0           # unsupported d
    assert fa.fa_fwd_split_num_splits(0, 1, 1, 300, 64) == 0


def dec(L, q=P(0), k=P(1), v=P(2), o=P(3), lse=P(4), B=2, H=2, Nkv=64, d=128, scale=0.1, S=4, ws=P(6),
        wsb=None, dtype=0):
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(B if B > 0 else 1, H if H > 0 else 1, max(Nkv, 1), 128, max(S, 1))
    return L.fa_decode(q, k, v, o, lse, B, H, Nkv, d, scale, S, ws, wsb, None, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nkv=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=72), fa.FA_ERR_UNSUPPORTED),
    (dict(S=-1), fa.FA_ERR_INVALID_ARG),
    (dict(S=65), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(wsb=16), fa.FA_ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(7 * A + 4)), fa.FA_ERR_WORKSPACE),
    (dict(dtype=1), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=5), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("-inf")), fa.FA_ERR_INVALID_ARG),
    (dict(o=P(1)), fa.FA_ERR_INVALID_ARG),   # o inside k
    (dict(ws=P(3)), fa.FA_ERR_INVALID_ARG),  # workspace overlaps o
])
def test_decode_rejects(L, kw, status):
    assert dec(L, **kw) == status


def test_split_and_combine_validate(L):
    wsb = fa.fa_decode_workspace_bytes(2, 2, 64, 128, 4)
    assert L.fa_decode_split(P(0), P(1), P(2), 2, 2, 64, 128, 0.1, 4, P(6), wsb - 1, None, 0) == fa.FA_ERR_WORKSPACE
    assert L.fa_decode_split(P(0), P(1), P(2), 2, 2, 64, 128, 0.1, 4, P(1), wsb, None, 0) == fa.FA_ERR_INVALID_ARG
    assert L.fa_decode_combine(P(6), wsb, P(3), P(4), 2, 2, 128, 0, None, 0) == fa.FA_ERR_INVALID_ARG
    assert L.fa_decode_combine(P(6), wsb, P(3), P(4), 2, 2, 128, 5, None, 0) == fa.FA_ERR_WORKSPACE
    assert L.fa_decode_combine(P(6), wsb, P(6), P(4), 2, 2, 128, 4, None, 0) == fa.FA_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x, torch.empty_like(x), None, 0.1, False)


def paged(L, q=P(0), kp=P(1), vp=P(2), bt=P(3), sl=P(4), o=P(5), lse=P(6), B=2, H=4, Hkv=2, pages=4, psz=16,
          mb=2, d=128, scale=0.1, S=2, ws=P(8), wsb=None, dtype=0):
    if wsb is None:
        wsb = fa.fa_decode_paged_workspace_bytes(2, 4, 2, 32, 128, 2)
    return L.fa_decode_paged(q, kp, vp, bt, sl, o, lse, B, H, Hkv, pages, psz, mb, d, scale, S, ws, wsb, None, dtype)


def test_paged_workspace_arithmetic(L):
    assert fa.fa_decode_paged_workspace_bytes(2, 4, 2, 32, 128, 2) == 2 * 4 * 2 * 129 * 4
    assert fa.fa_decode_paged_workspace_bytes(2, 4, 3, 32, 128, 2) == 0   # H not a multiple of H_kv
    assert fa.fa_decode_paged_workspace_bytes(2, 4, 2, 0, 128, 2) == 0    # no length bound
    assert fa.fa_decode_paged_num_splits(64, 8, 8192, 128, 0) == fa.fa_decode_num_splits(64, 8, 8192, 128, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(bt=None), fa.FA_ERR_INVALID_ARG),
    (dict(sl=None), fa.FA_ERR_INVALID_ARG),
    (dict(sl=ctypes.c_void_p(5 * A + 2)), fa.FA_ERR_INVALID_ARG),      # seq_lens misaligned
    (dict(kp=ctypes.c_void_p(2 * A + 8)), fa.FA_ERR_INVALID_ARG),
    (dict(Hkv=3), fa.FA_ERR_INVALID_ARG),                             # H % H_kv != 0
    (dict(H=12, Hkv=4, psz=4, mb=8), fa.FA_ERR_UNSUPPORTED),          # 3 per kv head on 4-token pages
    (dict(H=32, Hkv=2, psz=2, mb=16), fa.FA_ERR_UNSUPPORTED),         # 16 per kv head on 2-token pages
    (dict(psz=12), fa.FA_ERR_INVALID_ARG),                            # not a power of two
    (dict(psz=0), fa.FA_ERR_INVALID_ARG),
    (dict(psz=1 << 21), fa.FA_ERR_INVALID_ARG),
    (dict(mb=1 << 27), fa.FA_ERR_INVALID_ARG),                        # max length past 2^30
    (dict(pages=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(S=33), fa.FA_ERR_INVALID_ARG),                              # more splits than max_blocks * page_size
    (dict(S=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=1), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_WORKSPACE),
    (dict(wsb=64), fa.FA_ERR_WORKSPACE),
    (dict(o=P(3)), fa.FA_ERR_INVALID_ARG),                            # o overlaps the block table
    (dict(lse=P(1)), fa.FA_ERR_INVALID_ARG),                          # lse inside the key pool
    (dict(ws=P(4)), fa.FA_ERR_INVALID_ARG),                           # workspace overlaps seq_lens
])
def test_paged_rejects(L, kw, status):
    assert paged(L, **kw) == status
    assert fa.last_error() != ""


def test_probes_reject_bad_arguments(L):
    sink = ctypes.c_void_p(A * 7)
    # NULL, misaligned or too small arguments: status 1, nothing launched
    assert L.fa_probe_read_bandwidth(None, 1 << 20, sink, 1 << 20, 4, None) == 1
    assert L.fa_probe_read_bandwidth(ctypes.c_void_p(A + 8), 1 << 20, sink, 1 << 20, 4, None) == 1
    assert L.fa_probe_read_bandwidth(P(0), 8, sink, 1 << 20, 4, None) == 1
    assert L.fa_probe_read_bandwidth(P(0), 1 << 20, sink, 4 * 512 * 4 - 1, 4, None) == 1
    assert L.fa_probe_read_bandwidth(P(0), 1 << 20, sink, 1 << 20, 0, None) == 1
    assert L.fa_probe_clock(None, 100, 4, 10, None) == 1
    assert L.fa_probe_clock(P(0), 19, 4, 10, None) == 1
    assert L.fa_probe_clock(P(0), 20, 4, 0, None) == 1


def test_noalloc_scratch_limit(L):
    """fa_decode_noalloc: the scratch size in the header is the binding's, and requests whose partials do not
    fit it (or that fa_decode rejects by size) are refused before any device call."""
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES

    def call(B, H, N, d, S):
        return L.fa_decode_noalloc(P(0), P(1), P(2), P(3), P(4), B, H, N, d, 0.1, S, None, 0)

    # 64 x 32 heads x 64 splits x 129 floats = 67.6 MB of partials > 32 MiB
    assert call(64, 32, 8192, 128, 64) == fa.FA_ERR_WORKSPACE
    assert "scratch" in fa.last_error()
    # the largest split count that fits: B*H*S*(d+1)*4 <= 32 MiB
    assert 64 * 32 * 31 * 129 * 4 <= fa.NOALLOC_SCRATCH_BYTES < 64 * 32 * 32 * 129 * 4
    assert call(64, 32, 8192, 128, 32) == fa.FA_ERR_WORKSPACE
    assert call(1, 1, 8, 96, 1) == fa.FA_ERR_UNSUPPORTED
    assert call(1, 1, 8, 64, 9) == fa.FA_ERR_INVALID_ARG
    assert call(0, 1, 8, 64, 1) == fa.FA_ERR_INVALID_ARG
