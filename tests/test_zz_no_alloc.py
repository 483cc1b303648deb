"""fa_decode_noalloc (decode with the library's built-in per-GPU scratch, no device allocation) against
fa_decode with a caller workspace, through the C ABI: o and lse bit for bit, and sampled rows against the
oracle at the bf16 bar.  Two calls in a row, the second smaller, so the second runs over the first's
partials left in the shared scratch; then an automatic split count.
"""
import numpy as np
import pytest

from oracle import decode_ref
from tests.gpu_util import TOL_LSE, TOL_O, max_err, to_host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as fa
    fa.lib()


def run_pair(B, H, N, d, S, seed):
    import exact_tiled_attention_09_amd as fa
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, H, d, generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(B, H, N, d, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(B, H, N, d, generator=g, device="cuda").to(torch.bfloat16)
    scale = d ** -0.5
    ws = fa.decode_workspace(B, H, N, d, S)
    o_ws = torch.full_like(q, float("nan"))
    l_ws = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[fa_decode] B={B} H={H} N_kv={N} d={d} S={S} seed={seed}", flush=True)
    fa.fa_decode(q, k, v, o_ws, l_ws, scale, S, ws)
    o_na = torch.full_like(q, float("nan"))
    l_na = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[fa_decode_noalloc] B={B} H={H} N_kv={N} d={d} S={S} seed={seed}", flush=True)
    fa.fa_decode_noalloc(q, k, v, o_na, l_na, scale, S)
    torch.cuda.synchronize()
    assert torch.isfinite(o_na.float()).all() and torch.isfinite(l_na).all(), "an output element was not written"
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), "o differs from fa_decode"
    assert torch.equal(l_na.view(torch.int32), l_ws.view(torch.int32)), "lse differs from fa_decode"
    # sampled batch rows against the oracle
    rows = sorted({0, B - 1, B // 2})
    for b in rows:
        qq, kk, vv = (to_host64(t[b:b + 1]) for t in (q, k, v))
        Oref, Lref = decode_ref(qq, kk, vv, scale)
        eo, el = max_err(to_host64(o_na[b:b + 1]), Oref), max_err(to_host64(l_na[b:b + 1]), Lref)
        print(f"  b={b}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        assert eo <= TOL_O["bf16"] and el <= TOL_LSE


def test_noalloc_matches_decode_then_smaller_call():
    run_pair(64, 32, 8192, 128, 16, seed=41)   # the decode workload's shape: 16.9 MB of partials
    run_pair(3, 5, 1000, 64, 4, seed=42)       # smaller, over the first call's partials


def test_noalloc_auto_splits_and_ragged_ranges():
    run_pair(2, 3, 777, 128, 0, seed=43)       # automatic split count
    run_pair(1, 2, 5, 64, 5, seed=44)          # one key per split
    run_pair(1, 1, 3, 128, 3, seed=45)


def test_noalloc_rejects_what_does_not_fit():
    import exact_tiled_attention_09_amd as fa
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(64, 32, 64, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, float("nan"))
    with pytest.raises(fa.FaError, match="scratch"):
        fa.fa_decode_noalloc(q, k, k, o, None, 0.1, 64)  # 67.6 MB of partials > 32 MiB
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all(), "a rejected call wrote its output"
