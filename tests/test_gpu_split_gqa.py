"""GPU parity of the split-KV forward (fa_fwd_split) and grouped key/value decode (fa_decode_gqa).

Both are compared with the fp64 oracle at the bf16 tolerances of the forward (O <= 1.6e-2, LSE <= 1e-3).
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention_ref, gqa_decode_ref
from tests.gpu_util import TOL_LSE, TOL_O, inputs, max_err, to_dev, to_host64

pytestmark = pytest.mark.gpu


def fa():
    import exact_tiled_attention_09_amd as m
    return m


def check(O, L, Oref, Lref, what):
    eo, el = max_err(O, Oref), max_err(L, Lref)
    print(f"  {what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O["bf16"], f"O error {eo}"
    assert el <= TOL_LSE, f"LSE error {el}"


SPLIT_CASES = [
    # B, H, Nq, Nkv, d, causal, scale, splits
    (1, 2, 200, 200, 128, True, None, 3),
    (1, 2, 129, 1000, 64, True, None, 4),     # queries at the end of a longer cache; some ranges empty
    (2, 1, 64, 640, 128, False, None, 10),    # one 64-key tile per split
    (1, 1, 1, 77, 128, True, None, 2),
    (1, 2, 300, 5, 64, False, None, 5),       # more splits than tiles: empty ranges
    (1, 2, 100, 3000, 128, True, -0.3, 7),
    (1, 2, 256, 256, 128, False, 2.0, 4),     # very peaked rows
    (1, 1, 50, 50, 64, True, 0.0, 2),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "B{}H{}q{}kv{}d{}c{}s{}S{}".format(*c))
def test_fwd_split(case):
    B, H, Nq, Nkv, d, causal, scale, S = case
    w = syn.custom(B, H, Nq, Nkv, d, "bf16", causal, scale, seed=400 + SPLIT_CASES.index(case))
    host, f64 = inputs(w)
    q, k, v = (to_dev(host[t], "bf16") for t in "qkv")
    print(f"[fa_fwd_split] {case}", flush=True)
    o, lse = fa().attention_split(q, k, v, S, w.scale, causal)
    Oref, Lref = attention_ref(f64["q"], f64["k"], f64["v"], w.scale, causal)
    check(to_host64(o), to_host64(lse), Oref, Lref, w.name)


def test_chunked_prefill_split_full_rows():
    """1000 queries against an 8192-key cache with 4 splits: every row of two heads."""
    w = syn.NEXT_WORKLOADS["chunk"]
    host, f64 = inputs(w)
    q, k, v = (to_dev(host[t], "bf16") for t in "qkv")
    print("[fa_fwd_split] chunked prefill S=4", flush=True)
    o, lse = fa().attention_split(q, k, v, 4, w.scale, True)
    O, L = to_host64(o), to_host64(lse)
    for h in (0, w.H - 1):
        sl = slice(h, h + 1)
        Oref, Lref = attention_ref(f64["q"][:, sl], f64["k"][:, sl], f64["v"][:, sl], w.scale, True)
        check(O[:, sl], L[:, sl], Oref, Lref, f"head {h}")


GQA_CASES = [
    # B, H, H_kv, Nkv, d, splits, scale
    (2, 8, 2, 1000, 128, 4, None),
    (1, 4, 1, 513, 64, 0, None),              # multi-query, auto splits
    (3, 6, 3, 77, 128, 1, None),
    (1, 32, 8, 4096, 128, 16, None),
    (2, 16, 16, 300, 64, 3, -0.25),           # ungrouped
    (1, 64, 4, 2000, 128, 8, 0.0),            # 16 query heads per key/value head, uniform weights
]


@pytest.mark.parametrize("case", GQA_CASES, ids=lambda c: "B{}H{}Hkv{}kv{}d{}S{}s{}".format(*c))
def test_decode_gqa(case):
    B, H, Hkv, Nkv, d, S, scale = case
    rng_seed = 500 + GQA_CASES.index(case)
    wq = syn.custom(B, H, 1, 1, d, "bf16", False, scale, seed=rng_seed)
    wkv = syn.custom(B, Hkv, 1, Nkv, d, "bf16", False, scale, seed=rng_seed + 1000)
    hq = syn.make_tensor(wq, "q")[:, :, 0]
    hk, hv = syn.make_tensor(wkv, "k"), syn.make_tensor(wkv, "v")
    q, k, v = to_dev(hq, "bf16"), to_dev(hk, "bf16"), to_dev(hv, "bf16")
    print(f"[fa_decode_gqa] {case}", flush=True)
    o, lse = fa().decode_gqa(q, k, v, wq.scale, S)
    Oref, Lref = gqa_decode_ref(syn.as_f64(hq, "bf16"), syn.as_f64(hk, "bf16"), syn.as_f64(hv, "bf16"), wq.scale)
    check(to_host64(o), to_host64(lse), Oref, Lref, f"GQA B{B} H{H}/{Hkv} N{Nkv}")
