"""GPU parity: libfa (through its C ABI) against the fp64 CPU oracle on the same seeded inputs.

Bars: max |O - O_ref| <= 2e-5 (fp32 I/O) or 1.6e-2 (bf16 I/O, fp32 accumulation), max |LSE - LSE_ref|
<= 1e-3, absolute, over every compared element, no NaN/Inf.  Every element of every workload is compared,
the full-size ones included (one head or one batch index at a time on the host cores), in the launch
configuration the benchmark times.  Outputs are filled with NaN before the launch, so an element the
kernels never write fails.  Each workload prints its margins as "PARITY <name> max|dO|=... max|dLSE|=...".
"""
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synthetic as syn
from oracle import attention_ref, decode_ref, split_partials_ref
from tests.gpu_util import TOL_LSE, TOL_O, bf16_output_floor, host_workers, inputs, max_err, to_dev, to_host64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_tiled_attention_09_amd as fa
    fa.lib()  # loud failure if the library is missing


def fa():
    import exact_tiled_attention_09_amd as m
    return m


def run_fwd(w: syn.Workload, host):
    """fa_fwd on NaN-filled outputs; returns (O, LSE) as float64 host arrays."""
    q, k, v = (to_dev(host[t], w.dtype) for t in ("q", "k", "v"))
    print(f"[fa_fwd] {w.name} B={w.B} H={w.H} Nq={w.Nq} Nkv={w.Nkv} d={w.d} {w.dtype} causal={w.causal} "
          f"scale={w.scale}", flush=True)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:-1], float("nan"), dtype=torch.float32, device=q.device)
    fa().fa_fwd(q, k, v, o, lse, w.scale, w.causal)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(lse)


def check(w, O, L, Oref, Lref, what=""):
    eo, el = max_err(O, Oref), max_err(L, Lref)
    print(f"  {w.name}{what}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    assert eo <= TOL_O[w.dtype], f"O error {eo} > {TOL_O[w.dtype]}"
    assert el <= TOL_LSE, f"LSE error {el} > {TOL_LSE}"
    return eo, el


def compare_by_head(w, f64, O, L, label):
    """The oracle on every (b, h) slice in parallel on the host cores (numpy releases the GIL in its
    matrix products and element-wise kernels; BLAS is held to one thread per slice), every element of O
    and LSE compared.  Prints the PARITY margin line."""
    from threadpoolctl import threadpool_limits

    pairs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        sl = (slice(b, b + 1), slice(h, h + 1))
        Oref, Lref = attention_ref(f64["q"][sl], f64["k"][sl], f64["v"][sl], w.scale, w.causal)
        floor = bf16_output_floor(Oref) if w.dtype == "bf16" else 0.0
        return max_err(O[sl], Oref), max_err(L[sl], Lref), floor

    with threadpool_limits(1), ThreadPoolExecutor(host_workers()) as ex:
        errs = list(ex.map(one, pairs))
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    floor = max(e[2] for e in errs)
    print(f"PARITY {label} {w.name}: max|dO|={eo:.3e} (bar {TOL_O[w.dtype]:g}; bf16 rounding of the exact O "
          f"alone: {floor:.3e}) max|dLSE|={el:.3e} (bar {TOL_LSE:g}) over {O.size} O and {L.size} LSE elements",
          flush=True)
    assert eo <= TOL_O[w.dtype], f"O error {eo} > {TOL_O[w.dtype]}"
    assert el <= TOL_LSE, f"LSE error {el} > {TOL_LSE}"


# ----------------------------------------------------------------------------- the five workloads

@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4"])
def test_workload_every_element(cfg):
    w = syn.WORKLOADS[cfg]
    host, f64 = inputs(w)
    O, L = run_fwd(w, host)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), "an output element was not written"
    compare_by_head(w, f64, O, L, cfg)


def test_chunked_prefill_workload():
    """1000 new queries against an 8192-key cache (bottom-right causal): every row of every head."""
    w = syn.NEXT_WORKLOADS["chunk"]
    host, f64 = inputs(w)
    O, L = run_fwd(w, host)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    compare_by_head(w, f64, O, L, "chunk")


def test_decode_workload_every_row():
    """The decode workload through fa_decode (16 splits + combine): every (b, h) row of O and LSE and every
    split partial in the workspace, against the oracle one batch index at a time."""
    from threadpoolctl import threadpool_limits

    w = syn.WORKLOADS["c5"]
    print(f"[fa_decode] generating {w.name}", flush=True)
    q_h = syn.make_tensor(w, "q")
    k_h = syn.make_tensor(w, "k")
    v_h = syn.make_tensor(w, "v")
    q, k, v = to_dev(q_h[:, :, 0], "bf16"), to_dev(k_h, "bf16"), to_dev(v_h, "bf16")
    S = w.num_splits
    ws = fa().decode_workspace(w.B, w.H, w.Nkv, w.d, S)
    ws.view(torch.float32).fill_(float("nan"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H), float("nan"), dtype=torch.float32, device="cuda")
    print(f"[fa_decode] {w.name} S={S}", flush=True)
    fa().fa_decode(q, k, v, o, lse, w.scale, S, ws)
    torch.cuda.synchronize()
    O, L = to_host64(o), to_host64(lse)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L)), "an output element was not written"
    n_o = w.B * w.H * S * w.d
    ws_o = ws[: n_o * 4].view(torch.float32).reshape(w.B, w.H, S, w.d).cpu().numpy()
    ws_l = ws[n_o * 4:].view(torch.float32)[: w.B * w.H * S].reshape(w.B, w.H, S).cpu().numpy()

    def one(b):
        qq = syn.as_f64(q_h[b:b + 1], "bf16")[:, :, 0]
        kk = syn.as_f64(k_h[b:b + 1], "bf16")
        vv = syn.as_f64(v_h[b:b + 1], "bf16")
        Oref, Lref = decode_ref(qq, kk, vv, w.scale)
        Os_ref, Ls_ref = split_partials_ref(qq, kk, vv, w.scale, S)
        return (max_err(O[b], Oref[0]), max_err(L[b], Lref[0]), max_err(ws_o[b], Os_ref[0]),
                max_err(ws_l[b], Ls_ref[0]), bf16_output_floor(Oref))

    with threadpool_limits(1), ThreadPoolExecutor(host_workers()) as ex:
        errs = np.array(list(ex.map(one, range(w.B))))
    eo, el, eos, els, floor = errs.max(axis=0)
    print(f"PARITY c5 {w.name}: max|dO|={eo:.3e} (bar {TOL_O['bf16']:g}; bf16 rounding of the exact O alone: "
          f"{floor:.3e}) max|dLSE|={el:.3e} (bar {TOL_LSE:g}) "
          f"over {O.size} O and {L.size} LSE elements; partials max|dO_s|={eos:.3e} max|dlse_s|={els:.3e}",
          flush=True)
    assert eo <= TOL_O["bf16"] and el <= TOL_LSE
    # the fp32 partials are exact up to fp32 accumulation of bf16 products and weights
    assert eos <= 1e-3 and els <= TOL_LSE


def test_device_cu_count_drives_the_plan():
    """The library reads the device's compute-unit count and sizes its launches by it."""
    n = fa().device_num_cu()
    assert n == torch.cuda.get_device_properties(0).multi_processor_count
    for op in (fa().FA_PLAN_FWD, fa().FA_PLAN_DECODE, fa().FA_PLAN_BWD_DKDV):
        assert fa().plan(op, 1, 32, 8192, 8192, 128, True, num_cu=0) == fa().plan(op, 1, 32, 8192, 8192, 128, True,
                                                                                     num_cu=n)


# ----------------------------------------------------------------------------- edge shapes (every element)

EDGE = [
    # B, H, Nq, Nkv, d, dtype, causal, scale
    (1, 1, 1, 1, 64, "bf16", False, None),
    (1, 1, 1, 1, 128, "f32", True, None),
    (2, 3, 17, 17, 64, "bf16", True, None),
    (1, 2, 127, 127, 128, "bf16", True, None),
    (1, 2, 129, 129, 128, "bf16", False, None),
    (1, 1, 1000, 1000, 64, "bf16", True, None),
    (1, 1, 1000, 1000, 128, "f32", True, None),
    (2, 2, 129, 129, 64, "f32", False, None),
    (1, 2, 5, 300, 128, "bf16", True, None),      # queries at the end of a longer cache
    (1, 2, 129, 1000, 64, "bf16", True, None),
    (1, 1, 1, 77, 128, "bf16", True, None),
    (1, 2, 300, 5, 64, "bf16", False, None),      # more queries than keys, no mask
    (1, 2, 200, 200, 128, "bf16", True, 0.0),     # uniform weights over the allowed prefix
    (1, 2, 200, 200, 64, "bf16", True, -0.3),     # negative scale
    (1, 2, 256, 256, 128, "f32", False, -0.05),
    (1, 2, 200, 200, 128, "bf16", False, 2.0),    # very peaked rows
    (1, 1, 333, 333, 64, "f32", False, 0.0),
    (3, 1, 64, 640, 128, "bf16", False, None),
    # fp32 grids of at least one work-group per compute unit keep one wave per 32 rows over the whole row;
    # smaller ones split each row's keys over the waves of a work-group and merge their partials
    (2, 128, 128, 128, 64, "f32", True, None),    # 256 work-groups: whole-row waves
    (2, 128, 100, 300, 128, "f32", False, None),  # 256 work-groups: whole-row waves, ragged
    (1, 3, 40, 70, 64, "f32", True, None),        # key split: 3 tiles for 8 waves, bottom-right causal
    (1, 1, 33, 33, 128, "f32", True, 0.0),        # key split, uniform weights
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "B{}H{}q{}kv{}d{}{}{}s{}".format(*c))
def test_edge_shapes(case):
    B, H, Nq, Nkv, d, dtype, causal, scale = case
    w = syn.custom(B, H, Nq, Nkv, d, dtype, causal, scale, seed=100 + EDGE.index(case))
    host, f64 = inputs(w)
    O, L = run_fwd(w, host)
    Oref, Lref = attention_ref(f64["q"], f64["k"], f64["v"], w.scale, w.causal)
    check(w, O, L, Oref, Lref)


# Causal grids of at least two work-groups per compute unit run query tiles in pairs (tile n-1-j, then tile
# j, in one work-group); every element against the oracle.  Query tiles are 128 rows (4 waves), or 256
# rows (8 waves, one work-group per CU) at d = 128 when B*H*ceil(N_q/256) >= 256.
PAIRED = [
    # B, H, Nq, Nkv, d
    (1, 128, 1100, 1100, 128),  # 8 waves: 5 tiles of 256 per head, two pairs and a lone middle; ragged
    (1, 74, 1100, 1100, 64),    # 9 tiles per head: four pairs and a lone middle tile; ragged last tile
    (2, 36, 1000, 1500, 128),   # 8 waves, 4 unpaired tiles of 256, queries at the end of a longer cache
    (1, 256, 200, 200, 64),     # exactly 512 work-groups before pairing: tile 1 then tile 0
    (1, 255, 200, 200, 128),    # 510: just below the threshold, unpaired
]


@pytest.mark.parametrize("case", PAIRED, ids=lambda c: "B{}H{}q{}kv{}d{}".format(*c))
def test_paired_causal_tiles(case):
    B, H, Nq, Nkv, d = case
    w = syn.custom(B, H, Nq, Nkv, d, "bf16", True, None, seed=400 + PAIRED.index(case))
    host, f64 = inputs(w)
    O, L = run_fwd(w, host)
    Oref, Lref = attention_ref(f64["q"], f64["k"], f64["v"], w.scale, w.causal)
    check(w, O, L, Oref, Lref)


def test_identical_keys_give_mean_of_values():
    w = syn.custom(1, 2, 70, 300, 128, "bf16", False, None, seed=3)
    host, f64 = inputs(w)
    host["k"] = np.broadcast_to(host["k"][:, :, :1], host["k"].shape).copy()
    O, _ = run_fwd(w, host)
    mean_v = f64["v"].mean(axis=2, keepdims=True)
    assert max_err(O, np.broadcast_to(mean_v, O.shape)) <= TOL_O["bf16"]


def test_lse_optional_and_deterministic():
    w = syn.custom(2, 4, 300, 300, 64, "bf16", True, None, seed=9)
    host, _ = inputs(w)
    q, k, v = (to_dev(host[t], "bf16") for t in ("q", "k", "v"))
    o1 = torch.empty_like(q)
    fa().fa_fwd(q, k, v, o1, None, w.scale, True)
    o2, l2 = fa().attention(q, k, v, w.scale, True)
    o3, l3 = fa().attention(q, k, v, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16)) and torch.equal(l2, l3)


DECODE_EDGE = [
    # B, H, Nkv, d, splits, scale
    (2, 2, 1, 128, 1, None),
    (2, 3, 5, 64, 4, None),        # one empty split
    (1, 2, 511, 128, 16, None),
    (1, 2, 513, 128, 16, None),
    (2, 2, 1000, 64, 0, None),     # auto split count
    (1, 1, 3000, 128, 1, None),    # one split longer than the in-kernel chunk
    (1, 1, 100, 128, 100, None),   # one key per split
    (2, 2, 777, 128, 3, -0.2),
    (2, 2, 400, 64, 5, 0.0),
]


@pytest.mark.parametrize("case", DECODE_EDGE, ids=lambda c: "B{}H{}kv{}d{}S{}s{}".format(*c))
def test_decode_edge(case):
    B, H, Nkv, d, S, scale = case
    w = syn.custom(B, H, 1, Nkv, d, "bf16", False, scale, seed=Nkv + S, kind="decode", num_splits=S)
    host, f64 = inputs(w)
    q = to_dev(host["q"][:, :, 0], "bf16")
    k, v = to_dev(host["k"], "bf16"), to_dev(host["v"], "bf16")
    print(f"[fa_decode] B={B} H={H} Nkv={Nkv} d={d} S={S} scale={w.scale}", flush=True)
    o, lse = fa().decode(q, k, v, w.scale, S)
    torch.cuda.synchronize()
    Oref, Lref = decode_ref(f64["q"], f64["k"], f64["v"], w.scale)
    check(w, to_host64(o), to_host64(lse), Oref, Lref)


def test_decode_split_then_combine_equals_decode():
    w = syn.custom(2, 2, 1, 700, 128, "bf16", False, None, seed=21, kind="decode")
    host, _ = inputs(w)
    q = to_dev(host["q"][:, :, 0], "bf16")
    k, v = to_dev(host["k"], "bf16"), to_dev(host["v"], "bf16")
    ws = fa().decode_workspace(2, 2, 700, 128, 6)
    o1, l1 = fa().decode(q, k, v, w.scale, 6, workspace=ws)
    ws2 = fa().decode_workspace(2, 2, 700, 128, 6)
    fa().fa_decode_split(q, k, v, w.scale, 6, ws2)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    fa().fa_decode_combine(ws2, o2, l2, 6)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert torch.equal(ws, ws2)


# ----------------------------------------------------------------------------- stress inputs

STRESS = [
    # B, H, Nq, Nkv, d, dtype, causal, q dist, k dist
    (1, 2, 1000, 1000, 128, "bf16", True, "pos", "ramp"),     # scores rise along the keys: the reference
    (1, 2, 1000, 1000, 128, "bf16", False, "pos", "ramp"),    # maximum must move every few tiles
    (1, 2, 1000, 1000, 64, "bf16", True, "pos", "ramp"),
    (1, 1, 700, 700, 128, "f32", True, "pos", "ramp"),
    (1, 2, 500, 500, 128, "bf16", True, "normal16", "normal"),  # one key dominates almost every row
    # fp32 keeps the 2e-5 bar only while the fp32 score sums are accurate to ~1e-6: at 16x queries their
    # rounding alone reaches ~3e-5 in O, so the fp32 peaked case uses the 4x queries of the c2 workload
    (1, 2, 500, 500, 64, "f32", False, "normal4", "normal"),
]


@pytest.mark.parametrize("case", STRESS, ids=lambda c: "B{}H{}q{}kv{}d{}{}{}_{}_{}".format(*c))
def test_stress_inputs(case):
    B, H, Nq, Nkv, d, dtype, causal, dq, dk = case
    w = syn.custom(B, H, Nq, Nkv, d, dtype, causal, None, seed=300 + STRESS.index(case),
                   dist={"q": dq, "k": dk, "v": "normal"})
    host, f64 = inputs(w)
    O, L = run_fwd(w, host)
    Oref, Lref = attention_ref(f64["q"], f64["k"], f64["v"], w.scale, w.causal)
    check(w, O, L, Oref, Lref)


def test_stress_rising_scores_split_and_decode():
    """Rising scores through the split-KV forward (several ranges) and through decode."""
    w = syn.custom(1, 2, 300, 2000, 128, "bf16", True, None, seed=320, dist={"q": "pos", "k": "ramp", "v": "normal"})
    host, f64 = inputs(w)
    q, k, v = (to_dev(host[t], "bf16") for t in "qkv")
    print("[fa_fwd_split] rising scores", flush=True)
    o, lse = fa().attention_split(q, k, v, 5, w.scale, True)
    Oref, Lref = attention_ref(f64["q"], f64["k"], f64["v"], w.scale, True)
    check(w, to_host64(o), to_host64(lse), Oref, Lref, " split")
    print("[fa_decode] rising scores", flush=True)
    qd = q[:, :, -1].contiguous()
    od, ld = fa().decode(qd, k, v, w.scale, 4)
    Od, Ld = attention_ref(f64["q"][:, :, -1:], f64["k"], f64["v"], w.scale, False)
    check(w, to_host64(od)[:, :, None], to_host64(ld)[:, :, None], Od, Ld, " decode")
