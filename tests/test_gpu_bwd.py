"""GPU parity of the backward pass (fa_bwd) against the fp64 gradient oracle.

The forward output o and lse come from fa_fwd (as in training); dO is a seeded N(0,1) bf16 tensor.

Tolerance, derived before looking at any result (the pages give no figure).  The kernels compute
P = exp(s - LSE) in fp32 from fp32 scores, round P to bf16 for dV = P^T dO, form dS = P * (dP - D) in fp32
with D = rowsum(dO * O) taken from the bf16 forward output, round dS to bf16 for dQ = scale dS K and
dK = scale dS^T Q, accumulate every product in fp32 and round each gradient to bf16.  With the bf16 unit
roundoff u = 2^-8, first-order error analysis of those steps bounds every element by
    |d dV| <= u (|P|^T |dO|) + u |dV|
    |d dQ| <= scale (u |dS| |K| + (|P| * dD) |K|) + u |dQ|
    |d dK| <= scale (u |dS|^T |Q| + (|P| * dD)^T |Q|) + u |dK|
where dD = 2u rowsum(|dO| * (|P| |V|)) bounds the error of D through the forward output (its own bf16
weights and its bf16 rounding).  fp32 accumulation (n 2^-24 relative, n <= 8192) and the fp32 scores,
exponentials and LSE add terms orders of magnitude smaller, which the factor 2 of the bar covers together
with the second-order terms: the test requires |g - g_ref| <= 2 x bound for every element of dQ, dK, dV.
rounding_bound() computes the bound from the fp64 inputs; it is a tolerance, not a value compared with.
Each case also prints max|g - g_ref| / max|g_ref| and the relative Frobenius error (observations only).
"""
import numpy as np
import pytest

import synthetic as syn
from oracle import attention_bwd_ref
from tests.gpu_util import to_dev, to_host64

pytestmark = pytest.mark.gpu

U = 2.0 ** -8  # bf16 unit roundoff


def rounding_bound(q, k, v, do, scale, causal):
    """Elementwise first-order bounds (dq, dk, dv) of the errors the kernels' bf16 roundings can cause,
    computed from the fp64 inputs [B, H, N, d] one (b, h) slice at a time."""
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    n_q, n_kv = q.shape[2], k.shape[2]
    allowed = np.arange(n_kv)[None, :] <= np.arange(n_q)[:, None] + (n_kv - n_q) if causal else None
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            s = scale * Q @ K.T
            if causal:
                s = np.where(allowed, s, -np.inf)
            p = np.exp(s - s.max(-1, keepdims=True))
            p /= p.sum(-1, keepdims=True)
            o = p @ V
            dp = dO @ V.T
            dd = (dO * o).sum(-1, keepdims=True)
            ds = p * (dp - dd)
            dq, dk, dv = scale * ds @ K, scale * ds.T @ Q, p.T @ dO
            e_d = 2 * U * (np.abs(dO) * (p @ np.abs(V))).sum(-1, keepdims=True)  # error of D
            pe = p * e_d                                                          # its effect on dS
            bv[b, h] = U * (p.T @ np.abs(dO)) + U * np.abs(dv)
            bq[b, h] = abs(scale) * (U * (np.abs(ds) @ np.abs(K)) + pe @ np.abs(K)) + U * np.abs(dq)
            bk[b, h] = abs(scale) * (U * (np.abs(ds).T @ np.abs(Q)) + pe.T @ np.abs(Q)) + U * np.abs(dk)
    return bq, bk, bv


def fa():
    import exact_tiled_attention_09_amd as m
    return m


def run_case(B, H, Nq, Nkv, d, causal, scale, seed, dist=None):
    import torch
    w = syn.custom(B, H, Nq, Nkv, d, "bf16", causal, scale, seed=seed, dist=dist)
    host = {t: syn.make_tensor(w, t) for t in ("q", "k", "v", "do")}
    f64 = {t: syn.as_f64(host[t], "bf16") for t in host}
    q, k, v, do = (to_dev(host[t], "bf16") for t in ("q", "k", "v", "do"))
    print(f"[fa_bwd] B={B} H={H} Nq={Nq} Nkv={Nkv} d={d} causal={causal} scale={w.scale}", flush=True)
    o, lse = fa().attention(q, k, v, w.scale, causal)
    dq, dk, dv = fa().attention_backward(q, k, v, o, lse, do, w.scale, causal)
    torch.cuda.synchronize()
    ref = attention_bwd_ref(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, causal)
    bounds = rounding_bound(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, causal)
    out = {}
    for name, got, r, bd in (("dq", dq, ref[0], bounds[0]), ("dk", dk, ref[1], bounds[1]),
                             ("dv", dv, ref[2], bounds[2])):
        g = to_host64(got)
        assert np.all(np.isfinite(g)), name
        scale_ref = max(np.abs(r).max(), 1e-30)
        e_max = np.abs(g - r).max() / scale_ref
        e_fro = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)
        ratio = within_bound(g, r, bd)
        print(f"  {name}: max|err|/(2 x bound) = {ratio:.3f}  [max|err|/max|ref| = {e_max:.3e}  frobenius rel = "
              f"{e_fro:.3e}  max|ref| {scale_ref:.3e}]", flush=True)
        out[name] = (ratio, g, r)
    return out


def within_bound(g, r, bound):
    """max over elements of |g - r| / (2 x bound); elements whose bound is exactly 0 must match exactly."""
    err = np.abs(g - r)
    zero = bound == 0
    if np.any(err[zero] != 0):
        return float("inf")
    return float((err[~zero] / (2 * bound[~zero])).max()) if np.any(~zero) else 0.0


CASES = [
    # B, H, Nq, Nkv, d, causal, scale
    (1, 2, 64, 64, 64, True, None),
    (2, 2, 128, 128, 128, False, None),
    (1, 2, 200, 200, 128, True, None),
    (1, 1, 129, 300, 64, True, None),       # queries at the end of a longer cache
    (1, 2, 300, 5, 64, False, None),        # more queries than keys
    (1, 1, 1, 1, 128, False, None),
    (1, 1, 1, 77, 128, True, None),
    (1, 2, 33, 1000, 128, False, None),
    (1, 2, 160, 160, 64, True, 0.0),        # uniform weights: dq = dk = 0
    (1, 2, 160, 160, 128, True, -0.2),      # negative scale
    (1, 1, 1000, 1000, 128, True, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}H{}q{}kv{}d{}c{}s{}".format(*c))
def test_bwd_parity(case):
    out = run_case(*case, seed=200 + CASES.index(case))
    for name, (ratio, g, r) in out.items():
        assert ratio <= 1.0, f"{name}: error / (2 x rounding bound) = {ratio}"


# Causal grids of at least two work-groups per compute unit pair blocks j and n-1-j in one work-group, in
# both kernels (query blocks of 128 for dQ; key blocks of 256 at d = 128, 128 at d = 64 for dK / dV).
PAIRED = [
    # B, H, Nq, Nkv, d
    (1, 74, 1100, 1100, 64),    # 9 blocks per head each way: four pairs and a lone middle block; ragged
    (2, 36, 1000, 1500, 128),   # 8 query blocks (paired), 6 key blocks (not); queries at the end of a longer cache
    (1, 256, 200, 200, 64),     # exactly 512 work-groups per kernel before pairing
    (2, 64, 600, 1100, 128),    # d = 128: 5 key blocks of 256 and 5 query blocks of 128 per head, both paired
]


@pytest.mark.parametrize("case", PAIRED, ids=lambda c: "B{}H{}q{}kv{}d{}".format(*c))
def test_bwd_paired_blocks(case):
    B, H, Nq, Nkv, d = case
    out = run_case(B, H, Nq, Nkv, d, True, None, seed=450 + PAIRED.index(case))
    for name, (ratio, g, r) in out.items():
        assert ratio <= 1.0, f"{name}: error / (2 x rounding bound) = {ratio}"


@pytest.mark.parametrize("dist", [{"q": "pos", "k": "ramp", "v": "normal"}, {"q": "normal16", "k": "normal",
                                                                              "v": "normal"}],
                         ids=["rising_scores", "peaked_rows"])
def test_bwd_stress_inputs(dist):
    """Scores that rise along the keys (LSE up to ~118) and very peaked rows.  For dQ = scale sum_j dS_ij k_j
    the rising keys share a large common part that cancels in the sum (sum_j dS_ij = 0), so the bf16
    roundings of dS and of O (through D) are amplified far beyond u |dQ|: the elementwise bound accounts
    for exactly that through |dS| |K| and (|P| dD) |K|."""
    B, H, N, d, seed = 1, 2, 600, 128, 250
    out = run_case(B, H, N, N, d, True, None, seed=seed, dist=dist)
    for name, (ratio, g, r) in out.items():
        assert ratio <= 1.0, f"{name}: error / (2 x rounding bound) = {ratio}"


def test_bwd_deterministic():
    import torch
    w = syn.custom(1, 2, 300, 300, 128, "bf16", True, None, seed=7)
    q, k, v, do = (to_dev(syn.make_tensor(w, t), "bf16") for t in ("q", "k", "v", "do"))
    o, lse = fa().attention(q, k, v, w.scale, True)
    a = fa().attention_backward(q, k, v, o, lse, do, w.scale, True)
    b = fa().attention_backward(q, k, v, o, lse, do, w.scale, True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_full_causal_prefill_one_head_sampled():
    """The causal prefill shape (N = 8192, d = 128) on one head: dQ rows and dK / dV rows sampled against
    the oracle restricted to them (the oracle materialises the head's 8192 x 8192 matrices once)."""
    import torch
    w = syn.custom(1, 1, 8192, 8192, 128, "bf16", True, None, seed=300)
    host = {t: syn.make_tensor(w, t) for t in ("q", "k", "v", "do")}
    f64 = {t: syn.as_f64(host[t], "bf16") for t in host}
    q, k, v, do = (to_dev(host[t], "bf16") for t in ("q", "k", "v", "do"))
    print("[fa_bwd] B=1 H=1 N=8192 d=128 causal", flush=True)
    o, lse = fa().attention(q, k, v, w.scale, True)
    dq, dk, dv = fa().attention_backward(q, k, v, o, lse, do, w.scale, True)
    torch.cuda.synchronize()
    ref = attention_bwd_ref(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, True)
    bounds = rounding_bound(f64["q"], f64["k"], f64["v"], f64["do"], w.scale, True)
    rows = np.unique(np.concatenate([np.arange(0, 8192, 97), [1, 127, 128, 4095, 8190, 8191]]))
    for name, got, r, bd in (("dq", dq, ref[0], bounds[0]), ("dk", dk, ref[1], bounds[1]),
                             ("dv", dv, ref[2], bounds[2])):
        g = to_host64(got)
        assert np.all(np.isfinite(g)), name
        ratio = within_bound(g[0, 0, rows], r[0, 0, rows], bd[0, 0, rows])
        print(f"  {name}: max|err|/(2 x bound) on {rows.size} rows = {ratio:.3f}", flush=True)
        assert ratio <= 1.0, f"{name}: {ratio}"

