"""Pins for the backward oracle (gradients of attention), each independent of its formulas.

* finite differences of the forward oracle (a different code path: only attention_ref is used);
* torch autograd of torch's own scaled_dot_product_attention in fp64 on the CPU (a library routine);
* closed forms: a single key (dQ = dK = 0, dV = sum of dO); scale = 0 (dQ = dK = 0, dV = dO averaged
  over the rows that may see each key); identical keys (dQ = 0);
* the identity rowsum(P * dP) = rowsum(dO * O), which the GPU kernels rely on.

Planted mistakes (copies of the oracle with one change) must each fail at least one pin.
"""
import numpy as np
import pytest

import oracle.attention as oa
from oracle import attention_bwd_ref, attention_ref, allowed_mask, probabilities_ref


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(nq, nkv, d, seed, B=1, H=1):
    q = _rand((B, H, nq, d), seed)
    k = _rand((B, H, nkv, d), seed + 1)
    v = _rand((B, H, nkv, d), seed + 2)
    do = _rand((B, H, nq, d), seed + 3)
    return q, k, v, do


def pin_finite_differences(bwd):
    for nq, nkv, causal in ((3, 5, False), (4, 4, True), (3, 6, True)):
        q, k, v, do = _inputs(nq, nkv, 3, 10 + nq + nkv)
        scale = 0.7
        dq, dk, dv = bwd(q, k, v, do, scale, causal)

        def loss(q_, k_, v_):
            return float((attention_ref(q_, k_, v_, scale, causal)[0] * do).sum())

        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += eps
                xm[idx] -= eps
                args_p = {"q": q, "k": k, "v": v}
                args_m = dict(args_p)
                args_p[name], args_m[name] = xp, xm
                num[idx] = (loss(**{a + "_": b for a, b in args_p.items()}) -
                            loss(**{a + "_": b for a, b in args_m.items()})) / (2 * eps)
            assert np.abs(num - g).max() <= 1e-7 * max(1.0, np.abs(num).max()), (name, nq, nkv, causal)


def pin_torch_autograd(bwd):
    torch = pytest.importorskip("torch")
    for nq, nkv, causal in ((7, 7, True), (5, 9, True), (6, 4, False)):
        q, k, v, do = _inputs(nq, nkv, 8, 40 + nq, B=2, H=2)
        scale = 0.3
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        mask = torch.tensor(allowed_mask(nq, nkv, causal))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
        o.backward(torch.tensor(do))
        dq, dk, dv = bwd(q, k, v, do, scale, causal)
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.abs(got - ref.numpy()).max() <= 1e-10


def pin_single_key(bwd):
    q, k, v, do = _inputs(5, 1, 4, 3, B=1, H=2)
    dq, dk, dv = bwd(q, k, v, do, 0.9, False)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    assert np.abs(dv - do.sum(axis=2, keepdims=True)).max() <= 1e-12


def pin_scale_zero(bwd):
    for causal in (False, True):
        q, k, v, do = _inputs(6, 6, 4, 5)
        dq, dk, dv = bwd(q, k, v, do, 0.0, causal)
        assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
        allowed = allowed_mask(6, 6, causal).astype(np.float64)
        expect = (allowed / allowed.sum(axis=1, keepdims=True)).T @ do[0, 0]
        assert np.abs(dv[0, 0] - expect).max() <= 1e-12


def pin_identical_keys(bwd):
    q, _, v, do = _inputs(5, 7, 4, 8)
    k = np.broadcast_to(_rand((1, 1, 1, 4), 9), (1, 1, 7, 4)).copy()
    dq, _, _ = bwd(q, k, v, do, 0.8, False)
    assert np.abs(dq).max() <= 1e-12


def pin_delta_identity(bwd):
    # rowsum(P * dP) equals rowsum(dO * O): the gradient does not change if the kernels use either
    for causal in (False, True):
        q, k, v, do = _inputs(6, 9, 5, 12)
        P = probabilities_ref(q, k, 0.5, causal)
        dP = do @ np.swapaxes(v, -1, -2)
        O = attention_ref(q, k, v, 0.5, causal)[0]
        assert np.abs((P * dP).sum(-1) - (do * O).sum(-1)).max() <= 1e-12


PINS = [pin_finite_differences, pin_torch_autograd, pin_single_key, pin_scale_zero, pin_identical_keys]


@pytest.mark.parametrize("pin", PINS + [pin_delta_identity], ids=lambda f: f.__name__)
def test_pin(pin):
    pin(attention_bwd_ref)


def _mutant(change):
    """attention_bwd_ref with one planted change (the oracle's own steps, one of them altered)."""
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        B, H, n_q, _ = q.shape
        mask = allowed_mask(n_q, k.shape[2], causal)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                P, _ = oa._softmax_panel(scale * (q[b, h] @ k[b, h].T), mask)
                dP = do[b, h] @ v[b, h].T
                D = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - D)
                if change == "no_delta":
                    dS = P * dP
                if change == "delta_unweighted":
                    dS = P * (dP - dP.sum(axis=1, keepdims=True))
                dv[b, h] = (dS.T if change == "dv_from_ds" else P.T) @ do[b, h]
                dq[b, h] = scale * (dS @ (v[b, h] if change == "dq_uses_v" else k[b, h]))
                dk[b, h] = (1.0 if change == "dk_no_scale" else scale) * (dS.T @ q[b, h])
                if change == "dk_sign":
                    dk[b, h] = -dk[b, h]
        return dq, dk, dv
    return bwd


MUTANTS = ["no_delta", "delta_unweighted", "dv_from_ds", "dq_uses_v", "dk_no_scale", "dk_sign"]


@pytest.mark.parametrize("change", MUTANTS)
def test_mutant_is_caught(change):
    bwd = _mutant(change)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bwd)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {change} passed every pin"


def test_unmutated_copy_passes():
    # the mutant harness itself is faithful: with no change it passes every pin
    for pin in PINS:
        pin(_mutant("none"))
