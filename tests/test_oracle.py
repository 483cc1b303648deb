"""Pins for the CPU oracle: what the pages and the mathematics fix, independent of the oracle's own code.

Each ``pin_*`` takes an attention function ``attn(q, k, v, scale, causal) -> (O, LSE)``
(float64 [B,H,N,d] in, [B,H,N_q,d] and [B,H,N_q] out) and raises AssertionError
when it disagrees with a closed form, an invariant, a library routine or the
printed table.  The oracle must pass all of them; planted mistakes (mutants, in
test_oracle_mutants.py) must each fail at least one.
"""
import math
import os

import numpy as np
import pytest

from oracle import (attention_ref, combine_ref, merge_partials, probabilities_ref, split_bounds,
                    split_partials_ref, tiled_model)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- pins

def pin_single_key(attn):
    """One key: softmax weight 1, so O = V_0 and LSE = scale * q . k_0."""
    q, k, v = rnd(1, 2, 3, 5, 8), rnd(2, 2, 3, 1, 8), rnd(3, 2, 3, 1, 8)
    for causal in (False, True):
        qq = q if not causal else q[:, :, :1]
        O, L = attn(qq, k, v, 0.37, causal)
        np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), rtol=0, atol=1e-14)
        for b in range(2):
            for h in range(3):
                for i in range(qq.shape[2]):
                    s = 0.37 * sum(qq[b, h, i, t] * k[b, h, 0, t] for t in range(8))
                    assert abs(L[b, h, i] - s) < 1e-12


def pin_identical_keys(attn):
    """All keys equal: uniform weights, O = mean(V), LSE = scale * q . k + ln N."""
    n = 11
    q = rnd(4, 1, 2, 3, 6)
    k = np.broadcast_to(rnd(5, 1, 2, 1, 6), (1, 2, n, 6)).copy()
    v = rnd(6, 1, 2, n, 6)
    O, L = attn(q, k, v, 0.9, False)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-13)
    s = 0.9 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0])
    np.testing.assert_allclose(L, s + math.log(n), atol=1e-12)


def pin_scale_zero(attn):
    """scale = 0: every allowed key weighs the same; causal row i averages V_0..V_{i+off}."""
    nq, nkv = 6, 9
    q, k, v = rnd(7, 1, 1, nq, 4), rnd(8, 1, 1, nkv, 4), rnd(9, 1, 1, nkv, 4)
    O, L = attn(q, k, v, 0.0, False)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(v[0, 0].mean(0), (nq, 4)), atol=1e-14)
    np.testing.assert_allclose(L, math.log(nkv), atol=1e-14)
    O, L = attn(q, k, v, 0.0, True)
    off = nkv - nq
    for i in range(nq):
        np.testing.assert_allclose(O[0, 0, i], v[0, 0, :i + off + 1].mean(0), atol=1e-14)
        assert abs(L[0, 0, i] - math.log(i + off + 1)) < 1e-14


def pin_causal_first_row(attn):
    """Square causal: query 0 sees only key 0, so O_0 = V_0 and LSE_0 = scale q_0 . k_0."""
    q, k, v = rnd(10, 1, 2, 7, 5), rnd(11, 1, 2, 7, 5), rnd(12, 1, 2, 7, 5)
    O, L = attn(q, k, v, 0.5, True)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(L[:, :, 0], 0.5 * (q[:, :, 0] * k[:, :, 0]).sum(-1), atol=1e-13)


def pin_two_keys_logistic(attn):
    """Two keys: the weight of key 0 is the logistic function of the score difference."""
    q, k, v = rnd(13, 1, 1, 4, 3), rnd(14, 1, 1, 2, 3), rnd(15, 1, 1, 2, 3)
    O, L = attn(q, k, v, 0.8, False)
    for i in range(4):
        s0 = 0.8 * float(np.dot(q[0, 0, i], k[0, 0, 0]))
        s1 = 0.8 * float(np.dot(q[0, 0, i], k[0, 0, 1]))
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(O[0, 0, i], w0 * v[0, 0, 0] + (1 - w0) * v[0, 0, 1], atol=1e-14)
        assert abs(L[0, 0, i] - np.logaddexp(s0, s1)) < 1e-13


def pin_key_permutation(attn):
    """Non-causal attention does not depend on the order of the (key, value) pairs."""
    q, k, v = rnd(16, 2, 1, 5, 4), rnd(17, 2, 1, 13, 4), rnd(18, 2, 1, 13, 4)
    perm = np.random.default_rng(19).permutation(13)
    O1, L1 = attn(q, k, v, 0.6, False)
    O2, L2 = attn(q, k[:, :, perm], v[:, :, perm], 0.6, False)
    np.testing.assert_allclose(O1, O2, atol=1e-13)
    np.testing.assert_allclose(L1, L2, atol=1e-13)


def pin_key_shift(attn):
    """K + 1 u^T adds scale*q.u to every score of a row: O unchanged, LSE moves by scale*q.u."""
    q, k, v = rnd(20, 1, 2, 6, 4), rnd(21, 1, 2, 9, 4), rnd(22, 1, 2, 9, 4)
    u = rnd(23, 4)
    for causal in (False, True):
        O1, L1 = attn(q, k, v, 0.7, causal)
        O2, L2 = attn(q, k + u, v, 0.7, causal)
        np.testing.assert_allclose(O1, O2, atol=1e-12)
        np.testing.assert_allclose(L2 - L1, 0.7 * q @ u, atol=1e-12)


def pin_value_affine(attn):
    """Rows of P sum to one, so O(a V + 1 c^T) = a O(V) + c, and O is linear in V."""
    q, k = rnd(24, 1, 1, 5, 4), rnd(25, 1, 1, 8, 4)
    v1, v2, c = rnd(26, 1, 1, 8, 3), rnd(27, 1, 1, 8, 3), rnd(28, 3)
    for causal in (False, True):
        O1, _ = attn(q, k, v1, 0.5, causal)
        O2, _ = attn(q, k, v2, 0.5, causal)
        O3, _ = attn(q, k, 2.5 * v1 - v2 + c, 0.5, causal)
        np.testing.assert_allclose(O3, 2.5 * O1 - O2 + c, atol=1e-12)


def pin_hard_limit(attn):
    """As the scale grows, the softmax tends to a one-hot on the best key: O -> V[argmax]."""
    q, k, v = rnd(29, 1, 1, 6, 4), rnd(30, 1, 1, 10, 4), rnd(31, 1, 1, 10, 4)
    s = q[0, 0] @ k[0, 0].T
    srt = np.sort(s, axis=1)
    gap = (srt[:, -1] - srt[:, -2]).min()
    scale = 60.0 / gap  # runner-up weight <= e^-60
    O, _ = attn(q, k, v, scale, False)
    np.testing.assert_allclose(O[0, 0], v[0, 0][s.argmax(axis=1)], atol=1e-12)


def pin_causal_is_prefix(attn):
    """Bottom-right causal row i equals non-causal attention over keys 0..i+(N_kv-N_q)."""
    for nq, nkv in ((7, 7), (4, 9), (1, 5)):
        q, k, v = rnd(32, 1, 1, nq, 3), rnd(33, 1, 1, nkv, 3), rnd(34, 1, 1, nkv, 3)
        O, L = attn(q, k, v, 0.9, True)
        off = nkv - nq
        for i in range(nq):
            o1, l1 = attn(q[:, :, i:i + 1], k[:, :, :i + off + 1], v[:, :, :i + off + 1], 0.9, False)
            np.testing.assert_allclose(O[0, 0, i], o1[0, 0, 0], atol=1e-13)
            assert abs(L[0, 0, i] - l1[0, 0, 0]) < 1e-13


def pin_scipy(attn):
    """LSE and P against scipy.special.logsumexp / softmax (library routines) on small inputs."""
    from scipy.special import logsumexp, softmax
    q, k, v = rnd(35, 2, 2, 9, 7), rnd(36, 2, 2, 9, 7), rnd(37, 2, 2, 9, 5)
    O, L = attn(q, k, v, 0.3, True)
    for b in range(2):
        for h in range(2):
            S = 0.3 * q[b, h] @ k[b, h].T
            S[np.triu_indices(9, 1)] = -np.inf
            np.testing.assert_allclose(L[b, h], logsumexp(S, axis=1), atol=1e-13)
            np.testing.assert_allclose(O[b, h], softmax(S, axis=1) @ v[b, h], atol=1e-13)


def pin_torch_sdpa(attn):
    """The CPU fp64 scaled_dot_product_attention of PyTorch (the interface the pages name)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    q, k, v = rnd(38, 1, 1, 256, 64), rnd(39, 1, 1, 256, 64), rnd(40, 1, 1, 256, 64)
    for causal in (False, True):
        O, _ = attn(q, k, v, 1 / 8, causal)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                             is_causal=causal, scale=1 / 8).numpy()
        np.testing.assert_allclose(O, ref, atol=1e-12)


PINS = [pin_single_key, pin_identical_keys, pin_scale_zero, pin_causal_first_row, pin_two_keys_logistic,
        pin_key_permutation, pin_key_shift, pin_value_affine, pin_hard_limit, pin_causal_is_prefix,
        pin_scipy, pin_torch_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    pin(attention_ref)


# ----------------------------------------------------------------------------- oracle-specific pins

def test_score_matrix_table():
    """The number of score elements materialised per head equals the page's N x N table."""
    rows = [tuple(int(t) for t in line.split()) for line in open(os.path.join(GOLDEN, "score_matrix_elements.txt"))
            if line.strip() and not line.startswith("#")]
    assert len(rows) == 6
    for n, elems in rows:
        x = np.ones((1, 1, n, 1)) * 0.01
        _, _, count = attention_ref(x, x, x, 1.0, False, panel_rows=2048, return_count=True)
        assert count == elems


def test_rows_of_p_sum_to_one():
    for causal, (nq, nkv) in ((False, (9, 9)), (True, (9, 9)), (True, (5, 12)), (False, (12, 5))):
        P = probabilities_ref(rnd(41, 2, 3, nq, 6) * 3, rnd(42, 2, 3, nkv, 6), 0.5, causal)
        assert np.abs(P.sum(-1) - 1).max() <= 1e-12
        assert (P >= 0).all()
        if causal:
            off = nkv - nq
            for i in range(nq):
                assert (P[..., i, i + off + 1:] == 0).all()


def test_rows_subset_and_panels_agree():
    """Sampled rows and panel sizes give the same rows as the whole-matrix computation."""
    q, k, v = rnd(43, 2, 2, 37, 8), rnd(44, 2, 2, 37, 8), rnd(45, 2, 2, 37, 8)
    for causal in (False, True):
        O, L = attention_ref(q, k, v, 0.4, causal, panel_rows=1000)
        for pr in (1, 5, 16):
            O2, L2 = attention_ref(q, k, v, 0.4, causal, panel_rows=pr)
            np.testing.assert_allclose(O2, O, atol=1e-15)
            np.testing.assert_allclose(L2, L, atol=1e-14)
        rows = np.array([0, 3, 17, 36])
        O3, L3 = attention_ref(q, k, v, 0.4, causal, rows=rows, panel_rows=3)
        np.testing.assert_allclose(O3, O[:, :, rows], atol=1e-15)
        np.testing.assert_allclose(L3, L[:, :, rows], atol=1e-14)


def test_heads_independent():
    q, k, v = rnd(46, 2, 3, 6, 4), rnd(47, 2, 3, 8, 4), rnd(48, 2, 3, 8, 4)
    O, L = attention_ref(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            o, l = attention_ref(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], 0.5, True)
            np.testing.assert_allclose(o[0, 0], O[b, h], atol=1e-15)
            np.testing.assert_allclose(l[0, 0], L[b, h], atol=1e-15)


def test_rejects_row_without_keys():
    with pytest.raises(ValueError):
        attention_ref(rnd(1, 1, 1, 5, 2), rnd(2, 1, 1, 3, 2), rnd(3, 1, 1, 3, 2), 1.0, True)


# ----------------------------------------------------------------------------- the recurrence and the split merge

def test_two_tile_worked_shape():
    """One query, four scores: consuming two tiles of two with a running state gives the same row
    (the shape of the figure in the introduction of "How FlashAttention Speeds Up LLM Attention";
    the page prints no numbers, so the values are unpinned and drawn at random)."""
    q, k, v = rnd(50, 1, 1, 1, 3), rnd(51, 1, 1, 4, 3), rnd(52, 1, 1, 4, 3)
    O, L = attention_ref(q, k, v, 1.0, False)
    O2, L2 = tiled_model(q, k, v, 1.0, False, tile=2)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    np.testing.assert_allclose(L2, L, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_recurrence_brute_force(causal):
    """Every tile width from 1 to N gives the full-row result, including the peaked rows."""
    rng = np.random.default_rng(53)
    for nq, nkv, d in ((1, 1, 1), (3, 3, 2), (5, 12, 4), (12, 12, 5), (16, 16, 8), (2, 16, 3)):
        if not causal and nq > nkv:
            continue
        for trial in range(2):
            scale = (4.0 if trial else 1.0)
            q = rng.standard_normal((1, 2, nq, d)) * (3 if trial else 1)
            k, v = rng.standard_normal((1, 2, nkv, d)), rng.standard_normal((1, 2, nkv, d))
            O, L = attention_ref(q, k, v, scale, causal)
            for tile in range(1, nkv + 1):
                O2, L2 = tiled_model(q, k, v, scale, causal, tile)
                np.testing.assert_allclose(O2, O, atol=1e-13, rtol=0)
                np.testing.assert_allclose(L2, L, atol=1e-13, rtol=0)


def test_split_combine_every_split_count():
    """Splitting the keys into S contiguous ranges (some empty) and combining gives the full row."""
    rng = np.random.default_rng(54)
    for nkv in (1, 2, 7, 16, 33):
        q = rng.standard_normal((2, 2, 1, 8)) * 2
        k, v = rng.standard_normal((2, 2, nkv, 8)), rng.standard_normal((2, 2, nkv, 8))
        O, L = attention_ref(q, k, v, 0.5, False)
        for S in range(1, nkv + 4):
            b = split_bounds(nkv, S)
            assert b[0][0] == 0 and b[-1][1] == nkv and all(b[i][1] == b[i + 1][0] for i in range(S - 1))
            Os, Ls = split_partials_ref(q, k, v, 0.5, S)
            Oc, Lc = combine_ref(Os, Ls)
            np.testing.assert_allclose(Oc, O[:, :, 0], atol=1e-13)
            np.testing.assert_allclose(Lc, L[:, :, 0], atol=1e-13)


def test_merge_is_commutative_and_associative():
    rng = np.random.default_rng(55)
    q = rng.standard_normal((1, 1, 3, 4))
    k, v = rng.standard_normal((1, 1, 12, 4)), rng.standard_normal((1, 1, 12, 4))
    parts = [attention_ref(q, k[:, :, a:a + 4], v[:, :, a:a + 4], 1.0, False) for a in (0, 4, 8)]
    ab = merge_partials(*parts[0], *parts[1])
    ab_c = merge_partials(*ab, *parts[2])
    bc = merge_partials(*parts[1], *parts[2])
    a_bc = merge_partials(*parts[0], *bc)
    ba = merge_partials(*parts[1], *parts[0])
    full = attention_ref(q, k, v, 1.0, False)
    for x, y in ((ab_c, full), (a_bc, full), (ba, ab)):
        np.testing.assert_allclose(x[0], y[0], atol=1e-14)
        np.testing.assert_allclose(x[1], y[1], atol=1e-14)
    # an empty partial (LSE = -inf) carries no weight
    e = merge_partials(*parts[0], np.zeros_like(parts[0][0]), np.full_like(parts[0][1], -np.inf))
    np.testing.assert_allclose(e[0], parts[0][0], atol=0)
    np.testing.assert_allclose(e[1], parts[0][1], atol=0)
