"""Pins for the paged-KV decode oracle (paged_decode_ref), each independent of its gather code.

* an in-order page layout of a contiguous cache reduces to the (separately pinned) decode oracle;
* permuting the physical pages and the block table alike changes nothing;
* a shorter sequence length equals the decode oracle on that prefix;
* table entries outside the page pool drop exactly their tokens;
* with fewer key/value heads than query heads it equals the (separately pinned) grouped-head decode oracle;
* lengths beyond the table's width are cut at its width, negative lengths give an empty sequence.
Planted mistakes (page index off by one, row within the page shifted, length ignored) must fail a pin.
"""
import numpy as np
import pytest

from oracle import decode_ref, gqa_decode_ref, paged_decode_ref


def _contiguous(B, H, N, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, H, d)), rng.standard_normal((B, H, N, d)), rng.standard_normal((B, H, N, d))


def _to_pages(k, P):
    """[B, H, N, d] -> pages [B * N / P, H, P, d] in order, and the identity block table."""
    B, H, N, d = k.shape
    pages = k.reshape(B, H, N // P, P, d).transpose(0, 2, 1, 3, 4).reshape(B * (N // P), H, P, d)
    table = np.arange(B * (N // P)).reshape(B, N // P)
    return pages, table


def pin_in_order_layout(fn):
    q, k, v = _contiguous(2, 3, 24, 4, 1)
    kp, bt = _to_pages(k, 8)
    vp, _ = _to_pages(v, 8)
    o, lse = fn(q, kp, vp, bt, np.array([24, 24]), 0.6)
    o2, lse2 = decode_ref(q, k, v, 0.6)
    assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - lse2).max() <= 1e-12


def pin_page_permutation(fn):
    q, k, v = _contiguous(2, 2, 32, 4, 2)
    kp, bt = _to_pages(k, 4)
    vp, _ = _to_pages(v, 4)
    perm = np.random.default_rng(3).permutation(kp.shape[0])
    inv = np.argsort(perm)
    o, lse = fn(q, kp, vp, bt, np.array([32, 29]), 0.5)
    o2, lse2 = fn(q, kp[perm], vp[perm], inv[bt], np.array([32, 29]), 0.5)
    assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - lse2).max() <= 1e-12


def pin_prefix_length(fn):
    q, k, v = _contiguous(1, 2, 40, 5, 4)
    kp, bt = _to_pages(k, 8)
    vp, _ = _to_pages(v, 8)
    for n in (1, 7, 8, 9, 33):
        o, lse = fn(q, kp, vp, bt, np.array([n]), 0.4)
        o2, lse2 = decode_ref(q, k[:, :, :n], v[:, :, :n], 0.4)
        assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - lse2).max() <= 1e-12, n


def pin_absent_pages(fn):
    q, k, v = _contiguous(1, 2, 32, 4, 5)
    kp, bt = _to_pages(k, 8)
    vp, _ = _to_pages(v, 8)
    bt = bt.copy()
    bt[0, 1] = -1               # tokens 8..15 absent
    bt[0, 3] = kp.shape[0]      # tokens 24..31 absent
    o, lse = fn(q, kp, vp, bt, np.array([32]), 0.7)
    keep = np.r_[0:8, 16:24]
    o2, lse2 = decode_ref(q, k[:, :, keep], v[:, :, keep], 0.7)
    assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - lse2).max() <= 1e-12


def pin_grouped_heads(fn):
    rng = np.random.default_rng(6)
    q = rng.standard_normal((2, 8, 4))
    k, v = rng.standard_normal((2, 2, 16, 4)), rng.standard_normal((2, 2, 16, 4))
    kp, bt = _to_pages(k, 4)
    vp, _ = _to_pages(v, 4)
    o, lse = fn(q, kp, vp, bt, np.array([16, 11]), 0.5)
    for b, n in ((0, 16), (1, 11)):
        o2, lse2 = gqa_decode_ref(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.5)
        assert np.abs(o[b] - o2[0]).max() <= 1e-12 and np.abs(lse[b] - lse2[0]).max() <= 1e-12


def pin_length_clamp(fn):
    q, k, v = _contiguous(2, 2, 16, 4, 7)
    kp, bt = _to_pages(k, 4)
    vp, _ = _to_pages(v, 4)
    o, lse = fn(q, kp, vp, bt, np.array([1000, -3]), 0.5)
    o2, lse2 = decode_ref(q[:1], k[:1], v[:1], 0.5)
    assert np.abs(o[0] - o2[0]).max() <= 1e-12 and np.abs(lse[0] - lse2[0]).max() <= 1e-12
    assert np.all(o[1] == 0) and np.all(lse[1] == -np.inf)


PINS = [pin_in_order_layout, pin_page_permutation, pin_prefix_length, pin_absent_pages, pin_grouped_heads,
        pin_length_clamp]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(paged_decode_ref)


def _mutant(change):
    def fn(q, kp, vp, bt, sl, scale):
        q = np.asarray(q, np.float64)
        B, H, d = q.shape
        n_pages, _, P, _ = kp.shape
        O, L = np.zeros((B, H, vp.shape[3])), np.full((B, H), -np.inf)
        for b in range(B):
            n = bt.shape[1] * P if change == "length_ignored" else min(max(int(sl[b]), 0), bt.shape[1] * P)
            toks = [t for t in range(n) if 0 <= bt[b, t // P] < n_pages]
            if not toks:
                continue
            pg = (lambda t: min(bt[b, t // P] + 1, n_pages - 1)) if change == "page_off_by_one" else \
                 (lambda t: bt[b, t // P])
            row = (lambda t: (t + 1) % P) if change == "row_shifted" else (lambda t: t % P)
            kb = np.stack([kp[pg(t), :, row(t), :] for t in toks], axis=1)
            vb = np.stack([vp[pg(t), :, row(t), :] for t in toks], axis=1)
            o, lse = gqa_decode_ref(q[b][None], kb[None], vb[None], scale)
            O[b], L[b] = o[0], lse[0]
        return O, L
    return fn


@pytest.mark.parametrize("change", ["page_off_by_one", "row_shifted", "length_ignored"])
def test_mutant_is_caught(change):
    caught = 0
    for pin in PINS:
        try:
            pin(_mutant(change))
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught, change
