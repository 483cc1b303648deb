"""Pins for the grouped-key/value decode oracle (gqa_decode_ref), independent of how it is written.

* torch's own scaled_dot_product_attention with enable_gqa=True, fp64 on the CPU (a library routine);
* closed form: identical keys within each key/value head give O = mean of that head's values and
  LSE = scale q.k + ln N, so a query head mapped to the wrong key/value head shows up at once;
* H_kv == H reduces to the ungrouped decode oracle.
A planted grouping mistake (h % H_kv instead of h // (H / H_kv)) must fail a pin.
"""
import numpy as np
import pytest

from oracle import decode_ref, gqa_decode_ref


def _inputs(B, H, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, H, d)), rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d)))


def pin_torch_gqa(fn):
    torch = pytest.importorskip("torch")
    for B, H, Hkv, N, d in ((2, 8, 2, 9, 4), (1, 6, 1, 5, 8), (1, 4, 4, 7, 3)):
        q, k, v = _inputs(B, H, Hkv, N, d, 3 + H)
        o, lse = fn(q, k, v, 0.4)
        tq = torch.tensor(q)[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, torch.tensor(k), torch.tensor(v), scale=0.4,
                                                               enable_gqa=True)[:, :, 0]
        assert np.abs(o - ref.numpy()).max() <= 1e-12
        # LSE: logsumexp of the scores of the key/value head each query head uses
        g = H // Hkv
        s = 0.4 * np.einsum("bhd,bhnd->bhn", q, np.repeat(k, g, axis=1))
        assert np.abs(lse - np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) - s.max(-1)).max() <= 1e-12


def pin_identical_keys_per_group(fn):
    B, H, Hkv, N, d = 1, 6, 3, 5, 4
    rng = np.random.default_rng(11)
    q = rng.standard_normal((B, H, d))
    k = np.repeat(rng.standard_normal((B, Hkv, 1, d)), N, axis=2)
    v = rng.standard_normal((B, Hkv, N, d))
    o, lse = fn(q, k, v, 0.7)
    g = H // Hkv
    for h in range(H):
        kv = h // g
        assert np.abs(o[0, h] - v[0, kv].mean(axis=0)).max() <= 1e-12
        assert abs(lse[0, h] - (0.7 * q[0, h] @ k[0, kv, 0] + np.log(N))) <= 1e-12


def pin_ungrouped(fn):
    q, k, v = _inputs(2, 3, 3, 6, 5, 21)
    o, lse = fn(q, k, v, 0.3)
    o2, lse2 = decode_ref(q, k, v, 0.3)
    assert np.abs(o - o2).max() <= 1e-12 and np.abs(lse - lse2).max() <= 1e-12


PINS = [pin_torch_gqa, pin_identical_keys_per_group, pin_ungrouped]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(gqa_decode_ref)


def test_wrong_grouping_is_caught():
    def wrong(q, k, v, scale):
        H, Hkv = q.shape[1], k.shape[1]
        idx = [h % Hkv for h in range(H)]
        return decode_ref(q, k[:, idx], v[:, idx], scale)
    caught = 0
    for pin in PINS:
        try:
            pin(wrong)
        except AssertionError:
            caught += 1
    assert caught
