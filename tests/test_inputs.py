"""The seeded input generator: determinism, slice independence, bf16 rounding, workload arithmetic."""
import numpy as np
import pytest

import synthetic as syn


def test_deterministic_and_slice_addressable():
    w = syn.custom(2, 3, 5, 7, 64, "bf16", seed=11)
    a = syn.make_tensor(w, "k")
    b = syn.make_tensor(w, "k", workers=1)
    assert a.dtype == np.uint16 and a.shape == (2, 3, 7, 64)
    np.testing.assert_array_equal(a, b)
    part = syn.make_tensor(w, "k", bh=[(1, 2), (0, 1)])
    np.testing.assert_array_equal(part[0], a[1, 2])
    np.testing.assert_array_equal(part[1], a[0, 1])
    # different tensors / heads / seeds give different streams
    assert not np.array_equal(syn.make_tensor(w, "v"), a)
    assert not np.array_equal(a[0, 0], a[0, 1])
    w2 = syn.custom(2, 3, 5, 7, 64, "bf16", seed=12)
    assert not np.array_equal(syn.make_tensor(w2, "k"), a)


def test_distributions():
    w = syn.WORKLOADS["c4"]
    v = syn.draw_f32(w.seed, "v", 0, 0, 4096, 128, "uniform")
    assert v.min() >= -1 and v.max() < 1 and abs(v.mean()) < 0.01
    q4 = syn.draw_f32(1, "q", 0, 0, 2048, 64, "normal4")
    q1 = syn.draw_f32(1, "q", 0, 0, 2048, 64, "normal")
    np.testing.assert_array_equal(q4, q1 * 4)
    assert abs(q1.std() - 1) < 0.01


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40, np.inf, -np.inf], np.float32)])
    # exact ties: the low 16 bits are 0x8000, both for even and odd kept mantissas
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x3F800000 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = syn.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = syn.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_arithmetic():
    w = syn.WORKLOADS
    assert w["c1"].flops == 16_777_216 and w["c1"].io_bytes == 263_168
    assert w["c2"].flops == 34_376_515_584 and w["c2"].io_bytes == 67_633_152
    assert w["c3"].flops == 549_822_922_752 and w["c3"].io_bytes == 269_484_032
    assert w["c4"].flops == 2_199_090_364_416
    assert w["c5"].io_bytes == 8_590_991_360
    # bottom-right causal pairs equal a brute-force count
    for nq, nkv in ((3, 3), (3, 8), (1, 5), (9, 9)):
        ws = syn.custom(1, 1, nq, nkv, 64, causal=True)
        brute = sum(1 for i in range(nq) for j in range(nkv) if j <= i + nkv - nq)
        assert ws.allowed_pairs == brute


def test_page_table_and_paginate():
    """The paged layout helpers: a seeded permutation of distinct pages, and a scatter that the gather
    through the same table undoes exactly, with unnamed pages holding filler."""
    t = syn.page_table(3, 5, 20, seed=7)
    assert t.shape == (3, 5) and t.dtype == np.int32
    assert len(set(t.reshape(-1).tolist())) == 15 and t.min() >= 0 and t.max() < 20
    assert np.array_equal(t, syn.page_table(3, 5, 20, seed=7))
    x = syn.bf16_bits(np.random.default_rng(1).standard_normal((3, 2, 5 * 4, 8)).astype(np.float32))
    pool = syn.paginate(x, t, 20, 4, seed=7)
    assert pool.shape == (20, 2, 4, 8) and pool.dtype == x.dtype
    for b in range(3):
        for tok in range(20):
            assert np.array_equal(pool[t[b, tok // 4], :, tok % 4, :], x[b, :, tok, :])
    unnamed = sorted(set(range(20)) - set(t.reshape(-1).tolist()))
    assert len(unnamed) == 5 and all(np.any(pool[u] != 0) for u in unnamed)
    with pytest.raises(ValueError):
        syn.page_table(3, 5, 14, seed=7)  # a pool smaller than the blocks it must hold
