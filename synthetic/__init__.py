"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage type.  It
holds none of the attention arithmetic, so the CPU oracle and the GPU path can
both consume its output without sharing any of the method's code.

Recipe (one independent stream per tensor slice):
  * every (tensor, b, h) slice of shape [N, d] gets its own PCG64 generator,
    seeded with ``SeedSequence([seed, tensor_id, b, h])`` (tensor_id: q=0, k=1,
    v=2, and do=3 for the upstream gradient of the backward pass, N(0,1));
  * the slice is drawn as float32 in C order: ``standard_normal`` for N(0,1),
    ``2*random()-1`` for U(-1,1), and ``4*standard_normal`` for the scaled
    queries of the peaked-softmax workload (scaling by a power of two is exact);
    stress inputs for the tests use ``16*standard_normal`` ("normal16"),
    ``0.5 + 0.1*standard_normal`` ("pos") and ``0.02*j + 0.1*standard_normal``
    for row j ("ramp": scores that rise along the keys);
  * bf16 workloads round the float32 draws to bfloat16 with
    round-to-nearest-even (bit manipulation, no library conversion).

Because every slice is independent, a full-size workload can be generated in
parallel, and a test can regenerate only the (b, h) slices it samples.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3}  # "do": upstream gradient of O (backward pass)


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, storage dtype, mask, scale, seed, value distributions."""

    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    dtype: str  # "f32" or "bf16"
    causal: bool
    scale: float
    seed: int
    dist: dict = field(default_factory=lambda: {"q": "normal", "k": "normal", "v": "normal"})
    kind: str = "prefill"  # "prefill" (fa_fwd) or "decode" (fa_decode)
    num_splits: int = 0

    def shape(self, t: str):
        n = self.Nq if t in ("q", "do") else self.Nkv
        return (self.B, self.H, n, self.d)

    @property
    def allowed_pairs(self) -> int:
        """Number of (query, key) pairs the mask allows, per the bottom-right causal rule."""
        if not self.causal:
            return self.B * self.H * self.Nq * self.Nkv
        return self.B * self.H * _causal_pairs_closed(self.Nq, self.Nkv)

    @property
    def flops(self) -> int:
        """Algorithmic flops: 2*d for the score plus 2*d for the value sum, per allowed pair."""
        return 4 * self.d * self.allowed_pairs

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once; O written once; LSE (fp32) written once."""
        e = self.elem_bytes
        q = self.B * self.H * self.Nq * self.d * e
        kv = 2 * self.B * self.H * self.Nkv * self.d * e
        o = self.B * self.H * self.Nq * self.d * e
        lse = self.B * self.H * self.Nq * 4
        return q + kv + o + lse


def _causal_pairs_closed(nq: int, nkv: int) -> int:
    """Allowed pairs under the bottom-right rule (key j allowed for query i iff j <= i + nkv - nq)."""
    off = nkv - nq
    return sum(max(0, min(nkv, i + off + 1)) for i in range(nq)) if off < 0 else \
        nq * (off + 1) + nq * (nq - 1) // 2


WORKLOADS = {
    "c1": Workload("noncausal_f32_B1_H1_N256_d64", 1, 1, 256, 256, 64, "f32", False, 1 / math.sqrt(64), 0),
    "c2": Workload("causal_bf16_B4_H16_N2048_d64_q4x", 4, 16, 2048, 2048, 64, "bf16", True, 1 / math.sqrt(64), 1,
                   {"q": "normal4", "k": "normal", "v": "normal"}),
    "c3": Workload("causal_bf16_B1_H32_N8192_d128", 1, 32, 8192, 8192, 128, "bf16", True, 1 / math.sqrt(128), 2),
    "c4": Workload("causal_bf16_B1_H8_N32768_d128", 1, 8, 32768, 32768, 128, "bf16", True, 1 / math.sqrt(128), 3,
                   {"q": "normal", "k": "normal", "v": "uniform"}),
    "c5": Workload("decode_bf16_B64_H32_Nkv8192_d128_S16", 64, 32, 1, 8192, 128, "bf16", False, 1 / math.sqrt(128), 4,
                   kind="decode", num_splits=16),
}

# Workloads beyond the five listed configurations: a chunk of 1000 new queries (not a multiple of any tile height)
# appended to an 8192-key cache, bottom-right causal ("prefill against a cache").
NEXT_WORKLOADS = {
    "chunk": Workload("chunked_causal_bf16_B1_H32_Nq1000_Nkv8192_d128", 1, 32, 1000, 8192, 128, "bf16", True,
                      1 / math.sqrt(128), 5),
}


def draw_f32(seed: int, tensor: str, b: int, h: int, n: int, d: int, dist: str) -> np.ndarray:
    """Draw one [n, d] float32 slice from its own seeded stream."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TENSOR_ID[tensor], b, h])))
    if dist == "normal":
        return rng.standard_normal((n, d), dtype=np.float32)
    if dist == "normal4":
        return rng.standard_normal((n, d), dtype=np.float32) * np.float32(4.0)
    if dist == "uniform":
        return rng.random((n, d), dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    if dist == "normal16":  # very peaked rows
        return rng.standard_normal((n, d), dtype=np.float32) * np.float32(16.0)
    if dist == "pos":       # positive queries: 0.5 + 0.1 N(0,1)
        return rng.standard_normal((n, d), dtype=np.float32) * np.float32(0.1) + np.float32(0.5)
    if dist == "ramp":      # rows that grow along the sequence: 0.02 j + 0.1 N(0,1), so later keys score higher
        ramp = (np.arange(n, dtype=np.float32) * np.float32(0.02))[:, None]
        return rng.standard_normal((n, d), dtype=np.float32) * np.float32(0.1) + ramp
    raise ValueError(f"unknown distribution {dist!r}")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the 16-bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16 or int16) to float32 exactly."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_tensor(w: Workload, t: str, bh=None, workers: int | None = None) -> np.ndarray:
    """Generate tensor ``t`` of workload ``w`` in its storage type.

    Returns float32 [B,H,N,d] for f32 workloads and uint16 bf16 bit patterns for bf16
    workloads.  With ``bh`` (a list of (b, h)), returns only those slices, stacked as
    [len(bh), N, d].
    """
    B, H, n, d = w.shape(t)
    dist = w.dist.get(t, "normal")
    pairs = [(b, h) for b in range(B) for h in range(H)] if bh is None else list(bh)
    out_dtype = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty((len(pairs), n, d), dtype=out_dtype)

    def one(i):
        b, h = pairs[i]
        x = draw_f32(w.seed, t, b, h, n, d, dist)
        out[i] = x if w.dtype == "f32" else bf16_bits(x)

    nw = workers or _workers()
    if nw == 1 or len(pairs) == 1:
        for i in range(len(pairs)):
            one(i)
    else:
        with ThreadPoolExecutor(nw) as ex:
            list(ex.map(one, range(len(pairs))))
    if bh is None:
        return out.reshape(B, H, n, d)
    return out


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values (float32 or bf16 bit patterns)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    return bf16_to_f32(x).astype(np.float64)


def custom(B, H, Nq, Nkv, d, dtype="bf16", causal=False, scale=None, seed=0, dist=None, kind="prefill",
           num_splits=0) -> Workload:
    """An ad-hoc workload (edge shapes for tests) with the same generation recipe."""
    return Workload(f"custom_B{B}_H{H}_Nq{Nq}_Nkv{Nkv}_d{d}_{dtype}", B, H, Nq, Nkv, d, dtype, causal,
                    (1 / math.sqrt(d)) if scale is None else float(scale), seed,
                    dist or {"q": "normal", "k": "normal", "v": "normal"}, kind, num_splits)


# ----------------------------------------------------------------------------- paged KV cache layout

def page_table(B: int, n_blocks: int, num_pages: int, seed: int) -> np.ndarray:
    """Block table int32 [B, n_blocks]: logical block j of sequence b gets physical page perm[b * n_blocks + j],
    where perm is a seeded permutation of range(num_pages) (num_pages >= B * n_blocks)."""
    if num_pages < B * n_blocks:
        raise ValueError("the pool needs at least B * n_blocks pages")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 100])))
    perm = rng.permutation(num_pages).astype(np.int32)
    return perm[: B * n_blocks].reshape(B, n_blocks).copy()


def paginate(x: np.ndarray, table: np.ndarray, num_pages: int, page_size: int, seed: int) -> np.ndarray:
    """Scatter a contiguous cache x [B, H_kv, n_blocks * page_size, d] into a page pool
    [num_pages, H_kv, page_size, d] as ``table`` says (token t of sequence b -> page table[b, t // page_size],
    row t % page_size).  Pool pages that no entry names hold N(0,1)*8 filler from their own seeded stream, in
    x's storage type, so that reading a wrong page shows."""
    B, Hkv, N, d = x.shape
    nb = N // page_size
    if nb * page_size != N or table.shape != (B, nb):
        raise ValueError("x must hold n_blocks whole pages per sequence, matching the table")
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 101])))
    fill = rng.standard_normal((num_pages, Hkv, page_size, d), dtype=np.float32) * np.float32(8.0)
    pool = fill if x.dtype == np.float32 else bf16_bits(fill)
    blocks = x.reshape(B, Hkv, nb, page_size, d).transpose(0, 2, 1, 3, 4)  # [B, nb, Hkv, P, d]
    pool[table.reshape(-1)] = blocks.reshape(B * nb, Hkv, page_size, d)
    return pool
