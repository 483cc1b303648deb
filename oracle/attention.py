"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the test suite, the package's smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

What it computes (the plain definition, written out):

  * Attention(Q, K, V) = softmax(scale * Q K^T) V with scale = 1/sqrt(d_k) by
    default -- "FlashAttention Explained: How AI Models Process Attention Faster
    and Use Less Memory", section "Understanding Attention in Transformer
    Models" (the scaled dot-product attention equation).
  * It proceeds the conventional way the same page describes in "Why
    Traditional Attention Can Be Inefficient": the score matrix S = Q K^T is
    materialised, scaled and normalised row by row into P, then O = P V.  The
    number of score elements it materialises is counted so that the page's
    table of N x N element counts can pin it.
  * Masking keeps the "allowed positions" of "How FlashAttention Speeds Up LLM
    Attention" (introduction).  The causal rule is bottom-right aligned: key j
    is allowed for query i iff j <= i + (N_kv - N_q).  Masked scores are -inf
    before the exponential, i.e. exactly zero weight.
  * The per-row log-sum-exp LSE_i = ln sum_{allowed j} exp(scale * q_i . k_j)
    is returned with the output (natural log, scale included).

Large inputs are processed in panels of complete rows: every row is still the
full-row softmax; no online merge is involved.

The backward pass (``attention_bwd_ref``) is the plain derivative of that same
function for an upstream gradient dO, written out on materialised matrices
(training needs these gradients -- "FlashAttention Explained: How AI Models
Process Attention Faster and Use Less Memory", section "FlashAttention in AI
Training", "More Efficient Backpropagation"; the method recomputes the
probabilities instead of storing them, "How FlashAttention Speeds Up LLM
Attention", table of contents).  With P the row softmax of S = scale*Q K^T:
dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(P * dP)), dQ = scale*dS K,
dK = scale*dS^T Q.

Two further functions model the method itself and are used only to pin the
merge rules against the plain definition (they are never what the GPU result is
compared with):

  * ``tiled_model`` walks the keys in tiles with a running row maximum, a
    running denominator and a rescaled partial output -- "Flash Attention
    Explained: Same Maths, Far Less Memory", section "The idea: never
    materialise the matrix", and "How FlashAttention Works", part "3. Online
    Softmax", of the first page named above.
  * ``split_partials_ref`` / ``combine_ref`` split the keys into contiguous
    ranges, take the plain definition on each range, and merge the (O_s, LSE_s)
    pairs by their log-sum-exp weights (the decode case of "Where you actually
    feel it": one query against the cached keys and values).
"""
from __future__ import annotations


import numpy as np

__all__ = [
    "attention_ref",
    "probabilities_ref",
    "allowed_mask",
    "tiled_model",
    "merge_partials",
    "split_bounds",
    "split_partials_ref",
    "combine_ref",
    "decode_ref",
    "attention_bwd_ref",
    "gqa_decode_ref",
    "paged_decode_ref",
]


def _as4(x) -> np.ndarray:
    a = np.asarray(x, dtype=np.float64)
    if a.ndim != 4:
        raise ValueError(f"expected [B,H,N,d], got shape {a.shape}")
    return a


def allowed_mask(n_q: int, n_kv: int, causal: bool, rows=None, n_cols=None) -> np.ndarray:
    """Boolean [len(rows), n_cols] mask: True where key j may be attended by query i.

    Causal uses the bottom-right alignment j <= i + (n_kv - n_q); with n_q == n_kv
    this is the lower triangle, and with n_q == 1 every cached key is allowed.
    """
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    n_cols = n_kv if n_cols is None else n_cols
    cols = np.arange(n_cols)
    if not causal:
        return np.broadcast_to(cols[None, :] < n_kv, (rows.size, n_cols)).copy()
    off = n_kv - n_q
    return (cols[None, :] <= rows[:, None] + off) & (cols[None, :] < n_kv)


def _softmax_panel(S: np.ndarray, allowed: np.ndarray):
    """Row softmax of one materialised panel of scores (already scaled)."""
    S = np.where(allowed, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("a query row has no allowed key")
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    lse = (m + np.log(l))[:, 0]
    return P, lse


def attention_ref(q, k, v, scale: float, causal: bool, rows=None, panel_rows: int = 512,
                  return_count: bool = False):
    """Exact attention in fp64, materialising the score matrix panel by panel.

    q: [B,H,N_q,d]; k: [B,H,N_kv,d]; v: [B,H,N_kv,d_v] (any real dtype; upcast exactly).
    rows: optional query indices (same for every (b, h)); only those rows are computed.
    Returns (O [B,H,R,d_v], LSE [B,H,R]) in float64, plus the number of score
    elements materialised when ``return_count``.
    """
    q, k, v = _as4(q), _as4(k), _as4(v)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if k.shape[:2] != (B, H) or v.shape[:3] != (B, H, n_kv) or k.shape[3] != d:
        raise ValueError("shape mismatch between q, k, v")
    rows = np.arange(n_q) if rows is None else np.asarray(rows, dtype=np.int64)
    off = n_kv - n_q
    O = np.empty((B, H, rows.size, v.shape[3]), dtype=np.float64)
    LSE = np.empty((B, H, rows.size), dtype=np.float64)
    count = 0
    for b in range(B):
        for h in range(H):
            for p0 in range(0, rows.size, panel_rows):
                r = rows[p0:p0 + panel_rows]
                # keys beyond the last allowed one of this panel carry zero weight; a
                # causal panel only needs the prefix [0, max(r) + off] of the keys
                kmax = n_kv if not causal else int(min(n_kv, r.max() + off + 1))
                S = scale * (q[b, h, r, :] @ k[b, h, :kmax, :].T)
                count += S.size
                P, lse = _softmax_panel(S, allowed_mask(n_q, n_kv, causal, r, kmax))
                O[b, h, p0:p0 + r.size] = P @ v[b, h, :kmax, :]
                LSE[b, h, p0:p0 + r.size] = lse
    if return_count:
        return O, LSE, count
    return O, LSE


def probabilities_ref(q, k, scale: float, causal: bool) -> np.ndarray:
    """The full probability matrix P [B,H,N_q,N_kv] (small inputs only)."""
    q, k = _as4(q), _as4(k)
    B, H, n_q, _ = q.shape
    n_kv = k.shape[2]
    P = np.empty((B, H, n_q, n_kv))
    mask = allowed_mask(n_q, n_kv, causal)
    for b in range(B):
        for h in range(H):
            P[b, h], _ = _softmax_panel(scale * (q[b, h] @ k[b, h].T), mask)
    return P


def tiled_model(q, k, v, scale: float, causal: bool, tile: int):
    """The online-softmax recurrence over key tiles of width ``tile`` (a model of the method).

    State per query row: running max m (starts at -inf), running denominator l
    (starts at 0) and unnormalised output O (starts at 0).  For each key tile:
      m_new = max(m, rowmax S_tile);  alpha = exp(m - m_new)  (0 while m = -inf)
      P~ = exp(S_tile - m_new);  l = alpha*l + rowsum P~;  O = alpha*O + P~ V_tile
    and at the end O / l and LSE = m + ln l.
    """
    q, k, v = _as4(q), _as4(k), _as4(v)
    B, H, n_q, _ = q.shape
    n_kv = k.shape[2]
    O = np.empty((B, H, n_q, v.shape[3]))
    LSE = np.empty((B, H, n_q))
    for b in range(B):
        for h in range(H):
            m = np.full(n_q, -np.inf)
            l = np.zeros(n_q)
            acc = np.zeros((n_q, v.shape[3]))
            for j0 in range(0, n_kv, tile):
                j1 = min(n_kv, j0 + tile)
                S = scale * (q[b, h] @ k[b, h, j0:j1].T)
                allowed = allowed_mask(n_q, n_kv, causal)[:, j0:j1]
                S = np.where(allowed, S, -np.inf)
                m_new = np.maximum(m, S.max(axis=1))
                alpha = np.where(np.isneginf(m), 0.0, np.exp(m - np.where(np.isneginf(m_new), 0.0, m_new)))
                Pt = np.where(allowed, np.exp(S - np.where(np.isneginf(m_new), 0.0, m_new)[:, None]), 0.0)
                l = alpha * l + Pt.sum(axis=1)
                acc = alpha[:, None] * acc + Pt @ v[b, h, j0:j1]
                m = m_new
            O[b, h] = acc / l[:, None]
            LSE[b, h] = m + np.log(l)
    return O, LSE


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Merge two normalised partial results over disjoint key sets by their LSE weights."""
    o_a, o_b = np.asarray(o_a, np.float64), np.asarray(o_b, np.float64)
    lse_a, lse_b = np.asarray(lse_a, np.float64), np.asarray(lse_b, np.float64)
    M = np.maximum(lse_a, lse_b)
    Ms = np.where(np.isneginf(M), 0.0, M)
    wa = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - Ms))
    wb = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - Ms))
    w = wa + wb
    o = (wa[..., None] * o_a + wb[..., None] * o_b) / w[..., None]
    return o, M + np.log(w)


def split_bounds(n_kv: int, num_splits: int):
    """Contiguous key ranges: split s covers [s*c, min((s+1)*c, n_kv)) with c = ceil(n_kv / S)."""
    c = -(-n_kv // num_splits)
    return [(min(s * c, n_kv), min((s + 1) * c, n_kv)) for s in range(num_splits)]


def split_partials_ref(q, k, v, scale: float, num_splits: int):
    """Per-split normalised outputs and LSEs for one query per sequence.

    q: [B,H,1,d] (or [B,H,d]); k, v: [B,H,N_kv,d].  Returns O_s [B,H,S,d_v] and
    LSE_s [B,H,S]; an empty split has O_s = 0 and LSE_s = -inf (zero weight).
    """
    q = np.asarray(q, np.float64)
    if q.ndim == 3:
        q = q[:, :, None, :]
    k, v = _as4(k), _as4(v)
    B, H, n_kv, _ = k.shape
    Os = np.zeros((B, H, num_splits, v.shape[3]))
    Ls = np.full((B, H, num_splits), -np.inf)
    for s, (a, e) in enumerate(split_bounds(n_kv, num_splits)):
        if e > a:
            o, lse = attention_ref(q, k[:, :, a:e], v[:, :, a:e], scale, False)
            Os[:, :, s] = o[:, :, 0]
            Ls[:, :, s] = lse[:, :, 0]
    return Os, Ls


def combine_ref(o_parts, lse_parts):
    """Combine S partial results: M = max_s LSE_s, w_s = exp(LSE_s - M), O = sum w_s O_s / sum w_s."""
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    M = lse_parts.max(axis=-1)
    w = np.where(np.isneginf(lse_parts), 0.0, np.exp(lse_parts - M[..., None]))
    sw = w.sum(axis=-1)
    O = (w[..., None] * o_parts).sum(axis=-2) / sw[..., None]
    return O, M + np.log(sw)


def decode_ref(q, k, v, scale: float):
    """One query per sequence against all cached keys (no mask): O [B,H,d_v], LSE [B,H]."""
    q = np.asarray(q, np.float64)
    if q.ndim == 3:
        q = q[:, :, None, :]
    o, lse = attention_ref(q, k, v, scale, False)
    return o[:, :, 0], lse[:, :, 0]


def gqa_decode_ref(q, k, v, scale: float):
    """Decode with grouped key/value heads: q [B,H,d]; k, v [B,H_kv,N_kv,d], H a multiple of H_kv.

    Query head h attends to key/value head h // (H / H_kv) (consecutive query heads share one key/value
    head).  Written as the plain definition on explicitly repeated keys and values.
    """
    q = np.asarray(q, np.float64)
    k, v = _as4(k), _as4(v)
    H, H_kv = q.shape[1], k.shape[1]
    if H % H_kv:
        raise ValueError("H must be a multiple of H_kv")
    g = H // H_kv
    return decode_ref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), scale)


def paged_decode_ref(q, k_pages, v_pages, block_table, seq_lens, scale: float):
    """Decode against a paged KV cache (the paging idea of "Paged Attention: Fixing the KV Cache Memory
    Problem", listed among the related posts of "Flash Attention Explained: Speed From Memory Movement").

    k_pages, v_pages: [num_pages, H_kv, P, d]; token t of sequence b lives in page block_table[b, t // P],
    row t % P.  Sequence b has seq_lens[b] tokens, taken as min(max(seq_lens[b], 0), max_blocks * P) so
    that the table is never read past its width.  A table entry outside [0, num_pages) marks its tokens
    absent (they take no part).  q [B, H, d] with H a multiple of H_kv; query head h reads key/value head
    h // (H / H_kv).  Returns (O [B, H, d], LSE [B, H]); a sequence with no token gives O = 0 and
    LSE = -inf.  Written out: gather each sequence's tokens, then the grouped-head decode definition.
    """
    q = np.asarray(q, np.float64)
    kp, vp = np.asarray(k_pages, np.float64), np.asarray(v_pages, np.float64)
    bt, sl = np.asarray(block_table), np.asarray(seq_lens)
    B, H, d = q.shape
    n_pages, _, P, _ = kp.shape
    O = np.zeros((B, H, vp.shape[3]))
    L = np.full((B, H), -np.inf)
    for b in range(B):
        n = min(max(int(sl[b]), 0), bt.shape[1] * P)
        toks = [t for t in range(n) if 0 <= bt[b, t // P] < n_pages]
        if not toks:
            continue
        kb = np.stack([kp[bt[b, t // P], :, t % P, :] for t in toks], axis=1)  # [H_kv, n, d]
        vb = np.stack([vp[bt[b, t // P], :, t % P, :] for t in toks], axis=1)
        o, lse = gqa_decode_ref(q[b][None], kb[None], vb[None], scale)
        O[b], L[b] = o[0], lse[0]
    return O, L


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool):
    """Gradients (dQ, dK, dV) of O = softmax(scale Q K^T) V for the upstream gradient dO, fp64.

    q, do: [B,H,N_q,d]; k, v: [B,H,N_kv,d].  Each (b, h) materialises S, P, dP and dS in full
    (small and medium inputs only).  Masked positions have P = 0, so they carry no gradient.
    """
    q, k, v, do = _as4(q), _as4(k), _as4(v), _as4(do)
    B, H, n_q, d = q.shape
    n_kv = k.shape[2]
    if k.shape[:2] != (B, H) or v.shape[:3] != (B, H, n_kv) or do.shape != (B, H, n_q, v.shape[3]):
        raise ValueError("shape mismatch between q, k, v, do")
    mask = allowed_mask(n_q, n_kv, causal)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            P, _ = _softmax_panel(scale * (q[b, h] @ k[b, h].T), mask)
            dv[b, h] = P.T @ do[b, h]
            dP = do[b, h] @ v[b, h].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ k[b, h])
            dk[b, h] = scale * (dS.T @ q[b, h])
    return dq, dk, dv

