"""Planted mistakes in the oracle must each be caught by at least one pin.

Every mutant changes one thing in the CPU oracle (on the CPU, nothing else) -- a
dropped or flipped scale, a shifted or mirrored mask, a wrong normalisation
axis, a lost max term in the LSE, reordered values -- and the pin suite of
test_oracle.py is run against it.  A mutant that passes every pin means the pins
are too weak.
"""
import numpy as np
import pytest

import oracle.attention as oa
from tests.test_oracle import PINS


def _mask_variant(rule):
    def allowed_mask(n_q, n_kv, causal, rows=None, n_cols=None):
        rows = np.arange(n_q) if rows is None else np.asarray(rows)
        n_cols = n_kv if n_cols is None else n_cols
        cols = np.arange(n_cols)
        if not causal:
            return np.broadcast_to(cols[None, :] < n_kv, (rows.size, n_cols)).copy()
        return rule(rows[:, None], cols[None, :], n_kv - n_q) & (cols[None, :] < n_kv)
    return allowed_mask


def _softmax_variant(kind):
    def softmax_panel(S, allowed):
        S = np.where(allowed, S, -np.inf)
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        if kind == "uniform":
            E = allowed.astype(np.float64)
        l = E.sum(axis=1, keepdims=True)
        if kind == "col_norm":
            P = E / np.maximum(E.sum(axis=0, keepdims=True), 1e-300)
        else:
            P = E / l
        lse = (m + np.log(l))[:, 0]
        if kind == "lse_no_max":
            lse = np.log(l)[:, 0]
        if kind == "lse_log2":
            lse = (m + np.log2(l))[:, 0]
        return P, lse
    return softmax_panel


MUTANTS = {
    "scale_dropped": dict(wrap=lambda f: (lambda q, k, v, s, c: f(q, k, v, 1.0, c))),
    "scale_negated": dict(wrap=lambda f: (lambda q, k, v, s, c: f(q, k, v, -s, c))),
    "scale_sqrt": dict(wrap=lambda f: (lambda q, k, v, s, c: f(q, k, v, np.sqrt(abs(s)), c))),
    "values_reversed": dict(wrap=lambda f: (lambda q, k, v, s, c: f(q, k, v[:, :, ::-1], s, c))),
    "query_rows_reversed": dict(wrap=lambda f: (lambda q, k, v, s, c: f(q[:, :, ::-1], k, v, s, c))),
    "diagonal_excluded": dict(mask=lambda i, j, off: j < i + off),
    "top_left_alignment": dict(mask=lambda i, j, off: j <= i),
    "upper_triangle": dict(mask=lambda i, j, off: j >= i + off),
    "off_by_one_extra_key": dict(mask=lambda i, j, off: j <= i + off + 1),
    "uniform_weights": dict(softmax="uniform"),
    "column_normalised": dict(softmax="col_norm"),
    "lse_without_max": dict(softmax="lse_no_max"),
    "lse_in_log2": dict(softmax="lse_log2"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    spec = MUTANTS[name]
    if "mask" in spec:
        monkeypatch.setattr(oa, "allowed_mask", _mask_variant(spec["mask"]))
    if "softmax" in spec:
        monkeypatch.setattr(oa, "_softmax_panel", _softmax_variant(spec["softmax"]))
    attn = oa.attention_ref
    if "wrap" in spec:
        attn = spec["wrap"](attn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
