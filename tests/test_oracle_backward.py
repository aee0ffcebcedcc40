"""Pins of the fp64 backward oracle (``oracle/backward.py``) against facts that
do not come from it: central finite differences of the forward oracle, torch's
CPU autograd of scaled-dot-product attention in fp64, closed forms of the key
and value gradient sums, and the unsplit gradient for the ring decomposition.
Planted mistakes at the end check that the pins catch them.
"""

import importlib
import math

import numpy as np
import pytest
import torch

import oracle

backward_mod = importlib.import_module("oracle.backward")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _loss(q, k, v, dout, causal):
    o, _ = oracle.attention(q, k, v, causal=causal)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_central_differences(causal):
    """d(sum dO * O)/dx by central differences of the forward oracle, every element."""
    sq, heads, dim = 5, 2, 3
    q, k, v, dout = (_rand((sq, heads, dim), 90 + i) for i in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=causal)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = _loss(q, k, v, dout, causal)
            x[idx] = keep - eps
            down = _loss(q, k, v, dout, causal)
            x[idx] = keep
            num[idx] = (up - down) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-7


@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_torch_autograd_fp64(causal):
    sq, heads, dim = 37, 3, 16
    q, k, v, dout = (_rand((sq, heads, dim), 100 + i) for i in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=causal)
    tq, tk, tv = (torch.tensor(x).permute(1, 0, 2).contiguous().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    o.backward(torch.tensor(dout).permute(1, 0, 2))
    for got, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(got - t.grad.permute(1, 0, 2).numpy())) <= 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_key_and_value_gradient_sums(causal):
    """Rows of P sum to one, so sum_j dV_j = sum_i dO_i and sum_j dK_j = 0."""
    sq, heads, dim = 29, 2, 8
    q, k, v, dout = (_rand((sq, heads, dim), 110 + i) for i in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=causal)
    assert np.max(np.abs(dv.sum(axis=0) - dout.sum(axis=0))) <= 1e-12
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12


def test_single_key_row_has_no_query_gradient():
    """Causal row 0 sees one key with weight exactly 1: O_0 = v_0 whatever q_0 is."""
    sq, heads, dim = 6, 1, 4
    q, k, v, dout = (_rand((sq, heads, dim), 120 + i) for i in range(4))
    dq, _, _ = oracle.attention_backward(q, k, v, dout, causal=True)
    assert np.max(np.abs(dq[0])) == 0.0


@pytest.mark.parametrize("causal", [True, False])
def test_query_gradients_equal_rows_of_the_whole(causal):
    sq, heads, dim = 40, 2, 8
    q, k, v, dout = (_rand((sq, heads, dim), 125 + i) for i in range(4))
    dq, _, _ = oracle.attention_backward(q, k, v, dout, causal=causal)
    rows = [0, 7, 19, 39]
    got = oracle.query_gradients(q, k, v, dout, rows, causal=causal)
    assert np.max(np.abs(got - dq[rows])) <= 1e-13


CASES = [(64, 2, "zigzag", True), (96, 3, "zigzag", False), (64, 4, "contiguous", True),
         (80, 5, "contiguous", False), (101, 4, "zigzag", True), (13, 3, "contiguous", True),
         (21, 8, "zigzag", True)]


@pytest.mark.parametrize("seq,cp,layout,causal", CASES)
def test_ring_decomposition_equals_unsplit(seq, cp, layout, causal):
    heads, dim = 2, 8
    q, k, v, dout = (_rand((seq, heads, dim), 130 + i) for i in range(4))
    ref = oracle.attention_backward(q, k, v, dout, causal=causal)
    got = oracle.full_backward(q, k, v, dout, cp, layout=layout, causal=causal)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) <= 1e-12


def test_rank_share_touches_only_visible_sources():
    """Contiguous causal: rank r's keys of later sources get no gradient from it."""
    seq, cp, heads, dim = 64, 4, 1, 4
    q, k, v, dout = (_rand((seq, heads, dim), 140 + i) for i in range(4))
    _, dk, dv, pos = oracle.rank_backward(q, k, v, dout, cp, 1, layout="contiguous", causal=True)
    assert pos.tolist() == list(range(16, 32))
    assert np.all(dk[32:] == 0) and np.all(dv[32:] == 0)
    assert np.any(dk[:16] != 0) and np.any(dv[16:32] != 0)


# ----------------------------------------------------------------------------
# Document masks ("Context Parallelism for Long-Context Training", section
# "Prove attention equivalence": causal and document masks)
# ----------------------------------------------------------------------------

DOCS = [0, 1, 9, 10, 23]


@pytest.mark.parametrize("causal", [True, False])
def test_document_gradients_equal_each_document_alone(causal):
    """With document masks no pair crosses a boundary, so the gradients are
    those of every document run through the plain (maskless) backward alone."""
    seq, heads, dim = 31, 2, 4
    q, k, v, dout = (_rand((seq, heads, dim), 150 + i) for i in range(4))
    got = oracle.attention_backward(q, k, v, dout, causal=causal, doc_starts=DOCS)
    bounds = DOCS + [seq]
    for a, b in zip(bounds[:-1], bounds[1:]):
        ref = oracle.attention_backward(q[a:b], k[a:b], v[a:b], dout[a:b], causal=causal)
        for g, r in zip(got, ref):
            assert np.max(np.abs(g[a:b] - r)) <= 1e-13


def test_document_gradients_match_central_differences():
    seq, heads, dim = 7, 1, 2
    docs = [0, 3, 4]
    q, k, v, dout = (_rand((seq, heads, dim), 160 + i) for i in range(4))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, causal=True, doc_starts=docs)

    def loss():
        o, _ = oracle.attention(q, k, v, causal=True, doc_starts=docs)
        return float(np.sum(o * dout))
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + eps
            up = loss()
            x[idx] = keep - eps
            down = loss()
            x[idx] = keep
            num[idx] = (up - down) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-7


@pytest.mark.parametrize("seq,cp,layout,causal", [(64, 2, "zigzag", True), (101, 4, "zigzag", True),
                                                  (80, 5, "contiguous", False), (21, 8, "zigzag", True)])
def test_document_ring_decomposition_equals_unsplit(seq, cp, layout, causal):
    heads, dim = 2, 4
    docs = sorted({0, 1, 5, seq // 3, seq // 2 + 1, seq - 2})
    q, k, v, dout = (_rand((seq, heads, dim), 170 + i) for i in range(4))
    ref = oracle.attention_backward(q, k, v, dout, causal=causal, doc_starts=docs)
    got = oracle.full_backward(q, k, v, dout, cp, layout=layout, causal=causal, doc_starts=docs)
    for a, b in zip(got, ref):
        assert np.max(np.abs(a - b)) <= 1e-12
    rows = [0, 5, seq - 1]
    dq = oracle.query_gradients(q, k, v, dout, rows, causal=causal, doc_starts=docs)
    assert np.max(np.abs(dq - ref[0][rows])) <= 1e-13


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def test_planted_documents_ignored_in_the_pair_terms_are_caught(monkeypatch):
    real = backward_mod._pair_terms
    monkeypatch.setattr(backward_mod, "_pair_terms", lambda *a, **kw: real(*a))
    with pytest.raises(AssertionError):
        test_document_gradients_equal_each_document_alone(True)

def test_planted_missing_delta_term_is_caught(monkeypatch):
    real = backward_mod._pair_terms

    def no_delta(q, k, v, dout, o, lse, *rest, **kw):
        return real(q, k, v, dout, np.zeros_like(o), lse, *rest, **kw)
    monkeypatch.setattr(backward_mod, "_pair_terms", no_delta)
    with pytest.raises(AssertionError):
        test_gradients_match_central_differences(True)


def test_planted_unscaled_key_gradient_is_caught(monkeypatch):
    real = backward_mod._pair_terms

    def unscaled(*args, **kw):
        dq, dk, dv = real(*args, **kw)
        return dq, dk / args[9], dv
    monkeypatch.setattr(backward_mod, "_pair_terms", unscaled)
    with pytest.raises(AssertionError):
        test_gradients_match_torch_autograd_fp64(False)


def test_planted_swapped_sources_are_caught(monkeypatch):
    """Adding a step's key gradient to the wrong source breaks the decomposition."""
    real = backward_mod.ring_source
    monkeypatch.setattr(backward_mod, "ring_source", lambda r, s, cp: real(r, s, cp) if s != 1 else real(r, s + 1, cp))
    with pytest.raises(AssertionError):
        test_ring_decomposition_equals_unsplit(64, 4, "contiguous", True)
