"""O1: plain, unsplit softmax attention in fp64 (numpy only).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What is computed (the plain definition that context parallelism must reproduce
exactly; "Sequence Parallelism IV: Megatron Context Parallel and
Load-Balanced Rings", section 4 "What Actually Moves", states that the online
softmax state keeps the sharded result exact, and "Context Parallelism for
Long-Context Training", section "Prove attention equivalence", requires all
protected tensors to agree with the unsharded reference):

For every head ``h`` and query row ``i`` with global position ``pq[i]``:

* valid keys ``J(i) = {j : pk[j] <= pq[i]}`` when causal (a key in the query's
  future is masked; the diagonal is valid -- section 4 of the same page speaks
  of skipping sub-blocks that the causal mask makes future tokens), every key
  otherwise;
* ``s_ij = scale * <q_i, k_j>`` with ``scale = 1/sqrt(head_dim)`` by default;
* ``m_i = max_j s_ij``, ``w_ij = exp(s_ij - m_i)``, ``l_i = sum_j w_ij``;
* ``O_i = sum_j w_ij v_j / l_i`` and ``LSE_i = m_i + ln l_i`` (natural log).

A row with no valid key has ``LSE = -inf`` and ``O = 0``.

Rows are processed in blocks of at most ``block`` queries per head so memory
stays bounded; blocking splits only the query index, so every row's arithmetic
is unchanged.
"""

import math

import numpy as np


def _as_f64(x):
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def document_of(pos, doc_starts):
    """Index of the document holding each global position; documents are the
    runs ``[doc_starts[d], doc_starts[d + 1])`` (the first starts at 0)."""
    return np.searchsorted(np.asarray(doc_starts, dtype=np.int64), np.asarray(pos, dtype=np.int64), side="right") - 1


def valid_mask(q_pos, k_pos, causal, k_valid=None, doc_starts=None):
    """Boolean ``[len(q_pos), len(k_pos)]`` mask of valid (query, key) pairs.

    Causal: a key is valid when its global position is not after the query's.
    Bidirectional: every pair is valid.  ``k_valid`` (optional, per key) masks
    keys out entirely, as padded keys are.  ``doc_starts`` (optional; the
    document masks of "Context Parallelism for Long-Context Training",
    section "Prove attention equivalence") keeps only pairs whose query and
    key lie in the same document.
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        m = np.ones((q_pos.size, k_pos.size), dtype=bool)
    else:
        m = k_pos[None, :] <= q_pos[:, None]
    if k_valid is not None:
        m = m & np.asarray(k_valid, dtype=bool)[None, :]
    if doc_starts is not None:
        m = m & (document_of(q_pos, doc_starts)[:, None] == document_of(k_pos, doc_starts)[None, :])
    return m


def attention(q, k, v, *, causal, scale=None, q_pos=None, k_pos=None, k_valid=None, doc_starts=None, block=1024):
    """Unsplit softmax attention.

    q: ``[Sq, H, D]``; k, v: ``[Sk, H, D]`` (any real dtype; upcast to fp64).
    q_pos, k_pos: global token positions of the rows (default ``arange``).
    k_valid: optional per-key flags; False keys are masked out (padding).
    doc_starts: optional sorted document starts (first 0); pairs across
    documents are masked out.
    Returns ``(O [Sq, H, D] fp64, LSE [H, Sq] fp64)``.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    sq, heads, dim = q.shape
    sk = k.shape[0]
    if k.shape != (sk, heads, dim) or v.shape != (sk, heads, dim):
        raise ValueError("k and v must be [Sk, H, D] matching q")
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    q_pos = np.arange(sq, dtype=np.int64) if q_pos is None else np.asarray(q_pos, np.int64)
    k_pos = np.arange(sk, dtype=np.int64) if k_pos is None else np.asarray(k_pos, np.int64)

    out = np.zeros((sq, heads, dim), dtype=np.float64)
    lse = np.full((heads, sq), -np.inf, dtype=np.float64)
    if sq == 0 or sk == 0:
        return out, lse
    for h in range(heads):
        kh = k[:, h, :]
        vh = v[:, h, :]
        for i0 in range(0, sq, block):
            i1 = min(sq, i0 + block)
            s = scale * (q[i0:i1, h, :] @ kh.T)
            valid = valid_mask(q_pos[i0:i1], k_pos, causal, k_valid, doc_starts=doc_starts)
            s = np.where(valid, s, -np.inf)
            m = s.max(axis=1)
            has = np.isfinite(m)
            m_ref = np.where(has, m, 0.0)
            w = np.exp(s - m_ref[:, None])
            l = w.sum(axis=1)
            o = w @ vh
            o[has] /= l[has, None]
            o[~has] = 0.0
            out[i0:i1, h, :] = o
            lse[h, i0:i1] = np.where(has, m_ref + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def attention_probabilities(q, k, *, causal, scale=None, q_pos=None, k_pos=None):
    """Explicit probability matrix ``P [H, Sq, Sk]`` (small inputs only).

    ``P[h, i, j] = exp(s_ij - m_i) / l_i`` on valid pairs, 0 elsewhere.  Used to
    check that rows sum to one and that future keys get zero weight.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    sq, heads, dim = q.shape
    sk = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(dim)
    q_pos = np.arange(sq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(sk) if k_pos is None else np.asarray(k_pos)
    valid = valid_mask(q_pos, k_pos, causal)
    p = np.zeros((heads, sq, sk), dtype=np.float64)
    for h in range(heads):
        s = scale * (q[:, h, :] @ k[:, h, :].T)
        s = np.where(valid, s, -np.inf)
        m = s.max(axis=1)
        has = np.isfinite(m)
        w = np.exp(s - np.where(has, m, 0.0)[:, None])
        l = w.sum(axis=1)
        p[h][has] = w[has] / l[has, None]
    return p
