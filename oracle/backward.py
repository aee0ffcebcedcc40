"""Backward of softmax attention in fp64, unsplit and decomposed by ring step.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

"Context Parallelism for Long-Context Training", section "Prove attention
equivalence", asks that the sharded run match the unsharded reference for
outputs *and* gradients, parameter by parameter.  The gradients here are the
plain chain rule of the forward definition in ``oracle/attention.py``, for a
loss whose gradient with respect to the output is ``dO``:

* ``P_ij = exp(s_ij - LSE_i)`` on valid pairs (0 elsewhere),
  ``s_ij = scale <q_i, k_j>``;
* ``dV_j = sum_i P_ij dO_i``;
* ``dP_ij = <dO_i, v_j>`` and ``D_i = sum_j P_ij dP_ij = <dO_i, O_i>``;
* ``dS_ij = P_ij (dP_ij - D_i)``;
* ``dQ_i = scale sum_j dS_ij k_j`` and ``dK_j = scale sum_i dS_ij q_i``.

Decomposed by ring step (the reading of the pages' ring for the backward:
queries stay, K/V pass by as in the forward, and the gradient of a K/V chunk
is summed over the ranks whose queries see it): at step ``s`` rank ``r``
holds source ``j = (r - s) mod cp`` and adds the terms of its valid pairs,
with ``P`` and ``D`` taken from the complete forward (its LSE and O), to its
own ``dQ`` and to the source's ``dK``, ``dV``.  The valid pairs of all steps
partition those of the whole sequence, so the sums equal the unsplit
gradients.

Document masks (the same section: "Test causal and document masks") enter
only through the valid pairs: ``doc_starts`` drops the pairs whose query and
key lie in different documents, in the forward that gives ``P`` and in the
pair terms alike.
"""

import numpy as np

from .attention import attention, valid_mask
from .cp_reference import ZIGZAG, rank_positions, ring_source


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _pair_terms(q, k, v, dout, o, lse, q_pos, k_pos, causal, scale, doc_starts=None):
    """dQ, dK, dV contributions of the valid pairs between rows ``q`` and keys ``k``."""
    sq, heads, dim = q.shape
    dq = np.zeros((sq, heads, dim))
    dk = np.zeros((k.shape[0], heads, dim))
    dv = np.zeros((k.shape[0], heads, dim))
    valid = valid_mask(q_pos, k_pos, causal, doc_starts=doc_starts)
    for h in range(heads):
        s = scale * (q[:, h] @ k[:, h].T)
        lse_h = np.where(np.isfinite(lse[h]), lse[h], 0.0)[:, None]  # -inf only for rows with no valid key
        p = np.where(valid, np.exp(np.where(valid, s, -np.inf) - lse_h), 0.0)
        dp = dout[:, h] @ v[:, h].T
        d_row = np.sum(dout[:, h] * o[:, h], axis=1)
        ds = p * (dp - d_row[:, None])
        dv[:, h] = p.T @ dout[:, h]
        dq[:, h] = scale * (ds @ k[:, h])
        dk[:, h] = scale * (ds.T @ q[:, h])
    return dq, dk, dv


def attention_backward(q, k, v, dout, *, causal, scale=None, doc_starts=None):
    """Unsplit gradients ``(dQ, dK, dV)`` of natural-order ``[S, H, D]`` inputs."""
    q, k, v, dout = (_f64(x) for x in (q, k, v, dout))
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[2])
    o, lse = attention(q, k, v, causal=causal, scale=scale, doc_starts=doc_starts)
    pos = np.arange(q.shape[0])
    return _pair_terms(q, k, v, dout, o, lse, pos, pos, causal, scale, doc_starts=doc_starts)


def query_gradients(q, k, v, dout, rows, *, causal, scale=None, doc_starts=None):
    """dQ of the natural-order rows ``rows`` only (all keys; cost linear in
    ``len(rows)``): the same terms as ``attention_backward`` for those rows."""
    q, k, v, dout = (_f64(x) for x in (q, k, v, dout))
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[2])
    rows = np.asarray(rows, dtype=np.int64)
    o, lse = attention(q[rows], k, v, causal=causal, scale=scale, q_pos=rows, doc_starts=doc_starts)
    dq, _, _ = _pair_terms(q[rows], k, v, dout[rows], o, lse, rows, np.arange(k.shape[0]), causal, scale,
                           doc_starts=doc_starts)
    return dq


def rank_backward(q, k, v, dout, cp, rank, *, layout=ZIGZAG, causal=True, scale=None, doc_starts=None):
    """One rank's share of the backward, one ring step at a time.

    Returns ``(dQ_loc [n, H, D], dK [S, H, D], dV [S, H, D], positions [n])``:
    the gradient of the rank's rows, and the rank's contributions to the key
    and value gradients of every source (what travels back around the ring).
    """
    q, k, v, dout = (_f64(x) for x in (q, k, v, dout))
    seq_len, heads, dim = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(dim)
    o, lse = attention(q, k, v, causal=causal, scale=scale, doc_starts=doc_starts)  # the complete forward
    qpos = rank_positions(seq_len, cp, rank, layout)
    dq = np.zeros((qpos.size, heads, dim))
    dk = np.zeros((seq_len, heads, dim))
    dv = np.zeros((seq_len, heads, dim))
    for s in range(cp):
        kpos = rank_positions(seq_len, cp, ring_source(rank, s, cp), layout)
        a, b, c = _pair_terms(q[qpos], k[kpos], v[kpos], dout[qpos], o[qpos], lse[:, qpos], qpos, kpos, causal,
                              scale, doc_starts=doc_starts)
        dq += a
        dk[kpos] += b
        dv[kpos] += c
    return dq, dk, dv, qpos


def full_backward(q, k, v, dout, cp, *, layout=ZIGZAG, causal=True, scale=None, doc_starts=None):
    """Every rank's share; ``(dQ, dK, dV)`` in natural order."""
    q = _f64(q)
    dq = np.zeros(q.shape)
    dk = np.zeros(q.shape)
    dv = np.zeros(q.shape)
    for r in range(cp):
        a, b, c, pos = rank_backward(q, k, v, dout, cp, r, layout=layout, causal=causal, scale=scale,
                                     doc_starts=doc_starts)
        dq[pos] = a
        dk += b
        dv += c
    return dq, dk, dv
