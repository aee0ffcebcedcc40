"""O2: context-parallel decomposition of attention in fp64, plus work counts.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

This module has its own chunk map; it does not use the HIP library's plan.

* Chunk placement ("Sequence Parallelism IV: Megatron Context Parallel and
  Load-Balanced Rings", section 3 "Naive Ring Attention Is Imbalanced Under
  Causal Masks"): the sequence is cut into ``2*cp`` equal chunks and rank ``r``
  owns one early and one late chunk, ``{r, 2*cp-1-r}`` (the page's cp=4 example
  is ranks {0,7},{1,6},{2,5},{3,4}).  A rank keeps its two chunks in that
  order, early chunk first.  The naive placement gives rank ``r`` the
  contiguous slice ``[r*S/cp, (r+1)*S/cp)`` (same section, and the shard
  coverage check of "Context Parallelism for Long-Context Training", section
  "Test sequence divisibility and padding").  Per-rank length is
  ``S // cp`` ("Context Parallelism in MegaDLMs", section "Sequence
  Partitioning Across GPUs").
* Ring (same page, sections 4 "What Actually Moves" and 5 "Overlap"): Q stays
  on its rank; K/V chunks move to a neighbour each iteration.  The pages fix no
  direction; rank ``r`` receives from ``r-1``, so at step ``s`` it holds the
  K/V of rank ``(r - s) mod cp`` and step 0 is its own K/V.
* Exact merge (section 4): each step yields a partial ``(O_s, lse_s)`` over the
  keys present; partials are folded with log-sum-exp weights, which reproduces
  the unsplit softmax exactly up to rounding.
* Padding ("Context Parallelism for Long-Context Training", section "Test
  sequence divisibility and padding": the page asks which rank holds each pad
  token, that pad keys and pad queries be masked, and that adding them leave
  every real token's output as it was).  A length
  that does not divide into the chunks is padded at the end to the next
  multiple; the pad positions belong to the rank that owns their chunk, are
  never attended as keys and produce no output.  ``rank_positions`` lists the
  real positions only; for any chunk the real positions are a prefix of it,
  so a rank's real rows keep their local indices.
* Work counts (section 3): per ring iteration, the number of valid (q, k)
  pairs and of BMxBN tiles holding at least one valid pair, per rank; the
  imbalance of an iteration is max over ranks / mean over ranks, and the
  lockstep cost of a whole pass is sum of maxima / sum of means.
"""

import numpy as np

from .attention import attention, valid_mask

ZIGZAG = "zigzag"
CONTIGUOUS = "contiguous"


def _check(seq_len, cp, layout):
    if cp < 1:
        raise ValueError("cp must be >= 1")
    if seq_len < 1:
        raise ValueError("seq_len must be >= 1")
    if layout not in (ZIGZAG, CONTIGUOUS):
        raise ValueError(f"unknown layout {layout!r}")


def _parts(cp, layout):
    return 2 * cp if layout == ZIGZAG else cp


def padded_length(seq_len, cp, layout):
    """``seq_len`` rounded up to a multiple of the number of chunks."""
    _check(seq_len, cp, layout)
    n = _parts(cp, layout)
    return -(-seq_len // n) * n


def chunk_size(seq_len, cp, layout):
    """Length of one chunk of the padded sequence: ``S_pad/(2cp)`` (zigzag) or ``S_pad/cp``."""
    return padded_length(seq_len, cp, layout) // _parts(cp, layout)


def rank_chunks(cp, layout):
    """Chunk indices owned by each rank, in the rank's local order."""
    if layout == ZIGZAG:
        return [(r, 2 * cp - 1 - r) for r in range(cp)]
    if layout == CONTIGUOUS:
        return [(r,) for r in range(cp)]
    raise ValueError(f"unknown layout {layout!r}")


def rank_positions(seq_len, cp, rank, layout):
    """Global token positions of rank ``rank``'s real local rows, in local order
    (pad positions, at or past ``seq_len``, are left out)."""
    c = chunk_size(seq_len, cp, layout)
    parts = [np.arange(ch * c, min((ch + 1) * c, seq_len), dtype=np.int64) for ch in rank_chunks(cp, layout)[rank]]
    return np.concatenate(parts)


def ring_source(rank, step, cp):
    """Rank whose K/V chunks rank ``rank`` holds at ring step ``step``."""
    return (rank - step) % cp


def merge_partial(o_acc, lse_acc, o_s, lse_s):
    """Fold a partial ``(o_s, lse_s)`` into ``(o_acc, lse_acc)`` exactly.

    Shapes: ``o_* [N, H, D]``, ``lse_* [H, N]``.  A partial with ``lse = -inf``
    (no valid key) changes nothing; an empty accumulator takes the partial.
    Otherwise ``lse' = max + log1p(exp(-|lse_acc - lse_s|))`` and
    ``O' = exp(lse_acc - lse') O_acc + exp(lse_s - lse') O_s``.
    Returns new arrays.
    """
    o_acc = np.array(o_acc, dtype=np.float64)
    lse_acc = np.array(lse_acc, dtype=np.float64)
    o_s = np.asarray(o_s, dtype=np.float64)
    lse_s = np.asarray(lse_s, dtype=np.float64)
    a = lse_acc.T  # [N, H]
    b = lse_s.T
    take = np.isneginf(a) & ~np.isneginf(b)
    both = ~np.isneginf(a) & ~np.isneginf(b)
    new = a.copy()
    new[take] = b[take]
    o_new = o_acc.copy()
    o_new[take] = o_s[take]
    if np.any(both):
        aa, bb = a[both], b[both]
        lse_new = np.maximum(aa, bb) + np.log1p(np.exp(-np.abs(aa - bb)))
        wa = np.exp(aa - lse_new)
        wb = np.exp(bb - lse_new)
        o_new[both] = wa[:, None] * o_acc[both] + wb[:, None] * o_s[both]
        new[both] = lse_new
    return o_new, new.T.copy()


def rank_forward(q, k, v, cp, rank, *, layout=ZIGZAG, causal=True, scale=None, step_order=None, doc_starts=None):
    """One rank's share: its Q rows against every rank's K/V, one ring step at a time.

    q, k, v: natural-order ``[S, H, D]``.  Returns ``(O_loc [n, H, D],
    LSE_loc [H, n], positions [n])`` for the rank's local rows.
    ``step_order`` permutes the ring steps (the merge is order-invariant).
    """
    seq_len, heads, dim = np.shape(q)
    qpos = rank_positions(seq_len, cp, rank, layout)
    qloc = np.asarray(q)[qpos]
    o_acc = np.zeros((qpos.size, heads, dim), dtype=np.float64)
    lse_acc = np.full((heads, qpos.size), -np.inf, dtype=np.float64)
    steps = range(cp) if step_order is None else step_order
    for s in steps:
        j = ring_source(rank, s, cp)
        kpos = rank_positions(seq_len, cp, j, layout)
        o_s, lse_s = attention(qloc, np.asarray(k)[kpos], np.asarray(v)[kpos],
                               causal=causal, scale=scale, q_pos=qpos, k_pos=kpos, doc_starts=doc_starts)
        o_acc, lse_acc = merge_partial(o_acc, lse_acc, o_s, lse_s)
    return o_acc, lse_acc, qpos


def full_forward(q, k, v, cp, *, layout=ZIGZAG, causal=True, scale=None, step_orders=None, doc_starts=None):
    """Every rank's share, assembled back to natural token order.

    Returns ``(O [S, H, D], LSE [H, S])``.
    """
    seq_len, heads, dim = np.shape(q)
    out = np.zeros((seq_len, heads, dim), dtype=np.float64)
    lse = np.full((heads, seq_len), -np.inf, dtype=np.float64)
    for r in range(cp):
        order = None if step_orders is None else step_orders[r]
        o, l, pos = rank_forward(q, k, v, cp, r, layout=layout, causal=causal, scale=scale, step_order=order,
                                 doc_starts=doc_starts)
        out[pos] = o
        lse[:, pos] = l
    return out, lse


def sequence_shards(x, cp, layout):
    """Sequence ownership: ``[cp, S_pad/cp, H, D]``, rank ``r``'s rows in its
    local order (its real rows first; pad rows zero)."""
    x = np.asarray(x)
    seq_len = x.shape[0]
    n_loc = padded_length(seq_len, cp, layout) // cp
    out = np.zeros((cp, n_loc) + x.shape[1:], dtype=x.dtype)
    for r in range(cp):
        pos = rank_positions(seq_len, cp, r, layout)
        out[r, :pos.size] = x[pos]
    return out


def head_shards(x, cp):
    """Head ownership after the Ulysses all-to-all ("Sequence Parallelism IV",
    section 7 "CP vs Ulysses": a rank ends with every token of a head slice):
    ``[cp, S, H/cp, D]``, rank ``r`` holding heads ``[r H/cp, (r+1) H/cp)``."""
    x = np.asarray(x)
    heads = x.shape[1]
    if heads % cp:
        raise ValueError("the head count must divide by cp (Ulysses is bounded by the heads)")
    g = heads // cp
    return np.stack([x[:, r * g:(r + 1) * g] for r in range(cp)])


def ulysses_forward(q, k, v, cp, *, causal=True, scale=None):
    """Every rank's attention over all tokens of its head slice, assembled to
    natural order ``(O [S, H, D], LSE [H, S])``."""
    qs, ks, vs = (head_shards(x, cp) for x in (q, k, v))
    seq_len, heads, dim = np.shape(q)
    g = heads // cp
    out = np.zeros((seq_len, heads, dim))
    lse = np.zeros((heads, seq_len))
    for r in range(cp):
        o, l = attention(qs[r], ks[r], vs[r], causal=causal, scale=scale)
        out[:, r * g:(r + 1) * g] = o
        lse[r * g:(r + 1) * g] = l
    return out, lse


def step_valid_pairs(seq_len, cp, layout, causal, rank, step, doc_starts=None):
    """Valid (q, k) pairs of one head in ring step ``step`` of rank ``rank``."""
    qpos = rank_positions(seq_len, cp, rank, layout)
    kpos = rank_positions(seq_len, cp, ring_source(rank, step, cp), layout)
    if doc_starts is not None:
        return int(valid_mask(qpos, kpos, causal, doc_starts=doc_starts).sum())
    if not causal:
        return int(qpos.size * kpos.size)
    ks = np.sort(kpos)
    return int(np.searchsorted(ks, qpos, side="right").sum())


def step_valid_tiles(seq_len, cp, layout, causal, rank, step, bm, bn):
    """Tiles of ``bm`` local rows x ``bn`` local keys holding a valid pair.

    Tiles are laid on the rank's local row index and on the source's local key
    index from 0, the last tile of each axis clipped at the buffer end.
    """
    qpos = rank_positions(seq_len, cp, rank, layout)
    kpos = rank_positions(seq_len, cp, ring_source(rank, step, cp), layout)
    if not causal:
        return -(-qpos.size // bm) * -(-kpos.size // bn)
    # A tile holds a causal pair (k <= q) exactly when its smallest key
    # position is not after its largest query position.
    qmax = [int(qpos[i0:i0 + bm].max()) for i0 in range(0, qpos.size, bm)]
    kmin = [int(kpos[j0:j0 + bn].min()) for j0 in range(0, kpos.size, bn)]
    return sum(1 for a in qmax for b in kmin if b <= a)


def imbalance(work):
    """Load imbalance of a ``[cp, cp]`` (rank, step) work table.

    Returns ``(per_step, aggregate)``: per step ``max_r w / mean_r w`` (1.0 when
    the step has no work at all) and ``sum_s max_r w / sum_s mean_r w``.
    """
    w = np.asarray(work, dtype=np.float64)
    mx = w.max(axis=0)
    mean = w.mean(axis=0)
    per_step = [float(a / b) if b > 0 else 1.0 for a, b in zip(mx, mean)]
    aggregate = float(mx.sum() / mean.sum()) if mean.sum() > 0 else 1.0
    return per_step, aggregate


def valid_flops(pairs, heads, head_dim):
    """Mask-valid FLOPs: ``4 * head_dim`` per valid pair per head.

    ``Q K^T`` and ``P V`` each cost ``head_dim`` multiply-adds (two flops each)
    per valid pair; softmax and masked or skipped work are not counted.
    """
    return 4 * int(head_dim) * int(heads) * int(pairs)
