"""Fused ring (CP_ATTN_OPT_FUSED_RING 1, the default where served): every ring
step of a rank in one launch, the running max and sum carried in registers across steps, the
receives still arriving step by step on the copy stream and announced by
device flags.  The merge order differs from one launch per step, so results
agree with it to rounding; against the fp64 oracle they meet the same bounds.
The time-out path is forced from the host (mode 2: a flag value no signal
stores, 16 polls), so every kernel still ends normally.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd.inputs import WORKLOADS, make_qkv, workload_qkv, to_numpy_f64

pytestmark = pytest.mark.gpu


def _dev():
    assert torch.cuda.is_available(), "no GPU"
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _rank(p, qd, kd, vd, r):
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((p.heads, p.seq_len), float("nan"), device=qd.device)
    p.rank_forward(qd, kd, vd, out, lse, r)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _full(p, qd, kd, vd):
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((p.heads, p.seq_len), float("nan"), device=qd.device)
    p.full_forward(qd, kd, vd, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _same(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


def _rows_of(p, r):
    """Global rows of rank r (zigzag, no padding): chunks r and 2cp-1-r."""
    c = p.seq_len // (2 * p.cp_size)
    return np.concatenate([np.arange(r * c, (r + 1) * c), np.arange((2 * p.cp_size - 1 - r) * c, (2 * p.cp_size - r) * c)])


def _check_oracle(o, l, q, k, v, rows, heads, tol_o=2e-2, tol_l=1e-3):
    qn, kn, vn = (to_numpy_f64(t) for t in (q, k, v))
    for h in heads:
        o_r, l_r = oracle.attention(qn[rows][:, h:h + 1], kn[:, h:h + 1], vn[:, h:h + 1], causal=True, q_pos=rows)
        d_o = float(np.max(np.abs(o[rows, h:h + 1].double().numpy() - o_r)))
        d_l = float(np.max(np.abs(l[h, rows].double().numpy() - l_r[0])))
        assert d_o <= tol_o and d_l <= tol_l, (h, d_o, d_l)


CASES = [
    (2048, 4, 4),     # chunks of 256 keys
    (512, 2, 2),      # one receive; chunks of 128 keys
    (4096, 8, 3),     # heads not a multiple of 8; six receives
    (1536, 4, 2),     # chunks of 192 keys: runs of three tiles
]

# other layouts and masks: (seq, cp, heads, layout, causal)
LAYOUT_CASES = [
    (2048, 4, 3, "contiguous", True),    # a rank sees only the sources before it
    (2048, 4, 3, "contiguous", False),
    (2048, 4, 2, "zigzag", False),
    (4096, 8, 2, "contiguous", False),   # chunks of 512 keys, seven receives, key split
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_cp{c[1]}_h{c[2]}" for c in CASES])
def test_fused_ring_every_row_against_oracle_and_step_launches(case):
    seq, cp, heads = case
    _say(f"fused ring vs oracle and per-step launches: {case}")
    q, k, v = make_qkv(seq, heads, 128, "bf16", 91)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    p.set_fused_ring(False)
    ref_full = _full(p, qd, kd, vd)
    assert not p.fused_ring_active()
    p.set_fused_ring(True)
    o, l = _full(p, qd, kd, vd)
    assert p.fused_ring_active()
    assert not p.ring_wait_timeouts()
    assert torch.isfinite(o.float()).all() and torch.isfinite(l).all()
    # every row of every head against the oracle
    _check_oracle(o, l, q, k, v, np.arange(seq), range(heads))
    # against one launch per step: the same terms merged in another order
    assert float((o.float() - ref_full[0].float()).abs().max()) <= 1.6e-2
    assert float((l - ref_full[1]).abs().max()) <= 1e-4
    # a rank's call writes its rows only, the same values as in the full call
    for r in range(cp):
        o_r, l_r = _rank(p, qd, kd, vd, r)
        rows = torch.as_tensor(_rows_of(p, r))
        assert _same(o_r[rows], o[rows]) and _same(l_r[:, rows], l[:, rows]), r
        others = torch.ones(seq, dtype=torch.bool)
        others[rows] = False
        assert torch.isnan(o_r[others].float()).all(), r
    assert not p.ring_wait_timeouts()
    p.close()


def _rows_any(p, layout, r):
    if layout == "zigzag":
        return _rows_of(p, r)
    n = p.seq_len // p.cp_size
    return np.arange(r * n, (r + 1) * n)


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=[f"s{c[0]}_cp{c[1]}_h{c[2]}_{c[3]}_{'causal' if c[4] else 'bidir'}" for c in LAYOUT_CASES])
def test_fused_ring_layouts_and_bidirectional(case):
    """The contiguous layout (one row range per rank) and bidirectional
    attention in the fused launch: every row of every head against the
    oracle, within rounding of one launch per step, each rank's call
    writing its rows only."""
    seq, cp, heads, layout, causal = case
    _say(f"fused ring, layout/mask: {case}")
    q, k, v = make_qkv(seq, heads, 128, "bf16", 98)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, causal, layout)
    p.set_fused_ring(False)
    ref = _full(p, qd, kd, vd)
    p.set_fused_ring(True)
    o, l = _full(p, qd, kd, vd)
    assert p.fused_ring_active()
    assert not p.ring_wait_timeouts()
    qn, kn, vn = (to_numpy_f64(t) for t in (q, k, v))
    for h in range(heads):
        o_r, l_r = oracle.attention(qn[:, h:h + 1], kn[:, h:h + 1], vn[:, h:h + 1], causal=causal)
        assert float(np.max(np.abs(o[:, h:h + 1].double().numpy() - o_r))) <= 2e-2, h
        assert float(np.max(np.abs(l[h].double().numpy() - l_r[0]))) <= 1e-3, h
    assert float((o.float() - ref[0].float()).abs().max()) <= 1.6e-2
    assert float((l - ref[1]).abs().max()) <= 1e-4
    for r in (0, cp - 1):
        o_r, l_r = _rank(p, qd, kd, vd, r)
        rows = torch.as_tensor(_rows_any(p, layout, r))
        assert _same(o_r[rows], o[rows]) and _same(l_r[:, rows], l[:, rows]), r
        others = torch.ones(seq, dtype=torch.bool)
        others[rows] = False
        assert torch.isnan(o_r[others].float()).all(), r
    assert not p.ring_wait_timeouts()
    p.close()


def test_fused_ring_full_size_bidirectional_contiguous_rank0():
    """The 65536-token cp 16 bidirectional contiguous rank-0 share (8 heads):
    fused (key-split) launch within rounding of one launch per step on every
    row, sampled rows of the first and last head against the oracle."""
    w = WORKLOADS["bidir_s65536_cp16_contiguous_h8_d128_bf16_rank0"]
    _say(f"fused ring, full size: {w.name}")
    q, k, v = workload_qkv(w)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout)
    p.set_fused_ring(False)
    ref = _rank(p, qd, kd, vd, 0)
    p.set_fused_ring(True)
    o, l = _rank(p, qd, kd, vd, 0)
    assert p.fused_ring_active()
    assert not p.ring_wait_timeouts()
    p.close()
    rows = np.arange(w.seq_len // w.cp)
    rt = torch.as_tensor(rows)
    assert float((o[rt].float() - ref[0][rt].float()).abs().max()) <= 1.6e-2
    assert float((l[:, rt] - ref[1][:, rt]).abs().max()) <= 1e-4
    qn, kn, vn = (to_numpy_f64(t) for t in (q, k, v))
    sample = rows[::97]
    for h in (0, w.heads - 1):
        o_r, l_r = oracle.attention(qn[sample][:, h:h + 1], kn[:, h:h + 1], vn[:, h:h + 1], causal=False)
        assert float(np.max(np.abs(o[sample, h:h + 1].double().numpy() - o_r))) <= 2e-2, h
        assert float(np.max(np.abs(l[h, sample].double().numpy() - l_r[0]))) <= 1e-3, h


def test_fused_ring_calls_back_to_back_and_new_buffers():
    """Calls queued without a host synchronization between them, each with
    new output buffers and its own epoch, give the results of separate
    calls; so does a plan whose slots were made for an earlier call."""
    seq, cp, heads = 4096, 4, 8
    q, k, v = make_qkv(seq, heads, 128, "bf16", 92)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    p.set_fused_ring(True)
    ref = [_rank(p, qd, kd, vd, r) for r in range(cp)]
    _say("fused ring: calls back to back")
    outs = []
    for i in range(9):
        r = (3 * i) % cp
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((heads, seq), float("nan"), device=dev)
        p.rank_forward(qd, kd, vd, out, lse, r)
        outs.append((r, out, lse))
    torch.cuda.synchronize()
    for r, out, lse in outs:
        rows = torch.as_tensor(_rows_of(p, r))
        assert _same(out.cpu()[rows], ref[r][0][rows]) and _same(lse.cpu()[:, rows], ref[r][1][:, rows]), r
    # new inputs in the same buffers: the receives carry them
    qd.copy_(torch.flip(qd, dims=[1]))
    kd.mul_(0.5)
    o, l = _full(p, qd, kd, vd)
    _check_oracle(o, l, qd.cpu(), kd.cpu(), vd.cpu(), np.arange(0, seq, 7), (0, heads - 1))
    assert not p.ring_wait_timeouts()
    p.close()


def test_fused_ring_forced_timeout_is_reported():
    """Mode 2 makes every wait look for a flag value no signal stores and
    give up after 16 polls: the call returns, the time-out is reported once,
    and the plan then gives correct results in mode 1."""
    seq, cp, heads = 2048, 4, 2
    q, k, v = make_qkv(seq, heads, 128, "bf16", 93)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    p.set_fused_ring(True)
    ref = _rank(p, qd, kd, vd, 2)
    assert not p.ring_wait_timeouts()
    _say("fused ring: forced time-out")
    p.set_fused_ring("timeout_test")
    _rank(p, qd, kd, vd, 2)
    assert p.ring_wait_timeouts()
    assert not p.ring_wait_timeouts()  # cleared by the query
    p.set_fused_ring(True)
    o, l = _rank(p, qd, kd, vd, 2)
    assert _same(o, ref[0]) and _same(l, ref[1])
    assert not p.ring_wait_timeouts()
    p.close()


def test_fused_ring_falls_back_where_not_served():
    """Padding, documents,
    fp32, head_dim 64, the separate merge, the serial mode, the memcpy
    receive, work counters and poison take one
    launch per step with the option set: the same bits as without it, and
    no wait is polled (the time-out test mode would report one)."""
    dev = _dev()
    setups = [
        dict(seq=1003), dict(docs=[0, 100, 700]),
        dict(dtype=torch.float32), dict(dim=64), dict(opt="merge"), dict(opt="serial"), dict(opt="memcpy"),
        dict(opt="counters"), dict(opt="poison"),
    ]
    for st in setups:
        seq, layout, causal = st.get("seq", 1024), st.get("layout", "zigzag"), st.get("causal", True)
        dtype, dim = st.get("dtype", torch.bfloat16), st.get("dim", 128)
        _say(f"fused ring fallback: {st}")
        q, k, v = make_qkv(seq, 2, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 94)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        p = Plan(seq, 4, 2, dim, causal, layout, dtype=dtype)
        if "docs" in st:
            p.set_documents(st["docs"])
        opt = st.get("opt")
        if opt == "merge":
            p.set_merge(True)
        if opt == "serial":
            p.set_serialize(True)
        if opt == "memcpy":
            p.set_recv("memcpy")
        if opt == "counters":
            p.set_counters(True)
        if opt == "poison":
            p.set_poison(True)
        p.set_fused_ring(False)
        ref = _rank(p, qd, kd, vd, 1)
        p.set_fused_ring("timeout_test")
        for _ in range(2):
            o, l = _rank(p, qd, kd, vd, 1)
            assert _same(o, ref[0]) and _same(l, ref[1]), st
            assert not p.fused_ring_active(), st
        assert not p.ring_wait_timeouts(), st
        p.close()


@pytest.mark.parametrize("name", ["causal_s32768_cp8_zigzag_h32_d128_bf16_rank0", "causal_s8192_cp4_zigzag_h32_d128_bf16"])
def test_fused_ring_full_size(name):
    """The 32768-token cp 8 rank-0 share and the 8192-token cp 4 full forward:
    every row of the first and last head against the fp64 oracle, and every
    row of every head within rounding of one launch per step."""
    w = WORKLOADS[name]
    _say(f"fused ring, full size: {w.name}")
    q, k, v = workload_qkv(w)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout)
    rank0 = name.endswith("rank0")
    p.set_fused_ring(False)
    ref = _rank(p, qd, kd, vd, 0) if rank0 else _full(p, qd, kd, vd)
    p.set_fused_ring(True)
    o, l = _rank(p, qd, kd, vd, 0) if rank0 else _full(p, qd, kd, vd)
    assert p.fused_ring_active()
    assert not p.ring_wait_timeouts()
    p.close()
    rows = _rows_of(p, 0) if rank0 else np.arange(w.seq_len)
    rt = torch.as_tensor(rows)
    assert float((o[rt].float() - ref[0][rt].float()).abs().max()) <= 1.6e-2
    assert float((l[:, rt] - ref[1][:, rt]).abs().max()) <= 1e-4
    _check_oracle(o, l, q, k, v, rows, (0, w.heads - 1))


SPLIT_CASES = [
    (6144, 4, 5),     # three row tiles per chunk, heads not a multiple of 8
    (2048, 4, 4),     # one row tile per chunk; the last rank splits both row ranges
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[f"s{c[0]}_cp{c[1]}_h{c[2]}" for c in SPLIT_CASES])
def test_fused_ring_key_split_every_row(case):
    """With few workgroups the fused launch splits a row tile's keys in two
    parts (the first half of every step's keys, then the second halves and
    the diagonal), merged by the part that ends last: every row of every
    head of every rank against the oracle, within rounding of the unsplit
    fused launch, and the same bits call after call."""
    seq, cp, heads = case
    _say(f"fused ring key split: {case}")
    q, k, v = make_qkv(seq, heads, 128, "bf16", 97)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    for r in range(cp):
        p.set_key_split(False)
        ref = _rank(p, qd, kd, vd, r)
        assert p.fused_ring_active() == 1, r
        p.set_key_split(True)
        o, l = _rank(p, qd, kd, vd, r)
        assert p.fused_ring_active() == 2, r
        rows = _rows_of(p, r)
        rt = torch.as_tensor(rows)
        assert float((o[rt].float() - ref[0][rt].float()).abs().max()) <= 1.6e-2, r
        assert float((l[:, rt] - ref[1][:, rt]).abs().max()) <= 1e-4, r
        _check_oracle(o, l, q, k, v, rows, range(heads))
        o2, l2 = _rank(p, qd, kd, vd, r)
        assert _same(o2, o) and _same(l2, l), r
    assert not p.ring_wait_timeouts()
    p.close()


@pytest.mark.parametrize("rank", [0, 1, 3])
def test_fused_ring_key_split_full_size_16_heads(rank):
    """The 16384-token cp 4 workload with 16 heads: ranks 0 and 1 split
    (their launches alone would leave compute units idle), rank 3 does not;
    rows of the first and last head against the oracle, every row of every
    head within rounding of one launch per step."""
    w = WORKLOADS["causal_s16384_cp4_zigzag_h16_d128_bf16"]
    _say(f"fused ring key split, full size: {w.name} rank {rank}")
    q, k, v = workload_qkv(w)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout)
    p.set_fused_ring(False)
    ref = _rank(p, qd, kd, vd, rank)
    p.set_fused_ring(True)
    o, l = _rank(p, qd, kd, vd, rank)
    assert p.fused_ring_active() == (1 if rank == 3 else 2)
    assert not p.ring_wait_timeouts()
    p.close()
    rows = _rows_of(p, rank)
    rt = torch.as_tensor(rows)
    assert float((o[rt].float() - ref[0][rt].float()).abs().max()) <= 1.6e-2
    assert float((l[:, rt] - ref[1][:, rt]).abs().max()) <= 1e-4
    _check_oracle(o, l, q, k, v, rows[::5], (0, w.heads - 1))


def test_fused_ring_staged_equals_overlapped_bits():
    """Mode 3 waits for every receive before the launch (no wait is polled,
    nothing overlaps): the same kernel on the same data, so the same bits as
    mode 1, call after call."""
    seq, cp, heads = 4096, 8, 4
    q, k, v = make_qkv(seq, heads, 128, "bf16", 95)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    _say("fused ring: staged vs overlapped")
    ref = _full(p, qd, kd, vd)
    assert p.fused_ring_active()
    p.set_fused_ring("staged")
    for _ in range(2):
        o, l = _full(p, qd, kd, vd)
        assert p.fused_ring_active()
        assert _same(o, ref[0]) and _same(l, ref[1])
    assert not p.ring_wait_timeouts()
    p.close()


def test_fused_ring_graph_replays_match_eager():
    """Graph mode records the fused launch with its receives, their signals
    and the kernel that advances the call's epoch in device memory: every
    replay waits for its own receives, so each equals the eager call bit for
    bit (eager work and host synchronisation between replays), also after
    the inputs change in place, for one rank's share and the full forward."""
    seq, cp, heads = 4096, 4, 8
    q, k, v = make_qkv(seq, heads, 128, "bf16", 96)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    for rank in (1, None):
        _say(f"fused ring graph replays: rank {rank}")
        call = (lambda: _rank(p, qd, kd, vd, rank)) if rank is not None else (lambda: _full(p, qd, kd, vd))
        p.set_graph(False)
        ref = call()
        assert p.fused_ring_active() == 2  # (with the key split)
        p.set_graph(True)
        for i in range(4):
            junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
            torch.cuda.synchronize()
            o, l = call()
            assert torch.isfinite(junk)
            assert _same(o, ref[0]) and _same(l, ref[1]), (rank, i)
        assert p.fused_ring_active()
        # new contents in the same buffers: the replays receive them
        kd.mul_(0.75)
        vd.add_(0.5)
        p.set_graph(False)
        ref2 = call()
        assert not _same(ref2[0], ref[0])
        p.set_graph(True)
        for i in range(2):
            o, l = call()
            assert _same(o, ref2[0]) and _same(l, ref2[1]), (rank, "changed", i)
    assert not p.ring_wait_timeouts()
    p.close()
