"""Host-side tests of the C ABI (no GPU): exports, plan, descriptors, counts, errors.

These call only host-only entry points of libcpattn.so (no device work) and
compare the plan against the fp64 oracle's own chunk map and brute-force
global-position masks.
"""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from ring_context_parallelism_amd import _native as N
from ring_context_parallelism_amd import Plan, CpAttnError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cp_attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(N.LIB_PATH), reason="libcpattn.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 15
    lib = N.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(N.SIGNATURES), "binding table and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", N.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (cp_attn_\w+)", out))
    assert set(names) <= exported


@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
@pytest.mark.parametrize("cp", [1, 2, 3, 4, 8])
def test_chunk_map_and_sources_match_oracle(layout, cp):
    seq = 2 * cp * 32
    p = Plan(seq, cp, 2, 64, True, layout)
    want = oracle.rank_chunks(cp, layout)
    for r in range(cp):
        assert p.rank_chunks(r) == tuple(want[r])
        for s in range(cp):
            assert p.step_source(r, s) == oracle.ring_source(r, s, cp)
    assert p.local_rows() == oracle.rank_positions(seq, cp, 0, layout).size


def test_page_example_map():
    p = Plan(8192, 4, 32, 128)
    assert [p.rank_chunks(r) for r in range(4)] == [(0, 7), (1, 6), (2, 5), (3, 4)]
    assert p.local_rows() == 2048


def _descriptor_mask(p, r, s, seq, cp, layout):
    n = oracle.rank_positions(seq, cp, r, layout).size
    nk = oracle.rank_positions(seq, cp, oracle.ring_source(r, s, cp), layout).size
    mask = np.zeros((n, nk), dtype=bool)
    firsts = []
    for g in p.step_segments(r, s):
        for t in range(g["q_len"]):
            row = g["q_start"] + t
            pre = g["kv_full"] + (t + 1 if g["diag"] else 0)
            assert row < n and pre <= nk  # real rows see real keys only
            mask[row, :pre] = True
            assert g["q_global"] + t == oracle.rank_positions(seq, cp, r, layout)[row]
        firsts.append(g)
    return mask


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
def test_descriptors_equal_global_position_mask_exhaustive(causal, layout):
    """Every (rank, step) for S <= 64 (every length, divisible or padded), cp <= 8:
    descriptor mask == brute-force mask over the real rows and keys."""
    checked = 0
    for cp in range(1, 9):
        for seq in range(1, 65):
            p = Plan(seq, cp, 1, 64, causal, layout)
            assert p.local_rows() == oracle.padded_length(seq, cp, layout) // cp
            for r in range(cp):
                qpos = oracle.rank_positions(seq, cp, r, layout)
                assert p.rank_valid_rows(r) == qpos.size
                for s in range(cp):
                    kpos = oracle.rank_positions(seq, cp, oracle.ring_source(r, s, cp), layout)
                    want = oracle.valid_mask(qpos, kpos, causal)
                    got = _descriptor_mask(p, r, s, seq, cp, layout)
                    assert np.array_equal(got, want), (cp, seq, r, s)
                    checked += 1
            p.close()
    assert checked > 10000


@pytest.mark.parametrize("seq", [128, 101])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
def test_first_last_flags(layout, causal, seq):
    """Each run of local rows is initialised once and finalised once, in ring order."""
    cp = 4
    p = Plan(seq, cp, 1, 64, causal, layout)
    for r in range(cp):
        seen = {}
        for s in range(cp):
            for g in p.step_segments(r, s):
                seen.setdefault(g["q_start"], []).append((s, g["first"], g["last"]))
        covered = sum(p.step_segments(r, s)[0]["q_len"] for s in range(1) for _ in [0])
        assert covered > 0
        for steps in seen.values():
            assert [f for _, f, _ in steps] == [1] + [0] * (len(steps) - 1)
            assert [l for _, _, l in steps] == [0] * (len(steps) - 1) + [1]
        rows = sorted(q for q in seen)
        total = sum(next(g["q_len"] for s in range(cp) for g in p.step_segments(r, s) if g["q_start"] == q)
                    for q in rows)
        assert total == p.rank_valid_rows(r)  # every real local row gets a result


@pytest.mark.parametrize("seq,cp,layout,causal,bm,bn", [
    (16384, 4, "zigzag", True, 128, 128), (16384, 4, "contiguous", True, 128, 128),
    (16384, 4, "contiguous", True, 64, 64), (8192, 4, "zigzag", True, 128, 64),
    (32768, 8, "zigzag", True, 128, 64), (4096, 16, "contiguous", False, 128, 64),
    (800, 2, "zigzag", True, 128, 64), (960, 3, "contiguous", True, 64, 48),
    # padded lengths
    (1003, 4, "zigzag", True, 256, 64), (1003, 4, "zigzag", False, 256, 64),
    (4099, 8, "zigzag", True, 32, 64), (1000, 3, "contiguous", True, 64, 64),
    (999, 7, "contiguous", False, 32, 64), (21, 8, "zigzag", True, 256, 64),
])
def test_work_counts_match_oracle(seq, cp, layout, causal, bm, bn):
    p = Plan(seq, cp, 1, 128, causal, layout)
    for r in range(cp):
        for s in range(cp):
            tiles, pairs = p.valid_work(r, s, bm, bn)
            assert pairs == oracle.step_valid_pairs(seq, cp, layout, causal, r, s)
            assert tiles == oracle.step_valid_tiles(seq, cp, layout, causal, r, s, bm, bn)


def _status(fn):
    try:
        fn()
    except CpAttnError as e:
        return e.status
    return N.OK


def test_plan_error_codes():
    lib = N.lib()
    h = ctypes.c_void_p()
    cases = [
        ((0, 1, 2, 128, 1, N.ZIGZAG), N.EINVAL),
        ((64, 0, 2, 128, 1, N.ZIGZAG), N.EINVAL),
        ((64, 2, 0, 128, 1, N.ZIGZAG), N.EINVAL),
        ((64, 2, 2, 128, 2, N.ZIGZAG), N.EINVAL),        # causal flag
        ((64, 2, 2, 128, 1, 7), N.EINVAL),               # layout
        ((64, 2, 2, 96, 1, N.ZIGZAG), N.EUNSUPPORTED),   # head_dim
        ((1024, 512, 2, 128, 1, N.ZIGZAG), N.EUNSUPPORTED),  # cp > 256
        ((1 << 20, 1, 32, 128, 1, N.ZIGZAG), N.EUNSUPPORTED),  # one rank's fp32 rows reach 2^32 bytes
        ((1 << 31, 256, 1, 64, 1, N.ZIGZAG), N.EUNSUPPORTED),  # 2^31 tokens
    ]
    for args, want in cases:
        assert lib.cp_attn_plan(*args, ctypes.byref(h)) == want, args
        assert not h.value
        assert lib.cp_attn_last_error()
    assert lib.cp_attn_plan(64, 2, 2, 128, 1, N.ZIGZAG, None) == N.EINVAL
    # natural-order tensors beyond 4 GiB are fine while one rank's rows stay below it
    for args in ((1 << 19, 16, 32, 128, 1, N.ZIGZAG), ((1 << 20) - 5, 8, 16, 128, 1, N.CONTIGUOUS)):
        assert lib.cp_attn_plan(*args, ctypes.byref(h)) == N.OK, args
        assert lib.cp_attn_plan_destroy(h) == N.OK
    for s in (N.OK, N.EINVAL, N.EUNSUPPORTED, N.ENOWORKSPACE, N.EHIP, 12345):
        assert lib.cp_attn_status_string(s)


def test_call_error_codes_enqueue_nothing():
    lib = N.lib()
    p = Plan(256, 2, 2, 64, True, "zigzag", dtype=__import__("torch").float32)
    h = p._h
    dummy = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.cp_attn_rank_forward(h, dummy, dummy, dummy, dummy, dummy, 2, None) == N.EINVAL
    assert lib.cp_attn_rank_forward(h, dummy, dummy, dummy, dummy, dummy, -1, None) == N.EINVAL
    assert lib.cp_attn_rank_forward(h, None, dummy, dummy, dummy, dummy, 0, None) == N.EINVAL
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert lib.cp_attn_full_forward(h, dummy, mis, dummy, dummy, dummy, None) == N.EINVAL
    assert lib.cp_attn_rank_forward(None, dummy, dummy, dummy, dummy, dummy, 0, None) == N.EINVAL
    assert lib.cp_attn_set_dtype(h, 5) == N.EINVAL
    assert lib.cp_attn_set_option(h, 99, 1) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_MERGE, 3) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_RECV, 4) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_RECV, -1) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_RECV, 3) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_GRAPH, 2) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_GRAPH, 1) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_GRAPH, 0) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_KSPLIT, 2) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_KSPLIT, 0) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_KSPLIT, 1) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_BWD_KEYS, 2) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_BWD_KEYS, -1) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_BWD_KEYS, 1) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_BWD_KEYS, 0) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_LOCKSTEP, 2) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_LOCKSTEP, 1) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_LOCKSTEP, 0) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_FUSED_RING, 4) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_FUSED_RING, -1) == N.EINVAL
    for mode in (3, 2, 1, 0):
        assert lib.cp_attn_set_option(h, N.OPT_FUSED_RING, mode) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_BWD_FUSED, 3) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_BWD_FUSED, -1) == N.EINVAL
    for mode in (0, 2, 1):
        assert lib.cp_attn_set_option(h, N.OPT_BWD_FUSED, mode) == N.OK
    assert lib.cp_attn_set_option(h, N.OPT_RECV_BLOCKS, -2) == N.EINVAL
    for nb in (0, 3, 1024, -1):  # -1: the automatic grid
        assert lib.cp_attn_set_option(h, N.OPT_RECV_BLOCKS, nb) == N.OK
    assert lib.cp_attn_ring_wait_timeouts(h, None) == N.EINVAL
    t = ctypes.c_int32(7)
    assert lib.cp_attn_ring_wait_timeouts(h, ctypes.byref(t)) == N.OK and t.value == 0  # nothing run yet
    assert lib.cp_attn_set_option(h, N.OPT_COUNTERS, 2) == N.EINVAL
    assert lib.cp_attn_set_option(h, N.OPT_COUNTERS, 0) == N.OK
    assert lib.cp_attn_last_tile_counts(h, None, 4, None, None) == N.EINVAL
    assert lib.cp_attn_set_workspace(h, ctypes.c_void_p(256), 16) == N.ENOWORKSPACE
    assert lib.cp_attn_set_workspace(h, ctypes.c_void_p(100), 1 << 30) == N.EINVAL
    assert lib.cp_attn_step_source(h, 0, 5, ctypes.byref(ctypes.c_int32())) == N.EINVAL
    assert lib.cp_attn_valid_work(h, 0, 0, 0, 64, None, None) == N.EINVAL
    assert lib.cp_attn_lse_merge(None, None, None, None, 4, 1, 128, None) == N.EINVAL
    buf = (ctypes.c_float * 1)()
    assert lib.cp_attn_last_step_times(h, buf, 1) == N.EINVAL
    p.close()


def test_workspace_size_formula():
    import torch
    p = Plan(32768, 8, 32, 128, True, "zigzag")
    n, hd = 4096, 32 * 128
    kv = n * hd * 2
    o = n * hd * 4
    lse = 32 * n * 4
    cnt = -(-((n // 256 + 2) * 32 * 4) // 256) * 256
    doc = 32768 * 8  # document table: two int32 per token
    assert p.workspace_bytes() == 4 * kv + o + lse + 2 * (o + lse) + cnt + doc
    q = Plan(256, 2, 2, 64, True, "zigzag", dtype=torch.float32)
    assert q.workspace_bytes() == 4 * (128 * 128 * 4) + 3 * (128 * 128 * 4 + 2 * 128 * 4) + 256 + 256 * 8


def test_ulysses_argument_errors_enqueue_nothing():
    """Ulysses is bounded by the head count: heads % cp != 0 is unsupported;
    bad flags are rejected before any device work."""
    lib = N.lib()
    dummy = ctypes.c_void_p(1 << 20)  # never dereferenced
    with Plan(96, 3, 2, 64, True, "zigzag") as p:
        assert lib.cp_attn_ulysses_a2a(p._h, dummy, dummy, 1, None) == N.EUNSUPPORTED
        assert lib.cp_attn_ulysses_forward(p._h, dummy, dummy, dummy, dummy, dummy, None) == N.EUNSUPPORTED
    with Plan(96, 2, 4, 64, True, "zigzag") as p:
        assert lib.cp_attn_ulysses_a2a(p._h, dummy, dummy, 2, None) == N.EINVAL
        assert lib.cp_attn_ulysses_a2a(p._h, None, dummy, 1, None) == N.EINVAL
        assert lib.cp_attn_ulysses_forward(p._h, None, dummy, dummy, dummy, dummy, None) == N.EINVAL


# ------------------------------------------------------- document masks ----

def test_document_list_errors():
    """cp_attn_set_documents takes strictly increasing starts from 0, all below S."""
    lib = N.lib()
    with Plan(100, 2, 1, 64, True, "zigzag") as p:
        def put(xs, count=None):
            arr = (ctypes.c_int64 * max(1, len(xs)))(*xs)
            return lib.cp_attn_set_documents(p._h, arr, len(xs) if count is None else count)
        assert put([0, 10, 50]) == N.OK
        assert put([]) == N.OK
        for bad in ([1, 10], [0, 10, 10], [0, 50, 20], [0, 100], [0, -3]):
            assert put(bad) == N.EINVAL, bad
            assert lib.cp_attn_last_error()
        assert put([0], count=-1) == N.EINVAL
        assert lib.cp_attn_set_documents(p._h, None, 2) == N.EINVAL
        assert lib.cp_attn_set_documents(p._h, None, 0) == N.OK
        assert lib.cp_attn_set_documents(None, None, 0) == N.EINVAL


def _tiles_brute(seq, cp, layout, causal, r, s, bm, bn, docs):
    qpos = oracle.rank_positions(seq, cp, r, layout)
    kpos = oracle.rank_positions(seq, cp, oracle.ring_source(r, s, cp), layout)
    m = oracle.valid_mask(qpos, kpos, causal, doc_starts=docs)
    return sum(bool(m[i:i + bm, j:j + bn].any()) for i in range(0, qpos.size, bm) for j in range(0, kpos.size, bn))


@pytest.mark.parametrize("seq,cp,layout,causal,bm,bn,docs", [
    (256, 2, "zigzag", True, 32, 64, [0, 100, 130, 131, 200]),
    (256, 2, "zigzag", False, 32, 64, [0, 64, 128, 192]),
    (512, 4, "zigzag", True, 64, 32, [0, 1, 2, 63, 64, 65, 300, 511]),
    (1003, 4, "zigzag", True, 256, 64, "random"),
    (1000, 3, "contiguous", True, 64, 64, "random"),
    (999, 7, "contiguous", False, 32, 64, "random"),
    (4099, 8, "zigzag", True, 32, 64, "random"),
    (21, 8, "zigzag", True, 256, 64, [0, 5, 6, 20]),
])
def test_document_work_counts_match_oracle(seq, cp, layout, causal, bm, bn, docs):
    """Valid pairs and tiles under document masks equal the oracle's brute-force
    mask (same document and the plan's causal/bidirectional mask); clearing
    the documents restores the plain counts."""
    from ring_context_parallelism_amd.inputs import make_documents
    if docs == "random":
        docs = make_documents(seq, max(2, seq // 9), seed=seq + cp)
    p = Plan(seq, cp, 1, 128, causal, layout)
    p.set_documents(docs)
    total = 0
    for r in range(cp):
        for s in range(cp):
            tiles, pairs = p.valid_work(r, s, bm, bn)
            assert pairs == oracle.step_valid_pairs(seq, cp, layout, causal, r, s, doc_starts=docs), (r, s)
            assert tiles == _tiles_brute(seq, cp, layout, causal, r, s, bm, bn, docs), (r, s)
            total += pairs
    lens = np.diff(list(docs) + [seq])
    assert total == int(sum(n * (n + 1) // 2 for n in lens) if causal else sum(n * n for n in lens))
    p.set_documents(None)
    for r in range(cp):
        assert p.valid_work(r, 0, bm, bn)[1] == oracle.step_valid_pairs(seq, cp, layout, causal, r, 0)


@pytest.mark.parametrize("seq,cp,layout,causal", [(1003, 4, "zigzag", True), (1000, 3, "contiguous", True),
                                                  (999, 7, "contiguous", False), (4096, 8, "zigzag", True)])
def test_document_plan_drops_empty_segments(seq, cp, layout, causal):
    """Under document masks every kept segment holds a valid pair, step 0
    keeps every real row (a row sees itself), and each row run's first and last
    flags sit on the first and last steps that still hold it."""
    from ring_context_parallelism_amd.inputs import make_documents
    docs = make_documents(seq, 60, seed=seq)
    p = Plan(seq, cp, 1, 128, causal, layout)
    p.set_documents(docs)
    for r in range(cp):
        steps_of = {}
        for s in range(cp):
            segs = p.step_segments(r, s)
            for g in segs:
                qpos = oracle.rank_positions(seq, cp, r, layout)[g["q_start"]:g["q_start"] + g["q_len"]]
                kpos = oracle.rank_positions(seq, cp, oracle.ring_source(r, s, cp), layout)
                assert oracle.valid_mask(qpos, kpos, causal, doc_starts=docs).any(), (r, s, g)
                steps_of.setdefault(g["q_start"], []).append((s, g["first"], g["last"]))
        assert sum(g["q_len"] for g in p.step_segments(r, 0)) == p.rank_valid_rows(r)
        for run in steps_of.values():
            ss = [x[0] for x in run]
            for s, first, last in run:
                assert bool(first) == (s == min(ss)) and bool(last) == (s == max(ss))
    p.set_documents(None)
    q = Plan(seq, cp, 1, 128, causal, layout)
    for r in range(cp):
        for s in range(cp):
            assert p.step_segments(r, s) == q.step_segments(r, s)
