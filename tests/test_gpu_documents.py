"""GPU parity of document masks ("Context Parallelism for Long-Context
Training", section "Prove attention equivalence": causal and document masks)
against the fp64 oracle, through the C ABI.

A query attends only to keys of its own document, on top of the causal or
bidirectional mask.  Tolerances as in the other parity tests: fp32 inputs
max|dO|, max|dLSE| <= 1e-5; bf16 inputs max|dO| <= 2e-2, max|dLSE| <= 1e-3.
Document lists mix single-token documents, boundaries on 64- and 256-token
tile edges and boundaries inside chunks, so ring steps hold rows that see no
key at all (their partial is left out of the merge).
"""

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd.inputs import make_documents, make_qkv, to_numpy_f64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (2e-2, 1e-3)}


def _dev():
    assert torch.cuda.is_available(), "no GPU"
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _bufs(p, q, k, v):
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((p.heads, p.seq_len), float("nan"), device=dev)
    return qd, kd, vd, out, lse


def _full(p, q, k, v):
    qd, kd, vd, out, lse = _bufs(p, q, k, v)
    p.full_forward(qd, kd, vd, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(out, lse, q, k, v, causal, docs, dtype, rows=None):
    qn, kn, vn = (to_numpy_f64(t) for t in (q, k, v))
    rows = np.arange(qn.shape[0]) if rows is None else np.asarray(rows)
    o_ref, l_ref = oracle.attention(qn[rows], kn, vn, causal=causal, q_pos=rows, doc_starts=docs)
    o_got = out[rows].to(torch.float64).numpy()
    l_got = lse[:, rows].to(torch.float64).numpy()
    assert np.all(np.isfinite(o_got)) and np.all(np.isfinite(l_got))
    d_o = float(np.max(np.abs(o_got - o_ref)))
    d_l = float(np.max(np.abs(l_got - l_ref)))
    tol_o, tol_l = TOL[dtype]
    assert d_o <= tol_o and d_l <= tol_l, (d_o, d_l)
    return d_o, d_l


def _docs(kind, seq):
    if kind == "edges":  # single tokens, tile edges, a boundary inside every chunk
        d = {0, 1, 2, 3, 64, 65, 255, 256, 257, 511, 512, seq // 3, seq // 2 + 7, seq - 1}
        return sorted(x for x in d if x < seq)
    return make_documents(seq, int(kind), seed=seq)


CASES = [
    # seq, cp, layout, causal, heads, dim, dtype, docs
    (256, 2, "zigzag", True, 2, 64, torch.float32, "edges"),
    (1000, 3, "contiguous", True, 2, 128, torch.float32, "90"),
    (384, 3, "zigzag", False, 2, 64, torch.float32, "40"),
    (4096, 4, "zigzag", True, 2, 128, torch.bfloat16, "edges"),
    (4096, 4, "zigzag", True, 2, 128, torch.bfloat16, "300"),
    (4096, 4, "contiguous", True, 3, 128, torch.bfloat16, "700"),
    (2048, 4, "zigzag", False, 2, 128, torch.bfloat16, "200"),
    (4099, 8, "zigzag", True, 2, 128, torch.bfloat16, "150"),
    (2048, 2, "zigzag", True, 2, 64, torch.bfloat16, "edges"),
    (1536, 3, "contiguous", False, 2, 64, torch.bfloat16, "100"),
]


@pytest.mark.parametrize("seq,cp,layout,causal,heads,dim,dtype,docs", CASES)
def test_full_forward_with_documents_matches_oracle(seq, cp, layout, causal, heads, dim, dtype, docs):
    _say(f"documents full_forward seq={seq} cp={cp} {layout} causal={causal} h={heads} d={dim} {dtype} {docs}")
    docs = _docs(docs, seq)
    q, k, v = make_qkv(seq, heads, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 77)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    p.set_documents(docs)
    out, lse = _full(p, q, k, v)
    _check(out, lse, q, k, v, causal, docs, dtype)
    p.close()


@pytest.mark.parametrize("mode", ["default", "memcpy", "fused", "hybrid", "separate", "serial"])
def test_rank_forward_schedule_modes_with_documents(mode):
    seq, cp, heads, dim = 4096, 4, 2, 128
    _say(f"documents rank_forward mode={mode}")
    docs = _docs("edges", seq)
    q, k, v = make_qkv(seq, heads, dim, "bf16", 78)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    p.set_documents(docs)
    if mode in ("memcpy", "fused", "hybrid"):
        p.set_recv(mode)
    elif mode == "separate":
        p.set_merge(True)
    elif mode == "serial":
        p.set_serialize(True)
    p.set_poison(True)  # consumed slots and partials become NaN: stale reads would show
    qd, kd, vd, out, lse = _bufs(p, q, k, v)
    for r in range(cp):
        p.rank_forward(qd, kd, vd, out, lse, r)
    torch.cuda.synchronize()
    _check(out.cpu(), lse.cpu(), q, k, v, True, docs, torch.bfloat16)
    p.close()


def test_one_document_is_bit_identical_to_no_documents():
    """A single document masks nothing: the document-mask kernels then compute
    exactly what the plain kernels do (the key split is off in both)."""
    seq, cp, heads, dim = 4096, 4, 2, 128
    _say("documents: one document vs none")
    q, k, v = make_qkv(seq, heads, dim, "bf16", 79)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    p.set_key_split(False)
    p.set_fused_ring(False)  # documents run one launch per step: compare with that
    ref = _full(p, q, k, v)
    p.set_documents([0])
    got = _full(p, q, k, v)
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    p.set_documents(None)
    assert all(torch.equal(a, b) for a, b in zip(_full(p, q, k, v), ref))
    p.close()


def test_documents_change_the_result_and_can_be_replaced():
    """Masking across documents changes the rows after the first boundary; a
    new list takes effect on the next call."""
    seq, cp, heads, dim = 2048, 2, 2, 128
    _say("documents: effect and replacement")
    q, k, v = make_qkv(seq, heads, dim, "bf16", 80)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    plain = _full(p, q, k, v)
    for docs in ([0, 700], [0, 100, 1500], [0, 1024, 1025]):
        p.set_documents(docs)
        out, lse = _full(p, q, k, v)
        _check(out, lse, q, k, v, True, docs, torch.bfloat16)
        b = docs[1]
        assert float((lse[:, b + 1:] - plain[1][:, b + 1:]).abs().min()) > 1e-3  # fewer keys: a smaller LSE
    p.close()


@pytest.mark.parametrize("layout,causal,dtype", [("zigzag", True, torch.bfloat16), ("contiguous", False, torch.bfloat16),
                                                 ("zigzag", True, torch.float32)])
def test_allgather_with_documents_matches_oracle(layout, causal, dtype):
    seq, cp, heads, dim = 2048, 4, 2, 128
    _say(f"documents allgather {layout} causal={causal} {dtype}")
    docs = _docs("edges", seq)
    q, k, v = make_qkv(seq, heads, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 81)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    p.set_documents(docs)
    qd, kd, vd, out, lse = _bufs(p, q, k, v)
    for r in range(cp):
        p.allgather_forward(qd, kd, vd, out, lse, r)
    torch.cuda.synchronize()
    _check(out.cpu(), lse.cpu(), q, k, v, causal, docs, dtype)
    p.close()


@pytest.mark.parametrize("causal", [True, False])
def test_ulysses_forward_with_documents_matches_oracle(causal):
    seq, cp, heads, dim = 2048, 2, 4, 128
    _say(f"documents ulysses causal={causal}")
    docs = _docs("300", seq)
    q, k, v = make_qkv(seq, heads, dim, "bf16", 82)
    p = Plan(seq, cp, heads, dim, causal, "zigzag", dtype=torch.bfloat16)
    p.set_documents(docs)
    dev = _dev()
    g = heads // cp
    out = torch.full((seq, heads, dim), float("nan"), dtype=torch.bfloat16)
    lse = torch.full((heads, seq), float("nan"))
    for r in range(cp):
        sl = slice(r * g, (r + 1) * g)
        qd, kd, vd = (t[:, sl].contiguous().to(dev) for t in (q, k, v))
        o = torch.empty_like(qd)
        l = torch.empty((g, seq), device=dev)
        p.ulysses_forward(qd, kd, vd, o, l)
        torch.cuda.synchronize()
        out[:, sl] = o.cpu()
        lse[sl] = l.cpu()
    _check(out, lse, q, k, v, causal, docs, torch.bfloat16)
    p.close()


def test_graph_mode_with_documents():
    """Graph replays equal the eager result; a new document list records again."""
    seq, cp, heads, dim = 2048, 4, 2, 128
    _say("documents graph mode")
    q, k, v = make_qkv(seq, heads, dim, "bf16", 83)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    b = _bufs(p, q, k, v)

    def call():
        b[3].fill_(float("nan"))
        b[4].fill_(float("nan"))
        p.full_forward(*b)
        torch.cuda.synchronize()
        return b[3].cpu(), b[4].cpu()

    for docs in ([0, 300, 301, 1200], [0, 64, 512]):
        p.set_documents(docs)
        p.set_graph(False)
        ref = call()
        _check(ref[0], ref[1], q, k, v, True, docs, torch.bfloat16)
        p.set_graph(True)
        for _ in range(3):
            got = call()
            assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    p.close()


def test_padding_invariance_with_documents():
    """Awkward length with documents: the real rows equal those of the longer
    divisible sequence (its extra tokens close the last document, so causal
    real rows never see them), bit for bit."""
    seq, cp, heads, dim = 1003, 4, 2, 128
    _say("documents padding invariance")
    docs = [0, 200, 201, 640]
    q, k, v = make_qkv(1008, heads, dim, "bf16", 84)
    long = Plan(1008, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    long.set_documents(docs)
    ref = _full(long, q, k, v)
    short = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    short.set_documents(docs)
    got = _full(short, *(t[:seq].contiguous() for t in (q, k, v)))
    assert torch.equal(got[0], ref[0][:seq]) and torch.equal(got[1], ref[1][:, :seq])
    _check(got[0], got[1], *(t[:seq] for t in (q, k, v)), True, docs, torch.bfloat16)
    long.close()
    short.close()


def test_full_size_rank0_with_documents_sampled_rows():
    """The bench's workload and launch configuration (32k tokens, cp 8,
    zigzag, 32 heads x 128, bf16, rank 0's share, default schedule) with seeded
    documents: sampled rows of the share against the oracle."""
    from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv
    w = WORKLOADS["causal_s32768_cp8_zigzag_h32_d128_bf16_rank0"]
    q, k, v = workload_qkv(w)
    rows = oracle.rank_positions(w.seq_len, w.cp, w.rank, w.layout)
    sample = rows[np.linspace(0, rows.size - 1, 16).astype(np.int64)]
    for mean in (8192, 1024):
        docs = make_documents(w.seq_len, mean, seed=w.seed + mean)
        _say(f"documents full size: {len(docs)} documents (mean {mean})")
        p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, True, w.layout, dtype=torch.bfloat16)
        p.set_documents(docs)
        qd, kd, vd, out, lse = _bufs(p, q, k, v)
        p.rank_forward(qd, kd, vd, out, lse, w.rank)
        torch.cuda.synchronize()
        out_c, lse_c = out.cpu(), lse.cpu()
        _check(out_c, lse_c, q, k, v, True, docs, torch.bfloat16, rows=sample)
        # the rank writes only its own rows
        others = np.setdiff1d(np.arange(w.seq_len), rows)[::997]
        assert torch.isnan(out_c[others].float()).all() and torch.isnan(lse_c[:, others]).all()
        p.close()
