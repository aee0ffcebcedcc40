"""GPU parity of the backward (through the C ABI) against the fp64 oracle.

The GPU forward of the same plan supplies out and lse (as a training step
would); the oracle differentiates its own fp64 forward.  Tolerances, per
gradient tensor, relative to that tensor's largest reference magnitude:
bf16 inputs max|d| <= 2e-2 * max|ref|, fp32 inputs <= 1e-4 * max|ref|.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd.inputs import make_qkv, to_numpy_f64

pytestmark = pytest.mark.gpu

REL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def _dev():
    assert torch.cuda.is_available(), "no GPU"
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


def _inputs(seq, heads, dim, dtype, seed):
    kind = "bf16" if dtype == torch.bfloat16 else "fp32"
    q, k, v = make_qkv(seq, heads, dim, kind, seed)
    dout = make_qkv(seq, heads, dim, kind, seed + 1)[0]
    return q, k, v, dout


def _forward(p, qd, kd, vd):
    out = torch.empty_like(qd)
    lse = torch.empty((p.heads, p.seq_len), device=qd.device)
    p.full_forward(qd, kd, vd, out, lse)
    return out, lse


def _rel_err(got, ref, rows=None):
    g = got.double().cpu().numpy()
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.all(np.isfinite(g))
    return float(np.max(np.abs(g - ref)) / max(1e-30, np.max(np.abs(ref))))


CASES = [
    (1536, 2, "zigzag", True, 2, 128, torch.bfloat16),
    (1003, 4, "zigzag", True, 2, 128, torch.bfloat16),   # padded
    (768, 3, "contiguous", True, 2, 128, torch.bfloat16),
    (1024, 4, "zigzag", False, 2, 128, torch.bfloat16),
    (520, 2, "zigzag", True, 2, 64, torch.bfloat16),
    (256, 2, "zigzag", True, 2, 64, torch.float32),
    (299, 3, "contiguous", False, 2, 128, torch.float32),
    (21, 8, "zigzag", True, 1, 128, torch.bfloat16),     # ranks with no real row
]


def _ids(c):
    return f"s{c[0]}_cp{c[1]}_{c[2]}_{'causal' if c[3] else 'bidir'}_h{c[4]}_d{c[5]}_{str(c[6])[6:]}"


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_full_backward_matches_oracle(case):
    seq, cp, layout, causal, heads, dim, dtype = case
    _say(f"backward {_ids(case)}")
    q, k, v, dout = _inputs(seq, heads, dim, dtype, 91)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    dq, dk, dv = (torch.full((seq, heads, dim), float("nan"), device=dev) for _ in range(3))
    p.full_backward(qd, kd, vd, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(to_numpy_f64(t) for t in (q, k, v, dout)), causal=causal)
    errs = [_rel_err(g, r) for g, r in zip((dq, dk, dv), ref)]
    _say(f"  rel err dq={errs[0]:.2e} dk={errs[1]:.2e} dv={errs[2]:.2e}")
    assert max(errs) <= REL[dtype], errs
    p.close()


@pytest.mark.parametrize("layout", ["zigzag", "contiguous"])
def test_rank_backward_rows_and_travelling_terms(layout):
    """Each rank writes dq at its own rows only and adds exactly its terms to
    dk and dv (the oracle's per-rank contributions)."""
    seq, cp, heads, dim, dtype = 1024, 4, 2, 128, torch.bfloat16
    _say(f"rank backward {layout}")
    q, k, v, dout = _inputs(seq, heads, dim, dtype, 92)
    p = Plan(seq, cp, heads, dim, True, layout, dtype=dtype)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    qn, kn, vn, don = (to_numpy_f64(t) for t in (q, k, v, dout))
    for r in (0, cp - 1):
        dq = torch.full((seq, heads, dim), float("nan"), device=dev)
        dk = torch.zeros((seq, heads, dim), device=dev)
        dv = torch.zeros((seq, heads, dim), device=dev)
        p.rank_backward(qd, kd, vd, out, lse, dod, dq, dk, dv, r)
        torch.cuda.synchronize()
        rdq, rdk, rdv, pos = oracle.rank_backward(qn, kn, vn, don, cp, r, layout=layout, causal=True)
        others = np.setdiff1d(np.arange(seq), pos)
        assert torch.isnan(dq.cpu()[others]).all()
        full = np.zeros((seq, heads, dim))
        full[pos] = rdq
        assert _rel_err(dq, full, rows=pos) <= REL[dtype]
        for g, rf in ((dk, rdk), (dv, rdv)):
            assert _rel_err(g, rf) <= REL[dtype]
            untouched = np.all(rf == 0, axis=(1, 2))  # sources this rank never sees
            assert torch.all(g.cpu()[torch.from_numpy(untouched)] == 0)
    p.close()


def test_backward_is_deterministic():
    """No atomics: two runs give the same bits."""
    seq, cp, heads, dim = 1536, 3, 2, 128
    _say("backward determinism")
    q, k, v, dout = _inputs(seq, heads, dim, torch.bfloat16, 93)
    p = Plan(seq, cp, heads, dim, True, "zigzag")
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    runs = []
    for _ in range(2):
        g = [torch.empty((seq, heads, dim), device=dev) for _ in range(3)]
        p.full_backward(qd, kd, vd, out, lse, dod, *g)
        torch.cuda.synchronize()
        runs.append([t.cpu() for t in g])
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    p.close()


KEY_KERNEL_CASES = [c for c in CASES if c[6] == torch.bfloat16 and c[5] == 128]


def _backward_with(p, kind, qd, kd, vd, out, lse, dod):
    p.set_backward_key_kernel(kind)
    g = [torch.full(qd.shape, float("nan"), dtype=torch.float32, device=qd.device) for _ in range(3)]
    p.full_backward(qd, kd, vd, out, lse, dod, *g)
    torch.cuda.synchronize()
    return [t.cpu() for t in g]


def _assert_same_bits(a, b, what):
    for name, x, y in zip(("dq", "dk", "dv"), a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (what, name)


@pytest.mark.parametrize("case", KEY_KERNEL_CASES, ids=[_ids(c) for c in KEY_KERNEL_CASES])
def test_eight_wave_key_kernel_matches_four_wave_bits(case):
    """The eight-wave dK/dV kernel issues the same products in the same order
    per key as the four-wave one: every gradient bit-identical."""
    seq, cp, layout, causal, heads, dim, dtype = case
    _say(f"key-major kernels, same bits: {_ids(case)}")
    q, k, v, dout = _inputs(seq, heads, dim, dtype, 94)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    four = _backward_with(p, "four", qd, kd, vd, out, lse, dod)
    eight = _backward_with(p, "eight", qd, kd, vd, out, lse, dod)
    _assert_same_bits(four, eight, _ids(case))
    p.close()


def test_eight_wave_key_kernel_documents_and_full_size_bits():
    """Same check with document masks (boundaries inside and on the edges of
    64-row tiles) and on the 32k-token, cp 8 workload (32 heads x 128)."""
    from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv
    dev = _dev()
    seq, cp, heads, dim = 1536, 2, 2, 128
    _say("key-major kernels, same bits: documents s1536 cp2")
    q, k, v, dout = _inputs(seq, heads, dim, torch.bfloat16, 95)
    p = Plan(seq, cp, heads, dim, True, "zigzag")
    p.set_documents([0, 1, 2, 64, 128, 129, 500, 777, 1535])
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    _assert_same_bits(_backward_with(p, "four", qd, kd, vd, out, lse, dod),
                      _backward_with(p, "eight", qd, kd, vd, out, lse, dod), "documents")
    p.close()
    w = WORKLOADS["causal_s32768_cp8_zigzag_h32_d128_bf16_rank0"]
    _say(f"key-major kernels, same bits: {w.name}")
    q, k, v = workload_qkv(w)
    dout = make_qkv(w.seq_len, w.heads, w.head_dim, "bf16", w.seed + 7)[0]
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, True, w.layout)
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    _assert_same_bits(_backward_with(p, "four", qd, kd, vd, out, lse, dod),
                      _backward_with(p, "eight", qd, kd, vd, out, lse, dod), w.name)
    p.close()


def test_full_size_backward_sampled_rows_and_gradient_sums():
    """The 32k-token, cp 8 zigzag workload (32 heads x 128, bf16): dQ of sampled
    rows against the oracle, and two properties of the complete key/value
    gradients that hold at any size: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0."""
    from ring_context_parallelism_amd.inputs import WORKLOADS, workload_qkv
    w = WORKLOADS["causal_s32768_cp8_zigzag_h32_d128_bf16_rank0"]
    _say(f"full-size backward {w.name}")
    q, k, v = workload_qkv(w)
    dout = make_qkv(w.seq_len, w.heads, w.head_dim, "bf16", w.seed + 7)[0]
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, True, w.layout)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    dq, dk, dv = (torch.empty((w.seq_len, w.heads, w.head_dim), device=dev) for _ in range(3))
    p.full_backward(qd, kd, vd, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 2048, 9000, 16383, 16384, 30000, 32767])
    ref = oracle.query_gradients(*(to_numpy_f64(t) for t in (q, k, v, dout)), rows, causal=True)
    rel = float(np.max(np.abs(dq.cpu().double().numpy()[rows] - ref)) / np.max(np.abs(ref)))
    _say(f"  sampled dq rel err {rel:.2e}")
    assert rel <= REL[torch.bfloat16]
    sdv = dv.double().sum(dim=0).cpu()
    sdo = dod.double().sum(dim=0).cpu()
    assert float((sdv - sdo).abs().max()) <= 1e-2 * float(sdo.abs().max())
    sdk = dk.double().sum(dim=0).abs().max().cpu()
    adk = dk.double().abs().sum(dim=0).max().cpu()
    _say(f"  |sum dV - sum dO| {float((sdv - sdo).abs().max()):.3e}  |sum dK| {float(sdk):.3e} of {float(adk):.3e}")
    assert float(sdk) <= 1e-2 * float(adk)
    p.close()


# Document masks ("Context Parallelism for Long-Context Training", section
# "Prove attention equivalence": causal and document masks): single-token
# documents, boundaries on 64- and 128-token tile edges and inside chunks.
DOC_CASES = [
    (1536, 2, "zigzag", True, 2, 128, torch.bfloat16, [0, 1, 2, 64, 128, 129, 500, 777, 1535]),
    (1003, 4, "zigzag", True, 2, 128, torch.bfloat16, [0, 100, 101, 383, 640]),
    (1024, 4, "zigzag", False, 2, 128, torch.bfloat16, [0, 256, 300, 900]),
    (768, 3, "contiguous", True, 2, 128, torch.bfloat16, [0, 5, 260, 511, 512]),
    (520, 2, "zigzag", True, 2, 64, torch.bfloat16, [0, 33, 130, 131]),
    (256, 2, "zigzag", True, 2, 64, torch.float32, [0, 1, 64, 100, 200]),
    (299, 3, "contiguous", False, 2, 128, torch.float32, [0, 50, 51, 250]),
]


@pytest.mark.parametrize("case", DOC_CASES, ids=[_ids(c[:7]) for c in DOC_CASES])
def test_full_backward_with_documents_matches_oracle(case):
    seq, cp, layout, causal, heads, dim, dtype, docs = case
    _say(f"backward with documents {_ids(case[:7])} {docs}")
    q, k, v, dout = _inputs(seq, heads, dim, dtype, 93)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    p.set_documents(docs)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    dq, dk, dv = (torch.full((seq, heads, dim), float("nan"), device=dev) for _ in range(3))
    p.full_backward(qd, kd, vd, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(*(to_numpy_f64(t) for t in (q, k, v, dout)), causal=causal, doc_starts=docs)
    errs = [_rel_err(g, r) for g, r in zip((dq, dk, dv), ref)]
    _say(f"  rel err dq={errs[0]:.2e} dk={errs[1]:.2e} dv={errs[2]:.2e}")
    assert max(errs) <= REL[dtype], errs
    p.close()


def test_full_size_backward_with_documents_sampled_rows():
    """The 32k-token, cp 8 zigzag workload with seeded documents (mean length
    2048): dQ of sampled rows against the oracle's document gradients, and the
    per-document closed form sum_j dV_j = sum_i dO_i over each document."""
    from ring_context_parallelism_amd.inputs import WORKLOADS, make_documents, workload_qkv
    w = WORKLOADS["causal_s32768_cp8_zigzag_h32_d128_bf16_rank0"]
    docs = make_documents(w.seq_len, 2048, seed=w.seed + 11)
    _say(f"full-size backward with {len(docs)} documents {w.name}")
    q, k, v = workload_qkv(w)
    dout = make_qkv(w.seq_len, w.heads, w.head_dim, "bf16", w.seed + 7)[0]
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, True, w.layout)
    p.set_documents(docs)
    dev = _dev()
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, dout))
    out, lse = _forward(p, qd, kd, vd)
    dq, dk, dv = (torch.empty((w.seq_len, w.heads, w.head_dim), device=dev) for _ in range(3))
    p.full_backward(qd, kd, vd, out, lse, dod, dq, dk, dv)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 2047, 2048, 16383, 16384, 32767} | {d for d in docs[1:4]} | {docs[-1] - 1}))
    ref = oracle.query_gradients(*(to_numpy_f64(t) for t in (q, k, v, dout)), rows, causal=True, doc_starts=docs)
    rel = float(np.max(np.abs(dq.cpu().double().numpy()[rows] - ref)) / np.max(np.abs(ref)))
    _say(f"  sampled dq rel err {rel:.2e}")
    assert rel <= REL[torch.bfloat16]
    bounds = list(docs) + [w.seq_len]
    dv64, do64 = dv.double().cpu(), dod.double().cpu()
    for a, b in list(zip(bounds[:-1], bounds[1:]))[:6]:
        sdv, sdo = dv64[a:b].sum(dim=0), do64[a:b].sum(dim=0)
        assert float((sdv - sdo).abs().max()) <= 1e-2 * max(1.0, float(sdo.abs().max())), (a, b)
    p.close()
