"""Lockstep full forward (CP_ATTN_OPT_LOCKSTEP): every rank's ring step s in
one launch, every rank's receive of step s + 1 on the copy stream.  Each
rank runs the same kernel on the same inputs as when the ranks run back to
back, so with the key split off there (lockstep never splits) the outputs
agree bit for bit; one case is also checked against the fp64 oracle.
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


def _full(p, qd, kd, vd):
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((p.heads, p.seq_len), float("nan"), device=qd.device)
    p.full_forward(qd, kd, vd, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _same(a, b):
    return torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                       b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32))


def _both(p, qd, kd, vd):
    p.set_key_split(False)
    p.set_fused_ring(False)  # lockstep launches each step: compare with one launch per step
    p.set_lockstep(False)
    ref = _full(p, qd, kd, vd)
    p.set_lockstep(True)
    got = _full(p, qd, kd, vd)
    return ref, got


CASES = [
    (2048, 4, "zigzag", True, 4),
    (1003, 4, "zigzag", True, 2),      # padded
    (768, 3, "contiguous", True, 2),
    (1024, 4, "zigzag", False, 2),     # bidirectional
    (21, 8, "zigzag", True, 1),        # ranks with no real row
    (4096, 8, "zigzag", True, 3),      # heads not a multiple of 8
]


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}_cp{c[1]}_{c[2]}_{'causal' if c[3] else 'bidir'}_h{c[4]}"
                                             for c in CASES])
def test_lockstep_matches_back_to_back_bits(case):
    seq, cp, layout, causal, heads = case
    _say(f"lockstep vs back to back: {case}")
    q, k, v = make_qkv(seq, heads, 128, "bf16", 71)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, causal, layout)
    (o_ref, l_ref), (o, l) = _both(p, qd, kd, vd)
    assert _same(o, o_ref) and _same(l, l_ref), case
    p.close()


def test_lockstep_repeated_calls_new_buffers_memcpy_receive_documents_counters():
    """The step table is built once per buffer set: a second call reuses it,
    new output buffers rebuild it; the memcpy receive, document masks and the
    work counters give the back-to-back results."""
    seq, cp, heads = 1536, 4, 2
    q, k, v = make_qkv(seq, heads, 128, "bf16", 72)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, 128, True, "zigzag")
    p.set_key_split(False)
    p.set_fused_ring(False)
    ref = _full(p, qd, kd, vd)
    p.set_lockstep(True)
    _say("lockstep: repeated calls and new buffers")
    for _ in range(3):
        o, l = _full(p, qd, kd, vd)  # new out/lse tensors each call
        assert _same(o, ref[0]) and _same(l, ref[1])
    out = torch.empty_like(qd)
    lse = torch.empty((heads, seq), device=dev)
    for _ in range(2):  # same buffers: the uploaded table is reused
        out.fill_(float("nan"))
        p.full_forward(qd, kd, vd, out, lse)
        torch.cuda.synchronize()
        assert _same(out.cpu(), ref[0]) and _same(lse.cpu(), ref[1])
    _say("lockstep: memcpy receive")
    p.set_recv("memcpy")
    o, l = _full(p, qd, kd, vd)
    assert _same(o, ref[0]) and _same(l, ref[1])
    p.set_recv("kernel")
    _say("lockstep: documents")
    p.set_documents([0, 1, 2, 64, 300, 301, 777, 1200])
    p.set_lockstep(False)
    dref = _full(p, qd, kd, vd)
    p.set_lockstep(True)
    o, l = _full(p, qd, kd, vd)
    assert _same(o, dref[0]) and _same(l, dref[1])
    p.set_documents(None)
    _say("lockstep: work counters")
    p.set_counters(True)
    o, l = _full(p, qd, kd, vd)
    assert _same(o, ref[0]) and _same(l, ref[1])
    counts, (tr, tk) = p.last_tile_counts()
    for r in range(cp):
        for s in range(cp):
            assert counts[r][s] == heads * p.valid_work(r, s, tr, tk)[0], (r, s)
    p.close()


def test_lockstep_full_size_and_oracle():
    """The 8192-token, cp 4, 32-head workload: lockstep equals back to back bit
    for bit, and the first and last head match the fp64 oracle on every row."""
    w = WORKLOADS["causal_s8192_cp4_zigzag_h32_d128_bf16"]
    _say(f"lockstep, full size: {w.name}")
    q, k, v = workload_qkv(w)
    dev = _dev()
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(w.seq_len, w.cp, w.heads, w.head_dim, w.causal, w.layout)
    (o_ref, l_ref), (o, l) = _both(p, qd, kd, vd)
    assert _same(o, o_ref) and _same(l, l_ref)
    p.close()
    qn, kn, vn = (to_numpy_f64(t) for t in (q, k, v))
    rows = np.arange(w.seq_len)
    d_o = d_l = 0.0
    for h in (0, w.heads - 1):
        o_r, l_r = oracle.attention(qn[:, h:h + 1], kn[:, h:h + 1], vn[:, h:h + 1], causal=True, q_pos=rows)
        d_o = max(d_o, float(np.max(np.abs(o[:, h:h + 1].double().numpy() - o_r))))
        d_l = max(d_l, float(np.max(np.abs(l[h].double().numpy() - l_r[0]))))
    _say(f"  max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= 2e-2 and d_l <= 1e-3


def test_lockstep_falls_back_where_not_served():
    """fp32 plans, head_dim 64, the separate merge and the serial mode run the
    ranks back to back with the option set: same bits as without it."""
    dev = _dev()
    for dim, dtype, setup in ((128, torch.float32, None), (64, torch.bfloat16, None),
                              (128, torch.bfloat16, "merge"), (128, torch.bfloat16, "serial")):
        _say(f"lockstep fallback: d{dim} {dtype} {setup}")
        q, k, v = make_qkv(512, 2, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 73)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        p = Plan(512, 4, 2, dim, True, "zigzag", dtype=dtype)
        if setup == "merge":
            p.set_merge(True)
        if setup == "serial":
            p.set_serialize(True)
        (o_ref, l_ref), (o, l) = _both(p, qd, kd, vd)
        assert _same(o, o_ref) and _same(l, l_ref)
        p.close()
