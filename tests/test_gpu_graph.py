"""Graph mode (CP_ATTN_OPT_GRAPH) through the C ABI.

A forward recorded into a HIP graph and replayed on the caller's stream must
give the eager result bit for bit: replay after replay, with eager kernels and
host synchronisation between replays, after the inputs change in place (a
replay reads the buffers' current contents), and after a change of output
buffer or of options makes the library record it again.
"""

import pytest
import torch

from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _bufs(plan, q, k, v):
    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((plan.heads, plan.seq_len), device=dev)
    return [qd, kd, vd, out, lse]


def _call(plan, b, rank):
    qd, kd, vd, out, lse = b
    # eager work between calls: refill the outputs with NaN and run an
    # unrelated kernel, then synchronise with the host
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    junk = torch.randn(1 << 16, device=qd.device)
    junk.mul_(3.0)
    if rank is None:
        plan.full_forward(qd, kd, vd, out, lse)
    else:
        plan.rank_forward(qd, kd, vd, out, lse, rank)
    torch.cuda.synchronize()
    return out.cpu().clone(), lse.cpu().clone()


def _same(a, b):
    (oa, la), (ob, lb) = a, b
    ints = {torch.bfloat16: torch.int16, torch.float32: torch.int32}
    return torch.equal(oa.view(ints[oa.dtype]), ob.view(ints[ob.dtype])) and torch.equal(
        la.view(torch.int32), lb.view(torch.int32))


def _rank_rows(plan, rank):
    """Mask of the token rows rank `rank` writes (its zigzag chunks)."""
    import oracle
    rows = torch.zeros(plan.seq_len, dtype=torch.bool)
    rows[torch.from_numpy(oracle.rank_positions(plan.seq_len, plan.cp_size, rank, "zigzag"))] = True
    return rows


@pytest.mark.parametrize("mode", ["default", "memcpy", "hybrid", "separate", "serial", "poison"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_graph_replays_match_eager(mode, dtype):
    seq, cp, heads, dim = 2048, 4, 2, 128
    rank = 1
    _say(f"graph mode={mode} {dtype} seq={seq} cp={cp} rank={rank}")
    q, k, v = make_qkv(seq, heads, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 31)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=dtype)
    p.set_fused_ring(False)  # graph mode records the one-launch-per-step schedule
    if mode in ("memcpy", "hybrid"):
        p.set_recv(mode)
    elif mode == "separate":
        p.set_merge(True)
    elif mode == "serial":
        p.set_serialize(True)
    elif mode == "poison":
        p.set_poison(True)
    b = _bufs(p, q, k, v)
    rows = _rank_rows(p, rank)

    def eager():
        p.set_graph(False)
        r = _call(p, b, rank)
        p.set_graph(True)
        return r

    ref = eager()
    assert torch.isfinite(ref[0][rows].float()).all()
    for i in range(3):
        got = _call(p, b, rank)
        assert _same(got, ref), f"replay {i} differs from the eager result"
    # new contents in the same buffers: the replay reads them
    q2, k2, v2 = make_qkv(seq, heads, dim, "bf16" if dtype == torch.bfloat16 else "fp32", 32)
    for dst, src in zip(b[:3], (q2, k2, v2)):
        dst.copy_(src.to(dst.device))
    torch.cuda.synchronize()
    ref2 = eager()
    assert not _same(ref2, ref)
    for i in range(2):
        assert _same(_call(p, b, rank), ref2), f"replay {i} after an in-place input change differs"
    # another output buffer: recorded again
    b[3] = torch.empty_like(b[3])
    assert _same(_call(p, b, rank), ref2)
    p.close()


def test_graph_full_forward_and_option_change():
    seq, cp, heads, dim = 1536, 3, 2, 128
    _say(f"graph full_forward seq={seq} cp={cp}")
    q, k, v = make_qkv(seq, heads, dim, "bf16", 33)
    p = Plan(seq, cp, heads, dim, True, "zigzag", dtype=torch.bfloat16)
    p.set_fused_ring(False)  # graph mode records the one-launch-per-step schedule
    b = _bufs(p, q, k, v)
    ref = _call(p, b, None)
    p.set_graph(True)
    for _ in range(3):
        assert _same(_call(p, b, None), ref)
    # an option change records the graph again (serial schedule, same result)
    p.set_serialize(True)
    assert _same(_call(p, b, None), ref)
    p.set_serialize(False)
    assert _same(_call(p, b, None), ref)
    # rank forwards of every rank under graph mode rebuild the full output
    out_r = torch.full_like(b[3], float("nan"))
    lse_r = torch.full_like(b[4], float("nan"))
    for r in range(cp):
        p.rank_forward(b[0], b[1], b[2], out_r, lse_r, r)
    torch.cuda.synchronize()
    assert _same((out_r.cpu(), lse_r.cpu()), ref)
    p.close()
