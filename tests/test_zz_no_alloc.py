"""The no-allocation forward (cp_attn_rank_forward_noalloc) against the
ordinary one (cp_attn_rank_forward), through the C ABI.

Both run the same kernels on the same ring schedule; the no-allocation call
keeps its workspace in the library's static device array and runs every
kernel on the caller's stream, so its output must equal the ordinary call's
bit for bit, and both stay within the bf16 / fp32 tolerances of the fp64
oracle on sampled rows.  Two calls in a row, the second on a smaller plan,
check that the array's stale contents from a larger call do not leak.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd import _native as N
from ring_context_parallelism_amd.inputs import make_qkv, to_numpy_f64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (2e-2, 1e-3)}


def _say(msg):
    print(msg, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _both(seq, cp, layout, causal, heads, dim, dtype, rank, seed):
    """(ordinary, no-allocation) outputs of one rank's share, and the inputs."""
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(seq, heads, dim, "bf16" if dtype == torch.bfloat16 else "fp32", seed)
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    p.set_fused_ring(False)  # the no-allocation call runs one launch per step
    res = []
    for fn in (p.rank_forward, p.rank_forward_noalloc):
        out = torch.full_like(qd, float("nan"))
        lse = torch.full((heads, seq), float("nan"), device=dev)
        fn(qd, kd, vd, out, lse, rank)
        torch.cuda.synchronize()
        res.append((out.cpu(), lse.cpu()))
    p.close()
    return res, (q, k, v)


@pytest.mark.parametrize("cases", [
    # bf16 head_dim 128: the receive runs inside the step kernels; 8 heads at
    # 8192 tokens split the keys of the C x 2C steps (split counters in use)
    [(8192, 4, "zigzag", True, 8, 128, torch.bfloat16, 1, 71),
     (3000, 3, "contiguous", True, 4, 128, torch.bfloat16, 2, 72)],
    # fp32 head_dim 64: the receive is a copy kernel on the caller's stream
    [(1024, 4, "zigzag", True, 2, 64, torch.float32, 3, 73),
     (300, 2, "zigzag", False, 2, 64, torch.float32, 0, 74)],
])
def test_noalloc_equals_rank_forward_two_calls(cases):
    for seq, cp, layout, causal, heads, dim, dtype, rank, seed in cases:
        _say(f"noalloc seq={seq} cp={cp} {layout} causal={causal} H={heads} D={dim} {dtype} rank={rank}")
        (ref, got), (q, k, v) = _both(seq, cp, layout, causal, heads, dim, dtype, rank, seed)
        rows = oracle.rank_positions(seq, cp, rank, layout)
        rows_t = torch.from_numpy(rows)
        assert torch.equal(_bits(got[0][rows_t]), _bits(ref[0][rows_t]))
        assert torch.equal(_bits(got[1][:, rows_t]), _bits(ref[1][:, rows_t]))
        others = np.setdiff1d(np.arange(seq), rows)
        assert torch.isnan(got[0][torch.from_numpy(others)].float()).all()
        sub = rows[np.linspace(0, rows.size - 1, 24).astype(np.int64)]
        tol_o, tol_l = TOL[dtype]
        for h in sorted({0, heads - 1}):
            o_ref, l_ref = oracle.attention(to_numpy_f64(q[torch.from_numpy(sub), h:h + 1]), to_numpy_f64(k[:, h:h + 1]),
                                            to_numpy_f64(v[:, h:h + 1]), causal=causal, q_pos=sub)
            d_o = float(np.max(np.abs(got[0][torch.from_numpy(sub), h:h + 1].double().numpy() - o_ref)))
            d_l = float(np.max(np.abs(got[1][h, torch.from_numpy(sub)].double().numpy() - l_ref[0])))
            _say(f"  head {h}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
            assert d_o <= tol_o and d_l <= tol_l


def test_noalloc_rejects_what_it_cannot_hold():
    """A plan whose workspace exceeds the static array, and document masks,
    are refused before anything is enqueued."""
    dev = torch.device("cuda:0")
    seq, cp, heads, dim = 32768, 8, 32, 128
    p = Plan(seq, cp, heads, dim, True, "zigzag")
    assert p.workspace_bytes() > N.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((seq, heads, dim), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((heads, seq), device=dev)
    with pytest.raises(N.CpAttnError) as e:
        p.rank_forward_noalloc(q, q, q, q, lse, 0)
    assert e.value.status == N.ENOWORKSPACE
    p.close()
    p = Plan(1024, 2, 2, 128, True, "zigzag")
    p.set_documents([0, 100, 700])
    q = torch.zeros((1024, 2, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.zeros((2, 1024), device=dev)
    with pytest.raises(N.CpAttnError) as e:
        p.rank_forward_noalloc(q, q, q, q, lse, 0)
    assert e.value.status == N.EUNSUPPORTED
    p.close()


def test_noalloc_graph_capture_replays():
    """The call enqueues kernels only, on the caller's stream: captured into a
    HIP graph and replayed three times, with eager work and host
    synchronisation between replays, every replay equals the eager call."""
    dev = torch.device("cuda:0")
    seq, cp, heads, dim, rank = 4096, 4, 4, 128, 2
    q, k, v = (t.to(dev) for t in make_qkv(seq, heads, dim, "bf16", 75))
    p = Plan(seq, cp, heads, dim, True, "zigzag")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((heads, seq), float("nan"), device=dev)
    p.rank_forward_noalloc(q, k, v, out, lse, rank)
    torch.cuda.synchronize()
    want_o, want_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            p.rank_forward_noalloc(q, k, v, out, lse, rank, stream=s)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=dev).sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(_bits(out), _bits(want_o)), i
        assert torch.equal(_bits(lse), _bits(want_l)), i
    del g
    p.close()
