"""GPU parity of the Ulysses variant (all-to-all to head ownership, attention
over every token of a head slice, all-to-all back) against the fp64 oracle.
Tolerances as in the other parity tests: bf16 max|dO| <= 2e-2, max|dLSE| <=
1e-3; fp32 1e-5 for both.  The all-to-all itself is a copy: bit-exact."""

import numpy as np
import pytest
import torch

import oracle
from ring_context_parallelism_amd import Plan
from ring_context_parallelism_amd.inputs import make_qkv, to_numpy_f64

pytestmark = pytest.mark.gpu

TOL = {torch.float32: (1e-5, 1e-5), torch.bfloat16: (2e-2, 1e-3)}


def _dev():
    assert torch.cuda.is_available(), "no GPU"
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("dtype,layout,seq,cp,heads", [(torch.bfloat16, "zigzag", 1024, 4, 8),
                                                       (torch.float32, "contiguous", 999, 3, 6),
                                                       (torch.bfloat16, "zigzag", 1003, 4, 4)])
def test_a2a_bit_exact_against_oracle_layouts(dtype, layout, seq, cp, heads):
    _say(f"ulysses a2a {dtype} {layout} seq={seq} cp={cp} heads={heads}")
    dev = _dev()
    dim = 64
    p = Plan(seq, cp, heads, dim, True, layout, dtype=dtype)
    x = torch.randn(seq, heads, dim).to(dtype)
    xd = x.to(dev)
    seq_l = torch.empty((cp * p.local_rows(), heads, dim), device=dev, dtype=dtype)
    p.layout_gather(xd, seq_l)
    hs = torch.full((cp, seq, heads // cp, dim), float("nan"), device=dev, dtype=dtype)
    p.ulysses_a2a(seq_l, hs, True)
    torch.cuda.synchronize()
    xn = x.float().numpy()
    assert np.array_equal(hs.cpu().float().numpy(), oracle.head_shards(xn, cp))
    back = torch.full_like(seq_l, float("nan"))
    p.ulysses_a2a(hs, back, False)
    torch.cuda.synchronize()
    want = oracle.sequence_shards(xn, cp, layout)
    got = back.cpu().float().numpy().reshape(want.shape)
    for r in range(cp):
        n = p.rank_valid_rows(r)
        assert np.array_equal(got[r, :n], want[r, :n])
        assert np.all(np.isnan(got[r, n:]))  # pad rows are not written
    p.close()


CASES = [(8192, 4, "zigzag", True, 8, 128, torch.bfloat16),
         (1003, 4, "zigzag", True, 4, 128, torch.bfloat16),
         (4096, 2, "contiguous", False, 4, 64, torch.bfloat16),
         (512, 2, "zigzag", True, 2, 64, torch.float32)]


@pytest.mark.parametrize("case", CASES)
def test_ulysses_pipeline_matches_oracle(case):
    """natural -> sequence layout -> a2a -> per-rank attention -> a2a back ->
    natural, against unsplit attention on every row and head."""
    seq, cp, layout, causal, heads, dim, dtype = case
    _say(f"ulysses pipeline {case}")
    dev = _dev()
    kind = "bf16" if dtype == torch.bfloat16 else "fp32"
    q, k, v = make_qkv(seq, heads, dim, kind, 95)
    p = Plan(seq, cp, heads, dim, causal, layout, dtype=dtype)
    g = heads // cp
    n_seq = cp * p.local_rows()
    hs = []
    for t in (q, k, v):
        s_l = torch.empty((n_seq, heads, dim), device=dev, dtype=dtype)
        p.layout_gather(t.to(dev), s_l)
        h_l = torch.empty((cp, seq, g, dim), device=dev, dtype=dtype)
        p.ulysses_a2a(s_l, h_l, True)
        hs.append(h_l)
    out_h = torch.empty((cp, seq, g, dim), device=dev, dtype=dtype)
    lse = torch.empty((heads, seq), device=dev)
    for r in range(cp):
        p.ulysses_forward(hs[0][r], hs[1][r], hs[2][r], out_h[r], lse[r * g:(r + 1) * g])
    out_s = torch.zeros((n_seq, heads, dim), device=dev, dtype=dtype)
    p.ulysses_a2a(out_h, out_s, False)
    out = torch.empty((seq, heads, dim), device=dev, dtype=dtype)
    p.layout_scatter(out_s, out)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(*(to_numpy_f64(t) for t in (q, k, v)), causal=causal)
    d_o = float(np.max(np.abs(out.cpu().double().numpy() - o_ref)))
    d_l = float(np.max(np.abs(lse.cpu().double().numpy() - l_ref)))
    _say(f"  max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    tol_o, tol_l = TOL[dtype]
    assert d_o <= tol_o and d_l <= tol_l
    p.close()
