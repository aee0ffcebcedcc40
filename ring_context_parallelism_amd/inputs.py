"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no part of the attention method: it only names the
workloads (shapes, chunk placement, dtype, which share is run) and draws their
Q/K/V.  Values are i.i.d. N(0, 1), drawn on the CPU in fp32 with a
``torch.Generator`` seeded per workload, in the order Q, K, V, each of shape
``[S, H, D]`` (batch 1, natural token order, contiguous).  For bf16 workloads
the fp32 draw is rounded to bf16 (round-to-nearest-even); the oracle receives
exactly the rounded values.
"""

import hashlib
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seq_len: int
    cp: int
    layout: str          # "zigzag" or "contiguous"
    heads: int
    head_dim: int
    dtype: str           # "fp32" or "bf16"
    causal: bool
    rank: int | None     # None: every rank's share; else that rank's share only
    seed: int

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    w.name: w
    for w in [
        # Tiny fp32 case: 4 chunks of 64, rank 0 = {0,3}, rank 1 = {1,2}.
        Workload("causal_s256_cp2_zigzag_h2_d64_fp32", 256, 2, "zigzag", 2, 64, "fp32", True, None, 1000),
        # The pages' own example length (8192 tokens at cp 4), 32 heads x 128.
        Workload("causal_s8192_cp4_zigzag_h32_d128_bf16", 8192, 4, "zigzag", 32, 128, "bf16", True, None, 1001),
        # Zigzag vs naive placement at 16k.
        Workload("causal_s16384_cp4_zigzag_h16_d128_bf16", 16384, 4, "zigzag", 16, 128, "bf16", True, None, 1002),
        Workload("causal_s16384_cp4_contiguous_h16_d128_bf16", 16384, 4, "contiguous", 16, 128, "bf16", True, None, 1002),
        # One rank's share at long length: rank 0 owns chunks {0, 15}.
        Workload("causal_s32768_cp8_zigzag_h32_d128_bf16_rank0", 32768, 8, "zigzag", 32, 128, "bf16", True, 0, 1003),
        # Bidirectional, 16 contiguous chunks of 4096, rank 0's share.
        Workload("bidir_s65536_cp16_contiguous_h8_d128_bf16_rank0", 65536, 16, "contiguous", 8, 128, "bf16", False, 0, 1004),
    ]
}


def make_qkv(seq_len, heads, head_dim, dtype, seed):
    """Return CPU tensors ``(q, k, v)`` of shape ``[seq_len, heads, head_dim]``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    shape = (int(seq_len), int(heads), int(head_dim))
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x if dtype in ("fp32", torch.float32) else x.to(torch.bfloat16))
    return tuple(out)


def workload_qkv(w: Workload):
    return make_qkv(w.seq_len, w.heads, w.head_dim, w.dtype, w.seed)


def sha256_of(*tensors):
    """SHA-256 over the raw bytes of CPU tensors, in order."""
    h = hashlib.sha256()
    for t in tensors:
        t = t.contiguous()
        h.update(t.view(torch.uint8).numpy().tobytes() if t.dtype != torch.bfloat16
                 else t.view(torch.int16).numpy().tobytes())
    return h.hexdigest()


def to_numpy_f64(t):
    """Exact fp64 copy of a CPU fp32/bf16 tensor (both embed exactly in fp64)."""
    return t.to(torch.float64).numpy()


def make_documents(seq_len, mean_len, seed):
    """Seeded document starts for document masks: lengths i.i.d. uniform on
    ``[1, 2 mean_len - 1]`` (a mix of short and long documents, mean about
    ``mean_len``), laid end to end from position 0; the last document is cut
    at ``seq_len``.  Returns a sorted list whose first entry is 0."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    starts, pos = [], 0
    hi = max(1, 2 * int(mean_len) - 1)
    while pos < seq_len:
        starts.append(pos)
        pos += int(torch.randint(1, hi + 1, (1,), generator=g))
    return starts
