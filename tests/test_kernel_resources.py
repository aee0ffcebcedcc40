"""Register budget of the head_dim-128 step kernel (CPU only: compiles the
kernel source for gfx950 and reads the resources the compiler assigns).

Two waves of the step kernel share each SIMD's 512 VGPRs.  The ring-receive
copy kernel (one wave per workgroup, 16 VGPRs) runs beside it on the copy
stream only while each step-kernel wave leaves room for it, i.e. takes at
most 240 VGPRs (allocation granule 8); above that the copy waits for the
step kernel and the whole call slows down by about a third.  No variant may
spill to scratch (a scratch reload waits for every load in flight, which
would collapse the direct-to-LDS pipeline).
"""

import os
import re
import subprocess
import tempfile

import pytest

from ring_context_parallelism_amd import build as B


def _resources(source="attn_bf16.hip"):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "kernels.s")
        flags = [f for f in B.COMMON if f != "-fPIC"]
        cmd = [B.hipcc(), "-x", "hip", *B.HIP_FLAGS, *B.TU_FLAGS.get(source, []), *flags, "--cuda-device-only", "-S",
               os.path.join(B.CSRC, source), "-o", out]
        subprocess.run(cmd, check=True, capture_output=True, timeout=600)
        text = open(out).read()
    res = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        body = m.group(2)
        get = lambda key: int(re.search(rf"\.amdhsa_{key} (\d+)", body).group(1))
        res[m.group(1)] = {"vgpr": get("next_free_vgpr"), "scratch": get("private_segment_fixed_size")}
    return res


@pytest.fixture(scope="module")
def resources():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    return _resources()


def test_step_kernel_leaves_room_for_the_receive_kernel(resources):
    # <no in-kernel receive, no documents>: one rank's step, every rank's step
    # in one launch, and every step of one rank in one launch (fused ring,
    # whose receive copies must run beside it)
    plain = [v for k, v in resources.items() if "attn_step_bf16_d128x8ILb0ELb0EL" in k]
    assert len(plain) == 3, sorted(resources)
    assert all(v["vgpr"] <= 240 for v in plain), plain


def test_no_kernel_spills_to_scratch(resources):
    for name, r in resources.items():
        assert r["scratch"] == 0, (name, r)


def test_backward_kernels_do_not_spill():
    """The matrix-core backward kernels keep every value in registers; the
    eight-wave row-major dQ kernel and the eight-wave key-major kernel stay
    within 256 VGPRs (two of their waves per SIMD)."""
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    res = _resources("attn_bwd_bf16.hip")
    assert res
    for name, r in res.items():
        assert r["scratch"] == 0, (name, r)
    dq = [v for k, v in res.items() if "bwd_dq_bf16_d128x8" in k]
    assert len(dq) == 2 and all(v["vgpr"] <= 256 for v in dq), dq
    x8 = [v for k, v in res.items() if "bwd_dkdv_bf16_d128x8" in k]
    assert len(x8) == 2 and all(v["vgpr"] <= 256 for v in x8), x8
