"""Tensors of more than 2^31 elements: every element offset of the heads past
the 2^31 boundary overflows 32-bit arithmetic, so these heads check the
library's 64-bit index math.  B=3, H=700, N=8192, D=128 (2.2e9 elements per
tensor, 4.4 GB in fp16); causal.

* A head computed inside the large call is bitwise equal to the same head
  computed in a small call (forward O and LSE, backward dQ, dK, dV): the
  kernels treat heads independently and deterministically, so any addressing
  error in the large call shows as a difference.
* Sampled rows of the last head are checked against the float64 oracle.

Inputs are seeded N(0,1) values drawn on the device with a seeded torch
generator and rounded to fp16 (host generation of 8.8e9 values would take
minutes); the oracle receives host copies of the heads it checks.
"""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from oracle import attention_forward
from parity import LSE_TOL, o_error_ok, say, to_host

pytestmark = pytest.mark.gpu


def test_heads_beyond_2g_elements():
    B, H, N, D = 3, 700, 8192, 128
    assert B * H * N * D > 2 ** 31
    gen = torch.Generator(device="cuda")
    gen.manual_seed(8800)
    shape = (B, H, N, D)
    say("large: drawing 4 tensors of %d elements" % (B * H * N * D))
    q, k, v, do = (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).to(torch.float16)
                   for _ in range(4))
    scale = 1.0 / np.sqrt(D)
    say("large: forward")
    o, lse = fa.fwd(q, k, v, causal=True, scale=scale)
    say("large: backward")
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()

    # head (2, 648) is batch-head 2048: its first element is at 2^31.  Each
    # sampled head is recomputed as 32 copies of itself: that gives the
    # forward 1024 tiles of 256 queries, so it runs the same kernel as the
    # large call, and the dK/dV pass 2048 workgroups, so, as in the large
    # call, it does not split the head's query tiles into parts (parts would
    # add FP32 partial sums in another order); copy 0 must equal the large
    # call's head bitwise.
    for b, h in ((0, 0), (1, 347), (2, 647), (2, 648), (2, 699)):
        say("large: head (%d, %d) alone" % (b, h))
        sl = (slice(b, b + 1), slice(h, h + 1))
        qh, kh, vh, doh = (t[sl].expand(1, 32, N, D).contiguous() for t in (q, k, v, do))
        assert fa.bwd_workspace_bytes(1, 32, N, D, 1, 0) == 32 * N * 4  # one part
        o1, l1 = fa.fwd(qh, kh, vh, causal=True, scale=scale)
        g1 = fa.bwd(qh, kh, vh, o1, l1, doh, causal=True, scale=scale)
        torch.cuda.synchronize()
        first = (slice(0, 1), slice(0, 1))
        assert torch.equal(o1[first], o[sl]) and torch.equal(l1[first], lse[sl])
        for a, big in zip(g1, (dq, dk, dv)):
            assert torch.equal(a[first], big[sl])

    rows = np.array([0, 1, 63, 64, 4095, 8190, 8191])
    sl = (slice(2, 3), slice(699, 700))
    qh, kh, vh = (to_host(t[sl]) for t in (q, k, v))
    o_ref, lse_ref = attention_forward(qh, kh, vh, True, scale, rows=rows)
    o_gpu, lse_gpu = to_host(o[sl])[:, :, rows], to_host(lse[sl])[:, :, rows]
    assert o_error_ok(o_gpu, o_ref, "fp16")[0]
    assert np.abs(lse_gpu - lse_ref).max() <= LSE_TOL
