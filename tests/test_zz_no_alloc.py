"""fa_bwd_noalloc (the backward with the library's static scratch in place of
a caller's workspace) against fa_bwd, through the C ABI: two calls in a row,
the second with a smaller input, each bitwise equal to fa_bwd on the same
inputs (the same kernels run on the same workspace layout).  The rejection
of shapes beyond the scratch is checked on the CPU (tests/test_abi.py)."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd import binding
from exact_attention_25_amd.inputs import make_inputs
from parity import say, to_dev

pytestmark = pytest.mark.gpu

def _grads_noalloc(q, k, v, o, lse, do, causal, scale, code):
    B, H, N, D = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    st = binding.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, D, causal,
                                scale, code, torch.cuda.current_stream().cuda_stream)
    assert st == 0, binding.status_str(st)
    return dq, dk, dv


# the second case is smaller than the first (fewer rows, smaller head size)
CASES = [(2, 4, 1000, 128, True, "fp16"), (1, 2, 300, 64, False, "bf16")]


def test_bwd_noalloc_matches_bwd_twice():
    for i, (B, H, N, D, causal, dtype) in enumerate(CASES):
        say("noalloc call %d: B=%d H=%d N=%d D=%d causal=%d %s" % (i, B, H, N, D, causal, dtype))
        inp = make_inputs(B, H, N, D, dtype, seed=3100 + i, with_dout=True)
        q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
        scale = 1.0 / np.sqrt(D)
        o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
        want = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
        got = _grads_noalloc(q, k, v, o, lse, do, int(causal), scale, 0 if dtype == "fp16" else 1)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, want):
            assert torch.equal(a, b), "%s differs from fa_bwd on call %d" % (name, i)
