"""A seeded sweep of shapes through the forward and backward (C ABI) against
the float64 oracle.

The shapes are drawn once from a fixed seed: batch 1-2, 1-4 query heads with
a K/V head count that divides them, any N up to 2600 (ragged tails), D 64 or
128, causal or not, fp16 or bf16.  Small B*H*N drives the backward into its
split modes (the dK/dV pass over query positions, the dQ pass over key
tiles) at varying part counts, and the forward through both head sizes and
every tail length class.
"""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import round_to
from oracle import attention_backward, attention_forward
from parity import assert_fwd_close, assert_grads_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def draw_cases(n, seed=4242):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        Hkv = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
        N = int(rng.integers(1, 2601))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        dtype = str(rng.choice(["fp16", "bf16"]))
        cases.append((B, H, Hkv, N, D, causal, dtype))
    return cases


CASES = draw_cases(40)


@pytest.mark.parametrize("B,H,Hkv,N,D,causal,dtype", CASES)
def test_random_shape(B, H, Hkv, N, D, causal, dtype):
    say("shape B=%d H=%d Hkv=%d N=%d D=%d causal=%d %s" % (B, H, Hkv, N, D, causal, dtype))
    rng = np.random.default_rng(B * 1000003 + H * 10007 + N * 101 + D + causal)
    q = round_to(rng.standard_normal((B, H, N, D), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((B, Hkv, N, D), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((B, Hkv, N, D), dtype=np.float32), dtype)
    do = round_to(rng.standard_normal((B, H, N, D), dtype=np.float32), dtype)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(q, k, v, causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "N=%d" % N)
    ref = attention_backward(q, k, v, do, causal, scale)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "N=%d" % N)
