"""The C ABI used without PyTorch: tests/c_abi_client (a C++ program built by
build() against include/fa.h and libfa.so, with hipMalloc'd buffers and its
own stream) runs fa_fwd and fa_bwd on seeded inputs written to a file.  Its
outputs must match the float64 oracle to the usual tolerances and be bitwise
equal to the same entry points called through the Python binding."""

import os
import subprocess

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import make_inputs
from oracle import attention_backward, attention_forward
from parity import assert_fwd_close, assert_grads_close, say, to_dev

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_client")
DTYPE_CODE = {"fp16": 0, "bf16": 1}


def encode(x, dtype):
    """float32 array whose values are exact in dtype -> its 16-bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def decode(bits, dtype):
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("B,H,N,D,causal,dtype", [
    (1, 2, 192, 64, True, "fp16"),
    (2, 1, 320, 128, False, "bf16"),
    (1, 3, 200, 128, True, "fp16"),
])
def test_c_client_matches_oracle_and_binding(tmp_path, B, H, N, D, causal, dtype):
    if not os.path.exists(CLIENT):
        pytest.skip("tests/c_abi_client is not built (build() compiles it)")
    say("c client B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=4100 + N + D, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for n in ("q", "k", "v", "do"):
            f.write(encode(inp[n], dtype).tobytes())
    res = subprocess.run([CLIENT, str(src), str(dst), str(B), str(H), str(N), str(D), str(int(causal)),
                          str(DTYPE_CODE[dtype]), repr(float(scale))],
                         capture_output=True, text=True, timeout=60)
    say("  client: rc=%d %s%s" % (res.returncode, res.stdout.strip(), res.stderr.strip()))
    assert res.returncode == 0
    raw = np.fromfile(dst, dtype=np.uint8)
    elems, rows = B * H * N * D, B * H * N
    assert raw.size == 4 * elems * 2 + rows * 4
    bits = raw[:4 * elems * 2].view(np.uint16).reshape(4, B, H, N, D)
    o, dq, dk, dv = (decode(bits[i], dtype) for i in range(4))
    lse = raw[4 * elems * 2:].view(np.float32).astype(np.float64).reshape(B, H, N)

    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(o, lse, o_ref, lse_ref, dtype, "c client")
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close([dq, dk, dv], ref, "c client")

    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o_b, lse_b = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads_b = fa.bwd(q, k, v, o_b, lse_b, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for name, mine, theirs in zip(("O", "dQ", "dK", "dV"), (bits[0], bits[1], bits[2], bits[3]), (o_b,) + tuple(grads_b)):
        t = theirs.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(mine, t), "%s differs between the C client and the binding" % name
    assert np.array_equal(lse.astype(np.float32), lse_b.cpu().numpy()), "LSE differs"
