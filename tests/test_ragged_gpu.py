"""Sequence lengths that are not a multiple of the 64-row tile, on the GPU:
fa_fwd, the split-K/V fa_fwd_ex and fa_bwd (through the C ABI) against the float64
oracle, and guard regions after every output that must stay untouched.

"FlashAttention dataflow and engineering validation on MI50" (§6.1) names the
partial last tile as the most common hidden bug and asks for unit tests of
each boundary case; its boundary stress test uses seq_len 1025 with D=128.
"""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import make_inputs
from oracle import attention_backward, attention_forward
from parity import TORCH_DTYPE, assert_fwd_close, assert_grads_close, say, to_dev, to_host

pytestmark = pytest.mark.gpu

GUARD = 4096  # elements of sentinel after each output


def guarded(shape, dtype):
    """(view, whole buffer): an output tensor followed by NaN sentinels."""
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), float("nan"), dtype=dtype, device="cuda")
    return buf[:n].view(*shape), buf


def assert_guard(buf, n, what):
    tail = buf[n:].float()
    assert torch.isnan(tail).all(), "%s: %d sentinel values after the output were overwritten" % (
        what, int((~torch.isnan(tail)).sum()))


def fwd_guarded(inp, dtype, causal, scale, splits=0):
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    B, H, N, D = q.shape
    o, obuf = guarded((B, H, N, D), TORCH_DTYPE[dtype])
    lse, lbuf = guarded((B, H, N), torch.float32)
    if splits:
        fa.fwd_splitkv(q, k, v, splits, causal=causal, scale=scale, out=o, lse=lse)
    else:
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert_guard(obuf, o.numel(), "O")
    assert_guard(lbuf, lse.numel(), "LSE")
    return o, lse


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 2, 7), (2, 1, 63), (1, 1, 65), (2, 3, 100), (1, 2, 191),
                                   (1, 1, 257), (1, 1, 1025)])
def test_fwd_ragged(B, H, N, D, causal, dtype):
    say("fwd ragged B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=4000 + N + D)
    scale = 1.0 / np.sqrt(D)
    o, lse = fwd_guarded(inp, dtype, causal, scale)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "N=%d D=%d" % (N, D))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D,N,splits", [(64, 100, 3), (128, 1025, 4), (64, 33, 2), (128, 200, 64)])
def test_splitkv_ragged(N, D, splits, causal):
    say("splitkv ragged N=%d D=%d splits=%d causal=%d" % (N, D, splits, causal))
    inp = make_inputs(1, 2, N, D, "fp16", seed=4100 + N + splits)
    scale = 1.0 / np.sqrt(D)
    o, lse = fwd_guarded(inp, "fp16", causal, scale, splits=splits)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, "fp16", "N=%d splits=%d" % (N, splits))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 1, 1), (1, 2, 50), (2, 1, 65), (1, 2, 130), (1, 1, 1025)])
def test_bwd_ragged(B, H, N, D, causal, dtype):
    say("bwd ragged B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=4200 + N + D, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close([to_host(t) for t in grads], ref, "N=%d D=%d" % (N, D))


def test_bwd_ragged_leaves_memory_after_outputs_untouched():
    B, H, N, D = 1, 1, 200, 128
    inp = make_inputs(B, H, N, D, "fp16", seed=4300, with_dout=True)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True, scale=0.1)
    outs = [guarded((B, H, N, D), torch.float16) for _ in range(3)]
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, D, 1, 0), dtype=torch.uint8, device="cuda")
    st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                   outs[0][0].data_ptr(), outs[1][0].data_ptr(), outs[2][0].data_ptr(), B, H, N, D, 1, 0.1, 0,
                   ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    for name, (t, buf) in zip(("dQ", "dK", "dV"), outs):
        assert_guard(buf, t.numel(), name)
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.1)
    assert_grads_close([to_host(t) for t, _ in outs], ref, "guarded N=200")


def test_ragged_matches_padded_prefix():
    """Attention over the first N rows equals the causal attention of a
    longer sequence restricted to those rows (queries < N see keys < N)."""
    N, M, D = 321, 384, 64
    inp = make_inputs(1, 2, M, D, "fp16", seed=4400)
    q, k, v = (to_dev(inp[n], "fp16") for n in ("q", "k", "v"))
    o_full, lse_full = fa.fwd(q, k, v, causal=True, scale=0.125)
    o_cut, lse_cut = fa.fwd(q[:, :, :N].contiguous(), k[:, :, :N].contiguous(), v[:, :, :N].contiguous(),
                            causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.allclose(o_cut.float(), o_full[:, :, :N].float(), atol=2e-3, rtol=0)
    assert torch.allclose(lse_cut, lse_full[:, :, :N], atol=1e-4, rtol=0)


def nan_tailed(shape, dtype):
    """A tensor at the start of a buffer that continues with 64 rows of NaN
    (more than any tile reaches past the last row): a kernel that reads a
    row past the end gets NaN into its result (0 * NaN is NaN in a product)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 64 * shape[-1],), float("nan"), dtype=dtype, device="cuda")
    return buf[:n].view(*shape)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("N", [17, 1000])
def test_rows_past_the_end_are_never_read(N, D, causal, dtype):
    """The partial last K/V tile of the last head is followed by memory that
    is not the caller's: only its valid rows may reach the result.  Every
    input sits at the start of a buffer that continues with NaN, and
    fa_fwd, the split fa_fwd_ex and fa_bwd must still match the oracle."""
    say("rows past the end N=%d D=%d causal=%d %s" % (N, D, causal, dtype))
    inp = make_inputs(1, 2, N, D, dtype, seed=4500 + N + D, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (nan_tailed(inp[n].shape, TORCH_DTYPE[dtype]).copy_(to_dev(inp[n], dtype))
                   for n in ("q", "k", "v", "do"))
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "fa_fwd N=%d D=%d" % (N, D))
    o2, lse2 = fa.fwd_splitkv(q, k, v, 3, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert_fwd_close(to_host(o2), to_host(lse2), o_ref, lse_ref, dtype, "split fa_fwd_ex N=%d D=%d" % (N, D))
    o_t = nan_tailed(o.shape, o.dtype).copy_(o)
    lse_t = nan_tailed(lse.shape + (1,), torch.float32).view(lse.shape).copy_(lse)
    grads = fa.bwd(q, k, v, o_t, lse_t, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close([to_host(t) for t in grads], ref, "fa_bwd N=%d D=%d" % (N, D))
