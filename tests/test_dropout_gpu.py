"""Attention dropout on the GPU: the keep mask regenerated from (seed,
offset) by fa_dropout_mask (bit-exact against the oracle's Philox4x64-10
mapping), and fa_fwd_ex / fa_bwd_ex with fa_options.dropout (through the C ABI) against
the float64 oracle with the same (p, seed, offset).  "Why FlashAttention does
not need to store the attention matrix" §05: only the seed and offset are
kept; the backward pass regenerates the mask."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import make_inputs, make_key_mask, round_to
from oracle import attention_backward, attention_forward, dropout_keep
from parity import LSE_TOL, assert_fwd_close, assert_grads_close, o_error_ok, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,N,p,seed,offset", [
    (1, 1, 1, 0.5, 1, 0), (2, 3, 100, 0.1, 12345, 7), (1, 2, 1000, 0.5, (1 << 64) - 1, 3),
    (1, 1, 257, 0.9, 0xDEADBEEFCAFEF00D, (1 << 63) + 5), (1, 1, 64, 0.0, 9, 9),
])
def test_dropout_mask_bit_exact(B, H, N, p, seed, offset):
    say("dropout mask B=%d H=%d N=%d p=%g" % (B, H, N, p))
    keep = fa.dropout_mask(B, H, N, p, seed, offset)
    torch.cuda.synchronize()
    ref = dropout_keep(B, H, N, p, seed, offset)
    assert np.array_equal(keep.cpu().numpy().astype(bool), ref)


def _inputs(B, H, Hkv, N, D, dtype, seed):
    rng = np.random.default_rng(seed)
    out = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv), ("do", H)):
        out[name] = round_to(rng.standard_normal((B, heads, N, D), dtype=np.float32), dtype)
    return out


CASES = [(1, 2, 2, 128, 64), (2, 3, 3, 200, 128), (1, 4, 2, 257, 64), (1, 1, 1, 64, 128)]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,D", CASES)
def test_fwd_dropout(B, H, Hkv, N, D, causal, dtype):
    say("fwd dropout B=%d H=%d Hkv=%d N=%d D=%d causal=%d %s" % (B, H, Hkv, N, D, causal, dtype))
    inp = _inputs(B, H, Hkv, N, D, dtype, 7000 + N + D)
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    drop = (0.2, 424242 + N, 11)
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fwd_dropout(q, k, v, *drop, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale, dropout=drop)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "N=%d p=0.2" % N)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,D", CASES)
def test_bwd_dropout(B, H, Hkv, N, D, causal, dtype):
    say("bwd dropout B=%d H=%d Hkv=%d N=%d D=%d causal=%d %s" % (B, H, Hkv, N, D, causal, dtype))
    inp = _inputs(B, H, Hkv, N, D, dtype, 7100 + N + D)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    drop = (0.3, 99 + N, 5)
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fwd_dropout(q, k, v, *drop, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, lse, do, *drop, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, dropout=drop)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "N=%d p=0.3" % N)


def test_dropout_is_regenerated_deterministically():
    inp = make_inputs(1, 4, 512, 64, "fp16", seed=7200)
    q, k, v = (to_dev(inp[n], "fp16") for n in ("q", "k", "v"))
    a = fa.fwd_dropout(q, k, v, 0.1, 77, 0, causal=True)
    b = fa.fwd_dropout(q, k, v, 0.1, 77, 0, causal=True)
    c = fa.fwd_dropout(q, k, v, 0.1, 77, 1, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])  # LSE is the undropped one


@pytest.mark.parametrize("D", [64, 128])
def test_dropout_zero_probability_matches_plain_forward(D):
    # 2 x 43 heads of 300 queries: 258 tiles of 128 queries, enough for
    # fa_fwd to run the 128-query kernel that the dropout forward extends.
    inp = make_inputs(2, 43, 300, D, "bf16", seed=7300, with_dout=True)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    o0, l0 = fa.fwd(q, k, v, causal=True)
    o1, l1 = fa.fwd_dropout(q, k, v, 0.0, 1, 2, causal=True)
    g0 = fa.bwd(q, k, v, o0, l0, do, causal=True)
    g1 = fa.bwd_dropout(q, k, v, o1, l1, do, 0.0, 1, 2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.allclose(l0, l1, atol=1e-6, rtol=0)
    assert torch.equal(g0[0], g1[0])  # dQ: the same arithmetic
    for a, b in zip(g0[1:], g1[1:]):
        if D == 64:
            assert torch.equal(a, b)
        else:
            # dK, dV at D = 128: the plain kernel starts the S and dP
            # accumulators at -LSE/scale and -Delta, the dropout kernel
            # subtracts them afterwards.  The FP32 values of P and dS differ
            # by rounding order only, but that can flip their rounding to
            # bf16 before the dV/dK products, so single elements may differ
            # by a few units in the last place: the tensors agree to well
            # inside the oracle tolerance.
            r = rel_fro(to_host(a), to_host(b))
            say("  p = 0, D = 128: plain vs dropout relative difference %.2e" % r)
            assert r <= 2e-3
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, 1 / np.sqrt(D))
    assert_grads_close([to_host(t) for t in g1], ref, "p=0 D=%d" % D)


@pytest.mark.parametrize("N,D,in_seed,heads", [(4096, 64, 5, (0, 17)), (8192, 128, 3, (0, 31))],
                         ids=["n4096_d64", "n8192_d128"])
def test_dropout_long_sampled_heads(N, D, in_seed, heads):
    # the C5 geometry (causal fp16, H = 32, N = 4096, D = 64) and the headline
    # one (N = 8192, D = 128) with p = 0.1; a sampled head is checked alone
    # with the counter's head number of the full problem (the oracle's
    # head_numbers)
    B, H = 1, 32
    say("dropout p=0.1 B=%d H=%d N=%d D=%d causal, heads %s" % (B, H, N, D, heads))
    inp = make_inputs(B, H, N, D, "fp16", seed=in_seed, with_dout=True)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    p, seed, offset = 0.1, 2024, 0
    o, lse = fa.fwd_dropout(q, k, v, p, seed, offset, causal=True)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, lse, do, p, seed, offset, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    for h in heads:
        sl = (slice(0, 1), slice(h, h + 1))
        sub = [inp[n][sl] for n in ("q", "k", "v", "do")]
        drop = (p, seed, offset, [[h]])
        o_ref, lse_ref = attention_forward(*sub[:3], True, scale, dropout=drop)
        assert_fwd_close(to_host(o[sl]), to_host(lse[sl]), o_ref, lse_ref, "fp16", "head %d" % h)
        grads = attention_backward(*sub, True, scale, dropout=drop)
        assert_grads_close([to_host(t[sl]) for t in (dq, dk, dv)], grads, "head %d" % h)


def test_dropout_bwd_one_head_in_parts():
    # one head of 1500 keys: both backward passes split into 3 parts
    B, H, N, D = 1, 1, 1500, 128
    inp = make_inputs(B, H, N, D, "fp16", seed=7400, with_dout=True)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    p, seed, offset = 0.2, 99, 5
    o, lse = fa.fwd_dropout(q, k, v, p, seed, offset, causal=True)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, lse, do, p, seed, offset, causal=True)
    torch.cuda.synchronize()
    drop = (p, seed, offset)
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, 1 / np.sqrt(D), dropout=drop)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "one head dropout")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kind", ["lengths", "blocks", "random"])
def test_dropout_with_key_mask(kind, D, causal, dtype):
    # dropout and a key-padding mask together (both options of fa_fwd_ex /
    # fa_bwd_ex) against the oracle with both applied; the random
    # mask hides keys 0..2 so that causal rows 0..2 see no key at all
    B, H, N = 2, 2, 333
    say("dropout + %s mask D=%d causal=%d %s" % (kind, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=7500 + D + causal, with_dout=True)
    m = make_key_mask(B, N, kind, seed=7501, p=0.5)
    if kind == "random":
        m[:, :3] = 0
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    p, seed, offset = 0.25, 31337, 7
    o, lse = fa.fwd_dropout(q, k, v, p, seed, offset, causal=causal, scale=0.1, tiles=tiles)
    dq, dk, dv = fa.bwd_dropout(q, k, v, o, lse, do, p, seed, offset, causal=causal, scale=0.1, tiles=tiles)
    torch.cuda.synchronize()
    drop = (p, seed, offset)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, 0.1, key_mask=m, dropout=drop)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(to_host(lse)), empty)
    full = ~empty
    assert np.all(to_host(o)[empty] == 0)
    assert o_error_ok(to_host(o)[full], o_ref[full], dtype)[0]
    assert np.abs(to_host(lse)[full] - lse_ref[full]).max() <= LSE_TOL
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, 0.1, key_mask=m, dropout=drop)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "dropout + %s mask" % kind)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_masked_dropout_zero_probability_is_masked_forward(dtype):
    # bf16: the dropout path and the plain path both sum the row's FP32
    # probabilities, so p = 0 is bitwise the masked forward.  fp16: the plain
    # path sums the probabilities as packed to fp16 (the operand of P V), the
    # dropout path the FP32 ones before dropping, so the results differ by
    # that rounding only.
    B, H, N, D = 1, 2, 400, 128
    inp = make_inputs(B, H, N, D, dtype, seed=7600)
    m = make_key_mask(B, N, "blocks", seed=7601, p=0.5)
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o0, l0 = fa.fwd_masked(q, k, v, tiles, causal=True)
    o1, l1 = fa.fwd_dropout(q, k, v, 0.0, 3, 4, causal=True, tiles=tiles)
    torch.cuda.synchronize()
    if dtype == "bf16":
        assert torch.equal(o0, o1) and torch.allclose(l0, l1, atol=1e-6, rtol=0)
    else:
        assert (o0.float() - o1.float()).abs().max().item() <= 1e-3
        assert torch.equal(torch.isneginf(l0), torch.isneginf(l1))
        fin = torch.isfinite(l0)
        assert (l0[fin] - l1[fin]).abs().max().item() <= 1e-3
