"""Grouped K/V heads (GQA; MQA when H_kv = 1) on the GPU: fa_fwd_ex and
fa_bwd_ex with fa_options.h_kv (through the C ABI, via fa.fwd / fa.bwd with k, v of H_kv heads)
against the float64 oracle, whose grouped-head reading is pinned against
repeated K/V heads.  "CUDA FlashAttention ..." §7: query heads share a K/V
head in place, without copying K or V."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import make_key_mask, round_to
from oracle import attention_backward, attention_forward
from parity import LSE_TOL, assert_fwd_close, assert_grads_close, o_error_ok, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def gqa_inputs(B, H, Hkv, N, D, dtype, seed):
    """Seeded q, do [B, H, N, D] and k, v [B, Hkv, N, D], N(0,1) rounded to dtype."""
    rng = np.random.default_rng(seed)
    q = round_to(rng.standard_normal((B, H, N, D), dtype=np.float32), dtype)
    k = round_to(rng.standard_normal((B, Hkv, N, D), dtype=np.float32), dtype)
    v = round_to(rng.standard_normal((B, Hkv, N, D), dtype=np.float32), dtype)
    do = round_to(rng.standard_normal((B, H, N, D), dtype=np.float32), dtype)
    return {"q": q, "k": k, "v": v, "do": do}


CASES = [(1, 4, 2, 200, 64), (2, 8, 1, 130, 128), (1, 6, 3, 512, 128), (2, 4, 4, 96, 64), (1, 16, 2, 320, 64)]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,D", CASES)
def test_fwd_gqa(B, H, Hkv, N, D, causal, dtype):
    say("fwd gqa B=%d H=%d Hkv=%d N=%d D=%d causal=%d %s" % (B, H, Hkv, N, D, causal, dtype))
    inp = gqa_inputs(B, H, Hkv, N, D, dtype, 6000 + H * 10 + Hkv + N)
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "H=%d Hkv=%d N=%d" % (H, Hkv, N))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Hkv,N,D", CASES)
def test_bwd_gqa(B, H, Hkv, N, D, causal, dtype):
    say("bwd gqa B=%d H=%d Hkv=%d N=%d D=%d causal=%d %s" % (B, H, Hkv, N, D, causal, dtype))
    inp = gqa_inputs(B, H, Hkv, N, D, dtype, 6100 + H * 10 + Hkv + N)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    scale = 1.0 / np.sqrt(D)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert dk.shape == k.shape and dv.shape == v.shape
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "H=%d Hkv=%d N=%d" % (H, Hkv, N))


def test_gqa_long_sampled_heads():
    # a common grouped geometry: 32 query heads on 8 K/V heads, N = 4096, D = 128
    B, H, Hkv, N, D = 1, 32, 8, 4096, 128
    inp = gqa_inputs(B, H, Hkv, N, D, "fp16", 6200)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    for hk in (0, 5):
        hs = slice(hk * 4, hk * 4 + 4)  # the four query heads of K/V head hk
        sub = {"q": inp["q"][:, hs], "k": inp["k"][:, hk:hk + 1], "v": inp["v"][:, hk:hk + 1], "do": inp["do"][:, hs]}
        o_ref, lse_ref = attention_forward(sub["q"], sub["k"], sub["v"], True, scale)
        assert_fwd_close(to_host(o[:, hs]), to_host(lse[:, hs]), o_ref, lse_ref, "fp16", "group %d" % hk)
        ref = attention_backward(sub["q"], sub["k"], sub["v"], sub["do"], True, scale)
        got = [to_host(dq[:, hs]), to_host(dk[:, hk:hk + 1]), to_host(dv[:, hk:hk + 1])]
        assert_grads_close(got, ref, "group %d" % hk)


def test_mqa_headline_shape_all_heads():
    """One K/V head for the 32 query heads of the headline shape (causal
    fp16 B1 N8192 D128), as the bench times it: O and LSE of every query
    head, dQ of every head and the group-summed dK, dV against the oracle."""
    B, H, Hkv, N, D = 1, 32, 1, 8192, 128
    say("MQA B=%d H=%d H_kv=%d N=%d D=%d, all heads" % (B, H, Hkv, N, D))
    inp = gqa_inputs(B, H, Hkv, N, D, "fp16", 6300)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, "fp16", "MQA, all %d heads" % H)
    del o_ref, lse_ref
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, scale)
    assert_grads_close([to_host(dq), to_host(dk), to_host(dv)], ref, "MQA, all %d heads" % H)


def test_gqa_with_key_mask():
    B, H, Hkv, N, D = 2, 6, 2, 300, 64
    inp = gqa_inputs(B, H, Hkv, N, D, "bf16", 6300)
    m = make_key_mask(B, N, "blocks", seed=6301, p=0.3)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    for causal in (False, True):
        o, lse = fa.fwd_masked(q, k, v, tiles, causal=causal, scale=0.125)
        dq, dk, dv = fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=causal, scale=0.125)
        torch.cuda.synchronize()
        o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, 0.125, key_mask=m)
        empty = np.isneginf(lse_ref)
        assert np.array_equal(np.isneginf(to_host(lse)), empty)
        full = ~empty
        assert np.all(to_host(o)[empty] == 0)
        assert o_error_ok(to_host(o)[full], o_ref[full], "bf16")[0]
        assert np.abs(to_host(lse)[full] - lse_ref[full]).max() <= LSE_TOL
        ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, 0.125, key_mask=m)
        assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "masked gqa causal=%d" % causal)


def test_gqa_equals_mha_on_repeated_heads_bitwise():
    """The grouped kernels read K/V head h // G in place; feeding the same
    heads repeated to the plain kernels must give identical O, LSE and dQ."""
    B, H, Hkv, N, D = 1, 8, 2, 256, 128
    inp = gqa_inputs(B, H, Hkv, N, D, "fp16", 6400)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    k_rep = k.repeat_interleave(H // Hkv, dim=1).contiguous()
    v_rep = v.repeat_interleave(H // Hkv, dim=1).contiguous()
    o1, l1 = fa.fwd(q, k, v, causal=True)
    o2, l2 = fa.fwd(q, k_rep, v_rep, causal=True)
    dq1, _, _ = fa.bwd(q, k, v, o1, l1, do, causal=True)
    dq2, _, _ = fa.bwd(q, k_rep, v_rep, o2, l2, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(dq1, dq2)


def test_bwd_gqa_uneven_head_parts():
    # B*H_kv*ceil(N/128) = 256 workgroups -> the dK/dV pass splits each group
    # of G = 6 query heads into 4 parts of 1, 2, 1, 2 heads
    B, H, Hkv, N, D = 8, 12, 2, 2048, 64
    assert fa.bwd_ex_workspace_bytes(B, H, N, D, 1, 0, fa.options(h_kv=Hkv)) == B * H * N * 4 + 2 * 4 * B * Hkv * N * D * 4
    inp = gqa_inputs(B, H, Hkv, N, D, "fp16", 6500)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for b, hk in ((0, 0), (5, 1)):
        hs = slice(hk * 6, hk * 6 + 6)
        sl = (slice(b, b + 1),)
        sub = [inp["q"][sl][:, hs], inp["k"][sl][:, hk:hk + 1], inp["v"][sl][:, hk:hk + 1], inp["do"][sl][:, hs]]
        ref = attention_backward(*sub, True, 0.125)
        got = [to_host(dq[sl][:, hs]), to_host(dk[sl][:, hk:hk + 1]), to_host(dv[sl][:, hk:hk + 1])]
        assert_grads_close(got, ref, "b=%d group %d" % (b, hk))
