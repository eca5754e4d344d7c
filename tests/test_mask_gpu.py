"""Key-padding masks on the GPU: the tile table built by fa_mask_tiles
(bit-exact against the oracle's block-level words), fa_fwd_ex and
fa_bwd_ex with fa_options.mask_tiles (through the C ABI) against the float64 oracle with the same
mask.  Masks follow "FlashAttention dataflow and engineering validation on
MI50": padded variable-length batches (§4.3) and random mask patterns
(§5.1), plus tile-structured masks that give the block-level flags every
kind of tile (empty, full, partial)."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd.inputs import make_inputs, make_key_mask
from oracle import attention_backward, attention_forward, key_tile_words
from parity import (LSE_TOL, TORCH_DTYPE, assert_grads_close, o_error_ok, say, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _table(tiles, B, N):
    """Split a tile table (device uint8 tensor) into words, prefix, list."""
    T = -(-N // 64)
    raw = tiles.cpu().numpy()
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    p_off = up(8 * B * T)
    l_off = p_off + up(4 * B * (T + 1))
    words = raw[:8 * B * T].view(np.uint64).reshape(B, T)
    prefix = raw[p_off:p_off + 4 * B * (T + 1)].view(np.int32).reshape(B, T + 1)
    lst = raw[l_off:l_off + 4 * B * T].view(np.int32).reshape(B, T)
    return words, prefix, lst


@pytest.mark.parametrize("B,N,kind", [(1, 1, "all"), (2, 100, "random"), (3, 1025, "lengths"),
                                      (2, 64 * 300 + 5, "blocks"), (4, 640, "random"), (1, 70000, "blocks")])
def test_mask_tiles_match_oracle(B, N, kind):
    say("mask tiles B=%d N=%d %s" % (B, N, kind))
    m = make_key_mask(B, N, kind, seed=B * 1000 + N, p=0.3)
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    words, prefix, lst = _table(tiles, B, N)
    ref_words, ref_tiles = key_tile_words(m)
    for b in range(B):
        assert [int(w) for w in words[b]] == ref_words[b]
        cnt = len(ref_tiles[b])
        assert prefix[b, -1] == cnt
        assert lst[b, :cnt].tolist() == ref_tiles[b]
        nz = np.array([w != 0 for w in ref_words[b]], dtype=np.int64)
        assert prefix[b, :-1].tolist() == (np.cumsum(nz) - nz).tolist()


def _assert_masked_fwd(o, lse, o_ref, lse_ref, dtype, what):
    o, lse = to_host(o), to_host(lse)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), "%s: rows without a visible key differ" % what
    assert np.all(o[empty] == 0.0), "%s: a row without a visible key is not zero" % what
    full = ~empty
    ok, max_abs, excess = o_error_ok(o[full], o_ref[full], dtype)
    lse_err = float(np.abs(lse[full] - lse_ref[full]).max()) if full.any() else 0.0
    say("  %s: %d empty rows, O max abs err %.3e, LSE max abs err %.3e" % (what, int(empty.sum()), max_abs, lse_err))
    assert np.all(np.isfinite(o)) and ok, "%s: O error %.3e" % (what, max_abs)
    assert lse_err <= LSE_TOL, "%s: LSE error %.3e" % (what, lse_err)


def run_masked_fwd(inp, m, dtype, causal, scale):
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o, lse = fa.fwd_masked(q, k, v, tiles, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N,kind", [(2, 2, 200, "lengths"), (1, 2, 320, "random"), (2, 1, 513, "blocks"),
                                        (1, 1, 64, "random"), (3, 2, 130, "blocks")])
def test_fwd_masked(B, H, N, D, causal, dtype, kind):
    say("fwd masked B=%d H=%d N=%d D=%d causal=%d %s %s" % (B, H, N, D, causal, dtype, kind))
    inp = make_inputs(B, H, N, D, dtype, seed=5000 + N + D)
    m = make_key_mask(B, N, kind, seed=5100 + N, p=0.4)
    scale = 1.0 / np.sqrt(D)
    o, lse = run_masked_fwd(inp, m, dtype, causal, scale)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale, key_mask=m)
    _assert_masked_fwd(o, lse, o_ref, lse_ref, dtype, "N=%d %s" % (N, kind))


def test_fwd_masked_sparse_and_empty():
    # p = 0.02: most tiles empty, many rows without any visible key
    B, H, N, D = 2, 2, 700, 64
    inp = make_inputs(B, H, N, D, "fp16", seed=5200)
    for kind, p in (("random", 0.02), ("random", 0.0), ("blocks", 0.05)):
        m = make_key_mask(B, N, kind, seed=5201, p=p)
        for causal in (False, True):
            o, lse = run_masked_fwd(inp, m, "fp16", causal, 0.125)
            o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, 0.125, key_mask=m)
            _assert_masked_fwd(o, lse, o_ref, lse_ref, "fp16", "%s p=%g causal=%d" % (kind, p, causal))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,H", [(256, 64), (1000, 16)])
def test_fwd_masked_all_visible_is_bitwise_fwd(N, H, causal):
    # Sizes at which fa_fwd runs the 128-query kernel (at least one
    # 128-query tile per compute unit), the kernel the masked forward runs:
    # with every key visible the two share all arithmetic.
    inp = make_inputs(2, H, N, 128, "bf16", seed=5300)
    q, k, v = (to_dev(inp[n], "bf16") for n in ("q", "k", "v"))
    tiles = fa.mask_tiles(torch.ones(2, N, dtype=torch.uint8, device="cuda"))
    a = fa.fwd(q, k, v, causal=causal)
    b = fa.fwd_masked(q, k, v, tiles, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_masked_headline_shape_all_heads():
    """The headline shape (causal fp16 B1 H32 N8192 D128) with the seeded
    length mask the bench times (keys past a drawn length hidden): O, LSE
    and all gradients of every head against the oracle."""
    B, H, N, D = 1, 32, 8192, 128
    m = make_key_mask(B, N, "lengths", seed=3, p=0.5)
    say("masked headline shape, visible length %d, all heads" % int(m.sum()))
    inp = make_inputs(B, H, N, D, "fp16", seed=3, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o, lse = fa.fwd_masked(q, k, v, tiles, causal=True, scale=scale)
    dq, dk, dv = fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, scale, key_mask=m)
    _assert_masked_fwd(o, lse, o_ref, lse_ref, "fp16", "all %d heads" % H)
    del o_ref, lse_ref
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, scale, key_mask=m)
    got = [to_host(t) for t in (dq, dk, dv)]
    assert_grads_close(got, ref, "masked headline shape, all %d heads" % H)
    hidden = m[0] == 0
    assert np.all(got[1][0][:, hidden] == 0) and np.all(got[2][0][:, hidden] == 0)


def test_fwd_masked_long_sequences_sampled_heads():
    # the C2 geometry (H=32, N=4096, D=64) split over a padded batch of 2
    B, H, N, D = 2, 16, 4096, 64
    inp = make_inputs(B, H, N, D, "fp16", seed=5400)
    m = make_key_mask(B, N, "lengths", lengths=[4096, 2500])
    for causal in (False, True):
        o, lse = run_masked_fwd(inp, m, "fp16", causal, 0.125)
        for b, h in ((0, 0), (1, 5), (1, H - 1)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            o_ref, lse_ref = attention_forward(*(inp[n][sl] for n in ("q", "k", "v")), causal, 0.125,
                                               key_mask=m[b:b + 1])
            _assert_masked_fwd(o[sl], lse[sl], o_ref, lse_ref, "fp16", "b=%d h=%d causal=%d" % (b, h, causal))


def test_fwd_masked_writes_nothing_past_outputs():
    B, H, N, D = 1, 2, 300, 128
    inp = make_inputs(B, H, N, D, "fp16", seed=5500)
    q, k, v = (to_dev(inp[n], "fp16") for n in ("q", "k", "v"))
    m = make_key_mask(B, N, "blocks", seed=5501)
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    obuf = torch.full((q.numel() + 4096,), float("nan"), dtype=torch.float16, device="cuda")
    lbuf = torch.full((B * H * N + 4096,), float("nan"), dtype=torch.float32, device="cuda")
    o = obuf[:q.numel()].view(q.shape)
    lse = lbuf[:B * H * N].view(B, H, N)
    fa.fwd_masked(q, k, v, tiles, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isnan(obuf[q.numel():].float()).all() and torch.isnan(lbuf[B * H * N:]).all()
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, 1 / np.sqrt(D), key_mask=m)
    _assert_masked_fwd(o, lse, o_ref, lse_ref, "fp16", "guarded")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N,kind", [(2, 2, 200, "lengths"), (1, 2, 333, "blocks"), (2, 1, 256, "random")])
def test_bwd_masked(B, H, N, D, causal, dtype, kind):
    say("bwd masked B=%d H=%d N=%d D=%d causal=%d %s %s" % (B, H, N, D, causal, dtype, kind))
    inp = make_inputs(B, H, N, D, dtype, seed=5600 + N + D, with_dout=True)
    m = make_key_mask(B, N, kind, seed=5700 + N, p=0.3)
    scale = 1.0 / np.sqrt(D)
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o, lse = fa.fwd_masked(q, k, v, tiles, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale, key_mask=m)
    got = [to_host(t) for t in (dq, dk, dv)]
    assert_grads_close(got, ref, "N=%d %s" % (N, kind))
    hidden = m == 0
    for b in range(B):
        assert np.all(got[1][b][:, hidden[b]] == 0) and np.all(got[2][b][:, hidden[b]] == 0)
    empty = np.isneginf(to_host(lse))
    assert np.all(got[0][empty] == 0)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_masked_rows_without_keys(D):
    # at D = 128 the dK/dV accumulators of such rows start at -inf
    B, H, N = 1, 2, 150
    inp = make_inputs(B, H, N, D, "fp16", seed=5800, with_dout=True)
    m = make_key_mask(B, N, "random", seed=5801, p=0.05)
    m[0, :3] = 0  # causal rows 0..2 see no key
    q, k, v, do = (to_dev(inp[n], "fp16") for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o, lse = fa.fwd_masked(q, k, v, tiles, causal=True, scale=0.125)
    dq, dk, dv = fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=True, scale=0.125)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0, :, :3]).all() and (dq[0, :, :3] == 0).all()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.125, key_mask=m)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "sparse causal")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("kind", ["blocks", "random"])
def test_bwd_masked_one_head_in_parts(kind, causal, D):
    # one head of 1500 keys: both backward passes split into 3 parts; with
    # tile-structured masks the dQ parts divide the list of non-empty tiles
    B, H, N = 1, 1, 1500
    inp = make_inputs(B, H, N, D, "bf16", seed=5900 + D + causal, with_dout=True)
    m = make_key_mask(B, N, kind, seed=5901 + causal, p=0.5)
    q, k, v, do = (to_dev(inp[n], "bf16") for n in ("q", "k", "v", "do"))
    tiles = fa.mask_tiles(torch.from_numpy(m).cuda())
    o, lse = fa.fwd_masked(q, k, v, tiles, causal=causal, scale=0.1)
    dq, dk, dv = fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=causal, scale=0.1)
    torch.cuda.synchronize()
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, 0.1, key_mask=m)
    assert_grads_close([to_host(t) for t in (dq, dk, dv)], ref, "one head masked %s" % kind)
