"""Backward parity on the GPU: fa_fwd then fa_bwd (through the C ABI) against
the float64 oracle's gradients on the same seeded inputs."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd import workloads
from exact_attention_25_amd.inputs import make_inputs, round_to
from oracle import attention_backward, attention_forward
from parity import GRAD_REL_TOL, LSE_TOL, assert_grads_close, o_error_ok, rel_fro, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_fwd_bwd(inp, dtype, causal, scale):
    q, k, v, do = (to_dev(inp[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 1, 64), (2, 3, 192), (1, 2, 320)])
def test_bwd_small(B, H, N, D, causal, dtype):
    say("bwd small B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=2000 + N + D, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    got = [to_host(t) for t in run_fwd_bwd(inp, dtype, causal, scale)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close(got, ref, "N=%d D=%d" % (N, D))


def test_bwd_workload_all_heads():
    """dQ, dK, dV of the fwd+bwd workload against the oracle over the whole
    [B, H, N, D] tensors (relative Frobenius error per gradient), and the
    worst head reported beside it."""
    w = workloads.FWDBWD_D64
    say("bwd workload %s" % w.name)
    inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, with_dout=True)
    got = [to_host(t) for t in run_fwd_bwd(inp, w.dtype, w.causal, w.scale)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.causal, w.scale)
    assert_grads_close(got, ref, "%s, all %d heads" % (w.name, w.B * w.H))
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        worst = max((rel_fro(g[b, h], r[b, h]), b, h) for b in range(w.B) for h in range(w.H))
        say("  %s worst head (%d,%d): relative Frobenius error %.3e" % (name, worst[1], worst[2], worst[0]))
        assert worst[0] <= GRAD_REL_TOL


def test_bwd_headline_shape_all_heads():
    """The backward at the shapes whose throughput the bench reports beside
    the forward (causal fp16 B1 H32 N8192 D128, with a seeded dO): dQ, dK,
    dV against the oracle over every head."""
    w = workloads.CAUSAL_D128[8192]
    say("bwd headline shape %s, all heads" % w.name)
    inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, with_dout=True)
    got = [to_host(t) for t in run_fwd_bwd(inp, w.dtype, w.causal, w.scale)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], w.causal, w.scale)
    assert_grads_close(got, ref, "%s bwd, all %d heads" % (w.name, w.B * w.H))
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        worst = max((rel_fro(g[b, h], r[b, h]), b, h) for b in range(w.B) for h in range(w.H))
        say("  %s worst head (%d,%d): relative Frobenius error %.3e" % (name, worst[1], worst[2], worst[0]))
        assert worst[0] <= GRAD_REL_TOL


def test_bwd_long_bf16_sampled_heads():
    """The backward of the long bf16 workload (causal B1 H16 N32768 D128,
    every 64th key scaled by 8) on the GPU over all heads; dQ, dK, dV of its
    first and last heads -- whole heads, since dK and dV sum over every
    query -- against the oracle."""
    w = workloads.LONG_BF16
    say("bwd %s, heads 0 and %d against the oracle" % (w.name, w.H - 1))
    inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, spiky_keys=w.spiky_keys, with_dout=True)
    got = [to_host(t) for t in run_fwd_bwd(inp, w.dtype, w.causal, w.scale)]
    hs = [0, w.H - 1]
    for name, g in zip(("dQ", "dK", "dV"), got):
        assert np.all(np.isfinite(g)), name
    sub = {n: np.ascontiguousarray(inp[n][:, hs]) for n in ("q", "k", "v", "do")}
    ref = attention_backward(sub["q"], sub["k"], sub["v"], sub["do"], w.causal, w.scale)
    assert_grads_close([g[:, hs] for g in got], ref, "%s, heads %s" % (w.name, hs))


def test_bwd_scale_and_bf16_long_rows():
    inp = make_inputs(1, 2, 1024, 128, "bf16", seed=77, spiky_keys=True, with_dout=True)
    got = [to_host(t) for t in run_fwd_bwd(inp, "bf16", True, 0.2)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, 0.2)
    assert_grads_close(got, ref, "bf16 spiky N=1024 scale 0.2")


def test_bwd_is_bitwise_deterministic():
    inp = make_inputs(1, 4, 512, 64, "fp16", seed=9, with_dout=True)
    a = run_fwd_bwd(inp, "fp16", True, 0.125)
    b = run_fwd_bwd(inp, "fp16", True, 0.125)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [2.0 ** -64, 2.0 ** -20, 4.0])
def test_bwd_extreme_scales(D, scale):
    # The smallest accepted scale (2^-64: P is uniform to FP32 precision and
    # dQ, dK are ~2^-64, still normal in bf16), a small one, and a large one
    # (peaked rows).  At D = 128 the dK/dV kernel starts its accumulators at
    # -LSE/scale, which is ~1e20 at the smallest scale.
    say("bwd scale %g D=%d" % (scale, D))
    inp = make_inputs(1, 2, 192, D, "bf16", seed=7700 + D, with_dout=True)
    got = [to_host(t) for t in run_fwd_bwd(inp, "bf16", True, scale)]
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], True, scale)
    assert_grads_close(got, ref, "scale %g D=%d" % (scale, D))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_one_head_split_into_parts(D, causal):
    # B*H*ceil(N/128) = 12 workgroups: the dK/dV pass splits each key tile's
    # 24 query tiles into 3 parts (8 each, the last tile ragged), the dQ pass
    # each query tile's key tiles into 3 parts, and both add their FP32
    # partial sums in part order
    B, H, N = 1, 1, 1500
    assert fa.bwd_workspace_bytes(B, H, N, D, causal, 0) == 6144 + 2 * 3 * N * D * 4 + 3 * N * D * 4
    say("bwd one head in parts N=%d D=%d causal=%d" % (N, D, causal))
    inp = make_inputs(B, H, N, D, "fp16", seed=7800 + D + causal, with_dout=True)
    scale = 1.0 / np.sqrt(D)
    a = run_fwd_bwd(inp, "fp16", causal, scale)
    b = run_fwd_bwd(inp, "fp16", causal, scale)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ref = attention_backward(inp["q"], inp["k"], inp["v"], inp["do"], causal, scale)
    assert_grads_close([to_host(t) for t in a], ref, "one head N=%d D=%d" % (N, D))


def rounding_bounds(q, k, v, do, o_dev, lse_dev, causal, scale, u, tiny):
    """Per-element bounds on the error of dQ, dK, dV of the kernels, from the
    rounding their intermediates carry: P is rebuilt from the forward's FP32
    LSE (lse_dev), Delta from the forward's stored output (o_dev), and P and
    dS are rounded to a type of unit roundoff u (relative, and tiny below
    the type's normal range, where the spacing is 2*tiny) before the
    products.  A sum of a_j b_j with each a_j off by e_j is off by at most
    sum e_j |b_j|; the perturbations of P and Delta are evaluated exactly in
    float64 from the kernels' own LSE and O (which the kernels' FP32
    evaluation of P perturbs again at the 1e-4 level), and every term is
    taken twice over.  (Float64 magnitudes, for the bound only.)"""
    qd, kd, vd, dod = (x.astype(np.float64) for x in (q, k, v, do))
    s_ = scale * qd @ np.swapaxes(kd, -1, -2)
    if causal:
        n = s_.shape[-1]
        s_ = np.where(np.tril(np.ones((n, n), dtype=bool)), s_, -np.inf)
    m = s_.max(-1, keepdims=True)
    lse = m + np.log(np.exp(s_ - m).sum(-1, keepdims=True))
    p = np.exp(s_ - lse)
    p_k = np.exp(s_ - lse_dev[..., None])            # P as the kernels rebuild it
    dp = dod @ np.swapaxes(vd, -1, -2)
    delta = (p * dp).sum(-1, keepdims=True)
    delta_k = (dod * o_dev).sum(-1, keepdims=True)   # Delta from the stored O
    ds = p * (dp - delta)
    ds_k = p_k * (dp - delta_k)
    e_ds = 4 * u * np.abs(ds_k) + 2 * tiny + 2 * np.abs(ds_k - ds) + 2.0 ** -20 * p_k * (np.abs(dp) + np.abs(delta_k))
    e_p = 4 * u * p_k + 2 * tiny + 2 * np.abs(p_k - p)
    b_dq = scale * e_ds @ np.abs(kd)
    b_dk = scale * np.swapaxes(e_ds, -1, -2) @ np.abs(qd)
    b_dv = np.swapaxes(e_p, -1, -2) @ np.abs(dod)
    return b_dq, b_dk, b_dv


@pytest.mark.parametrize("kind", ["rise", "fall"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_bwd_huge_scores(kind, causal, D):
    # scores of about +-64*D next to scores of a few units (the inputs of the
    # forward's reference-mode test): the backward rebuilds P from an LSE of
    # magnitude ~64*D, which at D = 128 means accumulators starting near
    # -8192 / scale.  The rows are nearly one-hot, so dS = P (dP - Delta)
    # cancels and dQ is small next to the terms that make it: the relative
    # Frobenius bound does not apply; the rounding of the kernels' own
    # intermediates (LSE and O from the forward, P and dS in fp16) does.
    rng = np.random.default_rng(900 + D + 2 * causal + (kind == "fall"))
    B, H, N = 1, 2, 300
    ints = lambda lo, hi, *s: rng.integers(lo, hi, size=s).astype(np.float32)
    q = 8.0 + ints(-2, 3, B, H, N, D) / 8
    small = ints(-16, 17, B, H, N, D) / 64
    sign = np.where(rng.random((B, H, N, 1)) < 0.5, -1.0, 1.0).astype(np.float32)
    big = (8.0 + ints(-4, 5, B, H, N, D) / 8) * (sign if kind == "rise" else -1.0)
    first = np.arange(N)[None, None, :, None] < 128
    k = np.where(first, small if kind == "rise" else big, big if kind == "rise" else small).astype(np.float32)
    v = round_to(rng.standard_normal((B, H, N, D)).astype(np.float32), "fp16")
    do = round_to(rng.standard_normal((B, H, N, D)).astype(np.float32), "fp16")
    say("bwd huge scores %s D=%d causal=%d" % (kind, D, causal))
    qd, kd, vd, dod = (to_dev(x, "fp16") for x in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, scale=1.0)
    grads = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, scale=1.0)
    torch.cuda.synchronize()
    # The bounds below are built from the forward's own O and LSE, so those
    # are first held to the oracle: fp16 O within the output tolerance, LSE
    # (magnitude up to ~64*D here) within LSE_TOL plus a few FP32 ulps of it.
    o_ref, lse_ref = attention_forward(q, k, v, causal, 1.0)
    on, ln = to_host(o), to_host(lse)
    ok, max_abs, _ = o_error_ok(on, o_ref, "fp16")
    assert ok, "forward O error %.3e" % max_abs
    assert np.all(np.abs(ln - lse_ref) <= LSE_TOL + 1e-6 * np.abs(lse_ref)), "forward LSE"
    ref = attention_backward(q, k, v, do, causal, 1.0)
    bounds = rounding_bounds(q, k, v, do, to_host(o), to_host(lse), causal, 1.0, 2.0 ** -11, 2.0 ** -25)
    for name, t, r, bnd in zip(("dQ", "dK", "dV"), grads, ref, bounds):
        g = to_host(t)
        assert np.all(np.isfinite(g))
        err = np.abs(g - r)
        lim = bnd + 2.0 ** -11 * np.abs(r) + 1e-6  # + the rounding of the result itself
        say("  %s: max error %.3e, worst error / bound %.3f" % (name, err.max(), (err / lim).max()))
        assert np.all(err <= lim), name
