"""Forward parity on the GPU: libfa's fa_fwd (through the C ABI) against the
float64 oracle on the same seeded inputs."""

import numpy as np
import pytest
import torch

import exact_attention_25_amd as fa
from exact_attention_25_amd import binding, workloads
from exact_attention_25_amd.inputs import make_inputs, round_to
from oracle import attention_forward
from parity import LSE_TOL, assert_fwd_close, o_error_ok, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def run_fwd(inp, dtype, causal, scale):
    q, k, v = (to_dev(inp[n], dtype) for n in ("q", "k", "v"))
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


# ---- small shapes: several tiles, a ragged last query tile, B and H > 1 ----
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B,H,N", [(1, 1, 64), (2, 3, 192), (1, 2, 320), (1, 1, 512)])
def test_fwd_small(B, H, N, D, causal, dtype):
    say("fwd small B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=1000 + N + D)
    scale = 1.0 / np.sqrt(D)
    o, lse = run_fwd(inp, dtype, causal, scale)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "N=%d D=%d" % (N, D))


# ---- launches smaller than the chip: the key-split forward ----
# Fewer 128-query tiles than compute units select fa_fwd_short.hip: 32 or 64
# queries per workgroup, keys split over its four waves, partial states
# merged in LDS.  The shapes cover two workgroups sharing a CU (D = 64: 512
# workgroups), ragged N, and long key walks (many passes over the V ring).
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N,D", [(1, 32, 512, 64), (1, 32, 512, 128), (2, 8, 1000, 128), (1, 4, 2500, 64),
                                     (1, 2, 4000, 128)])
def test_fwd_small_grid(B, H, N, D, causal, dtype):
    say("fwd small grid B=%d H=%d N=%d D=%d causal=%d %s" % (B, H, N, D, causal, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=1500 + N + D + H)
    scale = 1.0 / np.sqrt(D)
    o, lse = run_fwd(inp, dtype, causal, scale)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, scale)
    assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "B=%d H=%d N=%d D=%d" % (B, H, N, D))


# ---- the workloads at full size: every head against the oracle ----
def _sample_rows(n, count, rng):
    base = np.unique(np.concatenate([np.arange(0, min(n, 64)), np.arange(max(0, n - 64), n),
                                     np.arange(0, n, 64)[:64]]))
    extra = rng.choice(n, size=max(0, count - base.size), replace=False)
    return np.unique(np.concatenate([base, extra]))


WORKLOADS = [workloads.SMALL, workloads.NONCAUSAL_D64, *workloads.CAUSAL_D128.values(),
             workloads.FWDBWD_D64, workloads.LONG_BF16, workloads.FEW_HEADS_LONG]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fwd_causal_long_keys_one_tile_per_cu(dtype):
    """Causal, 256 tiles of 128 queries and N >= 8192: the key-split forward
    (its heaviest wave walks 64 of the 256 key tiles).  256 sampled query
    rows of each head -- the first and last 64, every 64th, the rest random --
    against the oracle."""
    B, H, N, D = 1, 2, 16384, 128
    assert fa.fwd_kernel_name(B, H, N, D, 1) == "fwd_short_pipe_kernel"
    say("fwd causal long keys B=%d H=%d N=%d %s" % (B, H, N, dtype))
    inp = make_inputs(B, H, N, D, dtype, seed=1700)
    scale = 1.0 / np.sqrt(D)
    o, lse = run_fwd(inp, dtype, True, scale)
    rows = _sample_rows(N, 256, np.random.default_rng(1701))
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, scale, rows=rows)
    assert_fwd_close(to_host(o)[:, :, rows], to_host(lse)[:, :, rows], o_ref, lse_ref, dtype,
                     "N=%d, %d rows per head" % (N, rows.size))


@pytest.mark.parametrize("w", WORKLOADS, ids=[w.name for w in WORKLOADS])
def test_fwd_workload(w):
    """The whole output of every head against the oracle (the golden-reference
    comparison of "FlashAttention dataflow and engineering validation on
    MI50", §5.1).  The workloads with N above 8192 (the long bf16 one and the
    one-head N = 16384 one) compare 512 sampled query rows -- the first and
    last 64, every 64th, the rest random -- of every one of their heads."""
    say("fwd workload %s" % w.name)
    inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, spiky_keys=w.spiky_keys)
    o, lse = run_fwd(inp, w.dtype, w.causal, w.scale)
    rng = np.random.default_rng(w.seed)
    rows = None if w.N <= 8192 else _sample_rows(w.N, 512, rng)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], w.causal, w.scale, rows=rows)
    og, lg = to_host(o), to_host(lse)
    if rows is not None:
        og, lg = og[:, :, rows], lg[:, :, rows]
    assert_fwd_close(og, lg, o_ref, lse_ref, w.dtype, "%s, all %d heads%s" % (
        w.name, w.B * w.H, "" if rows is None else ", %d rows each" % rows.size))
    if w.dtype == "bf16":  # the literal figures beside the per-element bound
        o_ref_b = round_to(o_ref.astype(np.float32), "bf16").astype(np.float64)
        say("  literal max abs error %.3e; against bf16(O_ref) %.3e" % (
            np.abs(og - o_ref).max(), np.abs(og - o_ref_b).max()))
    del o_ref, lse_ref
    # properties over the whole output
    on = to_host(o)
    assert np.all(np.isfinite(on))
    if w.causal:  # causal row 0 attends only to key 0
        v0 = inp["v"][:, :, 0, :]
        assert np.array_equal(on[:, :, 0, :], v0.astype(np.float64))


# ---- edge cases, on every forward kernel ----
# fa_fwd picks its kernel from the launch size alone, so an edge case with
# few heads would only reach the key-split kernel.  Each case below is also
# run with its heads repeated along H until the launch falls in the band of
# each other kernel (128-query tiles; 64 queries per wave at D = 128): every
# copy of a head must equal copy 0 bitwise (heads are independent and the
# kernels deterministic), and copy 0 is checked against the oracle.
def head_repeats(B, H, N, D, causal, cap=4096):
    """{kernel name: smallest head repeat factor r that makes fa_fwd on
    [B, H*r, N, D] run that kernel}."""
    out = {}
    for r in range(1, cap + 1):
        out.setdefault(fa.fwd_kernel_name(B, H * r, N, D, int(causal)), r)
    return out


def fwd_each_kernel(inp, dtype, causal, scale):
    """[(kernel name, O, LSE)] of the original heads, one entry per kernel."""
    B, H, N, D = inp["q"].shape
    dev = {n: to_dev(inp[n], dtype) for n in ("q", "k", "v")}
    res = []
    for name, r in sorted(head_repeats(B, H, N, D, causal).items(), key=lambda x: x[1]):
        q, k, v = (dev[n].repeat(1, r, 1, 1) for n in ("q", "k", "v"))
        assert fa.fwd_kernel_name(B, H * r, N, D, int(causal)) == name
        o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
        torch.cuda.synchronize()
        o5, l5 = o.view(B, r, H, N, D), lse.view(B, r, H, N)
        for i in range(1, r):
            assert torch.equal(o5[:, i], o5[:, 0]) and torch.equal(l5[:, i], l5[:, 0]), (name, i)
        say("  %s: %d copies of %d heads" % (name, r, B * H))
        res.append((name, o5[:, 0], l5[:, 0]))
        del q, k, v, o, lse
    return res


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_fwd_constant_keys_give_prefix_mean(causal, D):
    B, H, N = 1, 2, 256
    inp = make_inputs(B, H, N, D, "fp16", seed=5)
    inp["k"][:] = inp["k"][:, :, :1, :]
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, 0.125)
    for name, o, lse in fwd_each_kernel(inp, "fp16", causal, 0.125):
        assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, "fp16", "constant keys, " + name)


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_largest_fp16_scale_one(D):
    # every input 65504 with scale 1: all scores equal and huge
    x = np.full((1, 1, 128, D), 65504.0, dtype=np.float32)
    o_ref, lse_ref = attention_forward(x, x, x, True, 1.0)
    for name, o, lse in fwd_each_kernel({"q": x, "k": x, "v": x}, "fp16", True, 1.0):
        on, ln = to_host(o), to_host(lse)
        assert np.all(on == 65504.0), name
        # the score 65504^2*D is rounded to fp32 on the GPU: compare LSE relatively
        assert np.abs(ln - lse_ref).max() <= 1e-6 * np.abs(lse_ref).max(), name


@pytest.mark.parametrize("kind", ["rise", "fall"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,D", [(300, 64), (300, 128), (1100, 128)])
def test_fwd_reference_mode_transitions(kind, causal, N, D):
    """Rows whose running max crosses |scale*log2e*m| = 4096 mid-sequence.
    rise: keys 0-127 give scores of a few units, later keys about +-64*D
    (the reference is raised into the raw-score mode); fall: keys 0-127 give
    scores about -64*D (raw mode from the first tile), later keys a few
    units (the reference rises back into the one-FMA mode).  Every product
    and partial sum of the scores is a multiple of 1/512 below 2^14, so FP32
    accumulation is exact and the probabilities can be held to the usual
    bound even at these magnitudes.  N = 1100 reaches the pipelined form of
    the key-split kernel."""
    rng = np.random.default_rng(400 + D + 2 * causal + (kind == "fall") + (N > 1000))
    B, H = 1, 2
    ints = lambda lo, hi, *s: rng.integers(lo, hi, size=s).astype(np.float32)
    q = 8.0 + ints(-2, 3, B, H, N, D) / 8
    small = ints(-16, 17, B, H, N, D) / 64
    sign = np.where(rng.random((B, H, N, 1)) < 0.5, -1.0, 1.0).astype(np.float32)
    big = (8.0 + ints(-4, 5, B, H, N, D) / 8) * (sign if kind == "rise" else -1.0)
    first = np.arange(N)[None, None, :, None] < 128
    k = np.where(first, small if kind == "rise" else big, big if kind == "rise" else small).astype(np.float32)
    inp = {"q": q, "k": k, "v": round_to(rng.standard_normal((B, H, N, D)).astype(np.float32), "fp16")}
    assert np.array_equal(round_to(q, "fp16"), q) and np.array_equal(round_to(k, "fp16"), k)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], causal, 1.0)
    for name, o, lse in fwd_each_kernel(inp, "fp16", causal, 1.0):
        on, ln = to_host(o), to_host(lse)
        assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln)), name
        ok, max_abs, _ = o_error_ok(on, o_ref, "fp16")
        assert ok, "%s: O error %.3e" % (name, max_abs)
        # |LSE| reaches ~6e3 here: a few fp32 ulps of it on top of the usual bound
        assert np.all(np.abs(ln - lse_ref) <= LSE_TOL + 1e-6 * np.abs(lse_ref)), name


def score_rounding_bound(q, k, v, causal, scale, o_ref, lse_ref):
    """First-order bound on |O - O_exact| from the FP32 accumulation of each
    score's D-term dot product (the pages keep S in FP32): a sum of D
    products errs by at most gamma_D * sum_i |q_i k_i| with
    gamma_D = D u / (1 - D u), u = 2^-24, and score errors ds_k move O_ij by
    at most sum_k P_ik |V_kj - O_ij| ds_ik.  Float64, per output element."""
    D = q.shape[-1]
    u = 2.0 ** -24
    gamma = D * u / (1 - D * u)
    out = np.zeros_like(o_ref)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            qh, kh, vh = (x[b, h].astype(np.float64) for x in (q, k, v))
            s = qh @ kh.T * scale
            ds = np.abs(qh) @ np.abs(kh).T * scale * gamma
            if causal:
                above = np.triu(np.ones(s.shape, dtype=bool), 1)
                s, ds = np.where(above, -np.inf, s), np.where(above, 0.0, ds)
            w = np.exp(s - lse_ref[b, h][:, None]) * ds
            out[b, h] = np.einsum("ik,ikj->ij", w, np.abs(vh[None, :, :] - o_ref[b, h][:, None, :]))
    return out


@pytest.mark.parametrize("D", [64, 128])
def test_fwd_plus_minus_1e4_mixture(D):
    """Inputs of magnitude up to 1e4 with scale 1e-4: scores near 5e4 whose
    FP32 dot products carry rounding errors of a few hundredths (partial
    sums near 5e8), which values near 1e4 magnify in O.  The tolerance adds
    that rounding bound (score_rounding_bound, with a tenth of margin for
    second-order terms) to the fp16 bound taken relative to |O|."""
    rng = np.random.default_rng(11 + D)
    B, H, N = 1, 2, 192
    inp = {n: round_to(rng.choice([-1e4, 1e4, 1.0, -1.0], size=(B, H, N, D)).astype(np.float32)
                       * rng.random((B, H, N, D)).astype(np.float32), "fp16") for n in ("q", "k", "v")}
    scale = 1e-4
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, scale)
    # outputs reach 1e4, so the fp16 output tolerance is relative to fp16 spacing there
    tol = 2e-3 + np.abs(o_ref) * 2.0 ** -10 + 1.1 * score_rounding_bound(
        inp["q"], inp["k"], inp["v"], True, scale, o_ref, lse_ref)
    for name, o, lse in fwd_each_kernel(inp, "fp16", True, scale):
        on = to_host(o)
        assert np.all(np.isfinite(on)), name
        assert np.all(np.abs(on - o_ref) <= tol), name
        assert np.abs(to_host(lse) - lse_ref).max() <= 1e-3 * max(1.0, np.abs(lse_ref).max()), name


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fwd_nondefault_scale(dtype):
    inp = make_inputs(2, 1, 256, 128, dtype, seed=21)
    o_ref, lse_ref = attention_forward(inp["q"], inp["k"], inp["v"], True, 0.3)
    for name, o, lse in fwd_each_kernel(inp, dtype, True, 0.3):
        assert_fwd_close(to_host(o), to_host(lse), o_ref, lse_ref, dtype, "scale 0.3, " + name)


def test_fwd_is_bitwise_deterministic():
    inp = make_inputs(1, 8, 1024, 128, "fp16", seed=3)
    a = run_fwd(inp, "fp16", True, 1 / np.sqrt(128))
    b = run_fwd(inp, "fp16", True, 1 / np.sqrt(128))
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fwd_rejects_misaligned_and_unsupported_on_device():
    q = torch.zeros(1, 1, 129 * 64 + 1, dtype=torch.float16, device="cuda")
    bad = q.view(-1)[1:].view(1, 1, 129, 64)  # 2-byte offset base
    good = torch.zeros(1, 1, 129, 64, dtype=torch.float16, device="cuda")
    o = torch.empty_like(good)
    lse = torch.empty(1, 1, 129, dtype=torch.float32, device="cuda")
    st = binding.fa_fwd(bad.data_ptr(), good.data_ptr(), good.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        1, 1, 128, 64, 0, 0.125, 0, torch.cuda.current_stream().cuda_stream)
    assert st == 4
    d96 = torch.zeros(1, 1, 129, 96, dtype=torch.float16, device="cuda")
    with pytest.raises(binding.FaError):
        fa.fwd(d96, d96, d96)  # head dimension 96 is not supported
