"""Helpers for GPU-vs-oracle parity tests (imported by the gpu tests only).

Tolerances (written here, applied element by element):
* fp16 O:  max |O_gpu - O_ref| <= 2e-3.
* bf16 O:  |O_gpu - O_ref| <= 1e-2 + half a bf16 ulp of |O_ref|, per element.
  A bare 1e-2 is unreachable for bf16 storage: rounding the exact result to
  bf16 alone errs by up to 1.56e-2 where |O| is in [4, 8).
* LSE:     max |LSE_gpu - LSE_ref| <= 1e-3.
* dQ, dK, dV: ||G_gpu - G_ref||_F / ||G_ref||_F <= 2e-2, per tensor.
"""

import math
import sys

import numpy as np
import torch

FP16_O_TOL = 2e-3
BF16_O_TOL = 1e-2
LSE_TOL = 1e-3
GRAD_REL_TOL = 2e-2

TORCH_DTYPE = {"fp16": torch.float16, "bf16": torch.bfloat16}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(x, dtype):
    """float32 numpy (values exact in dtype) -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(TORCH_DTYPE[dtype]).contiguous()


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def half_ulp_bf16(x):
    """Half of the bf16 spacing at |x| (2^(e-8) for |x| in [2^e, 2^(e+1)))."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    e = np.floor(np.log2(ax))
    return np.ldexp(1.0, (e - 8).astype(np.int64))


def o_error_ok(o_gpu, o_ref, dtype):
    """(passed, max_abs, worst_excess) for the output tolerance of dtype."""
    err = np.abs(o_gpu - o_ref)
    if dtype == "fp16":
        bound = np.full_like(err, FP16_O_TOL)
    else:
        bound = BF16_O_TOL + half_ulp_bf16(o_ref)
    excess = float((err - bound).max()) if err.size else -1.0
    return excess <= 0.0, float(err.max()) if err.size else 0.0, excess


def assert_fwd_close(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    ok, max_abs, excess = o_error_ok(o_gpu, o_ref, dtype)
    lse_err = float(np.abs(lse_gpu - lse_ref).max()) if lse_ref.size else 0.0
    say("  %s: O max abs err %.3e (excess over bound %.3e), LSE max abs err %.3e" % (what, max_abs, excess, lse_err))
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))
    assert ok, "%s: O error %.3e exceeds the %s bound" % (what, max_abs, dtype)
    assert lse_err <= LSE_TOL, "%s: LSE error %.3e" % (what, lse_err)


def rel_fro(g_gpu, g_ref):
    den = math.sqrt(float((g_ref ** 2).sum()))
    num = math.sqrt(float(((g_gpu - g_ref) ** 2).sum()))
    return num / den if den > 0 else num


def assert_grads_close(gpu, ref, what=""):
    for name, a, b in zip(("dQ", "dK", "dV"), gpu, ref):
        assert np.all(np.isfinite(a)), "%s %s has non-finite values" % (what, name)
        r = rel_fro(a, b)
        say("  %s: %s relative Frobenius error %.3e" % (what, name, r))
        assert r <= GRAD_REL_TOL, "%s: %s relative error %.3e" % (what, name, r)
