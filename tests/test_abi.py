"""C ABI checks that need no GPU: the library loads, exports every function
include/fa.h declares, and rejects bad arguments before anything is launched."""

import ctypes
import os
import re

import pytest

from exact_attention_25_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# fake but 16-byte-aligned, non-null "device" addresses: never dereferenced,
# because every call below fails argument checks first
P = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_ex", "fa_bwd_ex_workspace_bytes", "fa_bwd_noalloc",
                                    "fa_bwd_workspace_bytes", "fa_dropout_mask", "fa_fwd", "fa_fwd_ex",
                                    "fa_fwd_ex_workspace_bytes", "fa_fwd_kernel_name", "fa_fwd_splitkv_num_splits",
                                    "fa_mask_tiles", "fa_mask_tiles_bytes", "fa_status_str"]


def test_options_struct_layout_matches_the_header(tmp_path):
    """The binding's FaOptions has the size and field offsets of struct
    fa_options as a C compiler lays it out from include/fa.h."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "layout.c"
    fields = [f[0] for f in fb.FaOptions._fields_]
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fa.h"\nint main(void) {\n'
                   '  fa_options d = FA_OPTIONS_DEFAULT; (void)d;\n  printf("%zu", sizeof(fa_options));\n' +
                   "".join('  printf(" %%zu", offsetof(fa_options, %s));\n' % f for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got == [ctypes.sizeof(fb.FaOptions)] + [getattr(fb.FaOptions, f).offset for f in fields]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fb.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert fb.status_str(0) == "FA_OK"
    for code in range(1, 8):
        assert fb.status_str(code).startswith("FA_ERR_")
    assert "unknown" in fb.status_str(99)


def fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=2, N=128, D=64, causal=1, scale=0.125, dtype=0, stream=None)
    a.update(kw)
    return fb.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"],
                     a["causal"], a["scale"], a["dtype"], a["stream"])


def bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, N=128, D=64, causal=1,
             scale=0.125, dtype=0, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return fb.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                     a["B"], a["H"], a["N"], a["D"], a["causal"], a["scale"], a["dtype"], a["ws"],
                     a["wsb"], a["stream"])


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse"])
def test_fwd_null(name):
    assert fwd(**{name: None}) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(H=-1), 2), (dict(N=0), 2),
    (dict(D=96), 3), (dict(D=256), 3), (dict(dtype=2), 3), (dict(causal=2), 3),
    (dict(N=(1 << 30) + 1), 2), (dict(scale=0.0), 3), (dict(scale=-1.0), 3),
    (dict(scale=float("inf")), 3), (dict(scale=float("nan")), 3), (dict(scale=2.0 ** -65), 3),
    (dict(q=P + 2), 4), (dict(o=P + 8), 4), (dict(lse=P + 4), 4),
    (dict(B=1 << 40, H=1 << 30), 2),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null(name):
    assert bwd(**{name: None}) == 1


@pytest.mark.parametrize("kw,code", [
    (dict(N=(1 << 30) + 64), 2), (dict(D=32), 3), (dict(dk=P + 2), 4), (dict(ws=None), 5),
    (dict(wsb=4 * 2 * 128 - 1), 5), (dict(ws=P + 4), 4), (dict(H=0), 2),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_workspace_bytes():
    assert fb.bwd_workspace_bytes(2, 3, 128, 64, 1, 0) == 2 * 3 * 128 * 4
    assert fb.bwd_workspace_bytes(1, 1, 64, 128, 0, 1) == 256
    assert fb.bwd_workspace_bytes(1, 1, 100, 64, 0, 0) == 512  # any N: 400 bytes, rounded up
    assert fb.bwd_workspace_bytes(1, 1, 100, 96, 0, 0) == 0


def fwd_ex(opt, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=4, N=256, D=64, causal=1, scale=0.125, dtype=0, ws=P, wsb=1 << 30)
    a.update(kw)
    return fb.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"], a["causal"],
                        a["scale"], a["dtype"], opt, a["ws"], a["wsb"], None)


def bwd_ex(opt, **kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=4, N=128, D=128, causal=0, scale=0.1,
             dtype=1, ws=P, wsb=1 << 30)
    a.update(kw)
    return fb.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                        a["H"], a["N"], a["D"], a["causal"], a["scale"], a["dtype"], opt, a["ws"], a["wsb"], None)


def bad_flag():
    o = fb.options()
    o.dropout = 2
    return o


ALL = dict(h_kv=2, tiles=P, dropout=(0.1, 1, 0))  # every option at once (a valid combination)


@pytest.mark.parametrize("opt,kw,code", [
    (None, dict(q=None), 1), (fb.options(), dict(lse=None), 1), (fb.options(**ALL, num_splits=3), dict(k=None), 1),
    (fb.options(h_kv=3), {}, 2), (fb.options(h_kv=-1), {}, 2), (fb.options(h_kv=5), {}, 2),
    (fb.options(**ALL), dict(N=-1), 2), (fb.options(**ALL, num_splits=2), dict(B=0), 2),
    (fb.options(tiles=P + 4), {}, 4), (fb.options(**ALL), dict(o=P + 2), 4), (fb.options(h_kv=2), dict(v=P + 2), 4),
    (bad_flag(), {}, 3), (fb.options(dropout=(1.0, 1, 0)), {}, 3), (fb.options(dropout=(-0.1, 1, 0)), {}, 3),
    (fb.options(dropout=(float("nan"), 1, 0)), {}, 3), (fb.options(**ALL), dict(D=80), 3),
    (fb.options(num_splits=65), {}, 3), (fb.options(num_splits=-1), {}, 3),
    (fb.options(num_splits=4), dict(ws=None), 5), (fb.options(**ALL, num_splits=4), dict(wsb=1000), 5),
    (fb.options(num_splits=4), dict(ws=P + 8), 4),
])
def test_fwd_ex_rejects(opt, kw, code):
    assert fwd_ex(opt, **kw) == code


@pytest.mark.parametrize("opt,kw,code", [
    (None, dict(dq=None), 1), (fb.options(**ALL), dict(dk=None), 1),
    (fb.options(h_kv=3), {}, 2), (fb.options(**ALL), dict(H=0), 2),
    (fb.options(tiles=P + 4), {}, 4), (fb.options(**ALL), dict(ws=P + 4), 4),
    (fb.options(dropout=(1.5, 1, 0)), {}, 3), (bad_flag(), {}, 3), (fb.options(**ALL), dict(dtype=3), 3),
    (fb.options(**ALL), dict(ws=None), 5), (fb.options(h_kv=1), dict(wsb=4 * 4 * 128 - 1), 5),
])
def test_bwd_ex_rejects(opt, kw, code):
    assert bwd_ex(opt, **kw) == code


def test_fwd_ex_workspace_bytes():
    rows = 2 * 3 * 128 * 4
    assert fb.fwd_ex_workspace_bytes(2, 3, 128, 64, 1, 0, fb.options(num_splits=4)) == rows * 4 + rows * 64 * 4
    assert fb.fwd_ex_workspace_bytes(1, 1, 64, 128, 0, 0, fb.options(num_splits=1)) == 256 + 64 * 128 * 4
    # with grouped heads and the other options the states are still per query head
    rows = 2 * 4 * 300 * 3  # 28800 bytes of LSE, rounded up to 28928
    assert fb.fwd_ex_workspace_bytes(2, 4, 300, 64, 1, 0, fb.options(h_kv=2, tiles=P, dropout=(0.1, 1, 0),
                                                                     num_splits=3)) == 28928 + rows * 64 * 4
    # one pass needs none; rejected options give 0
    assert fb.fwd_ex_workspace_bytes(1, 1, 64, 128, 0, 0, None) == 0
    assert fb.fwd_ex_workspace_bytes(1, 1, 64, 128, 0, 0, fb.options(num_splits=0)) == 0
    assert fb.fwd_ex_workspace_bytes(1, 1, 64, 128, 0, 0, fb.options(num_splits=65)) == 0
    assert fb.fwd_ex_workspace_bytes(1, 4, 64, 128, 0, 0, fb.options(h_kv=3, num_splits=2)) == 0


def test_bwd_ex_workspace_bytes():
    kv = lambda h: fb.options(h_kv=h)
    # H_kv = H (or no options): Delta only, as fa_bwd_workspace_bytes
    assert fb.bwd_ex_workspace_bytes(2, 4, 100, 64, 1, 0, kv(4)) == fb.bwd_workspace_bytes(2, 4, 100, 64, 1, 0)
    assert fb.bwd_ex_workspace_bytes(2, 4, 100, 64, 1, 0, None) == fb.bwd_workspace_bytes(2, 4, 100, 64, 1, 0)
    # enough workgroups (B*H_kv*ceil(N/128) >= 1024): one part, Delta only
    assert fb.bwd_ex_workspace_bytes(1, 64, 16384, 128, 1, 0, kv(8)) == 64 * 16384 * 4
    # MQA, B1 H32 N8192: 64 workgroups -> 16 parts of FP32 dK and dV partials
    delta = 32 * 8192 * 4
    part = 16 * 8192 * 128 * 4
    assert fb.bwd_ex_workspace_bytes(1, 32, 8192, 128, 1, 0, kv(1)) == delta + 2 * part
    # parts never exceed the group size
    assert fb.bwd_ex_workspace_bytes(1, 2, 64, 64, 0, 1, kv(1)) == 2 * 64 * 4 + 2 * 2 * 64 * 64 * 4
    assert fb.bwd_ex_workspace_bytes(1, 4, 64, 64, 0, 0, kv(3)) == 0
    # the mask and dropout options need no more; num_splits is ignored by the backward
    assert fb.bwd_ex_workspace_bytes(1, 32, 8192, 128, 1, 0, fb.options(h_kv=1, tiles=P, dropout=(0.2, 3, 4),
                                                                        num_splits=99)) == delta + 2 * part


@pytest.mark.parametrize("shape,splits", [
    ((1, 1, 16384, 128, 0), 4), ((1, 2, 16384, 128, 0), 2), ((1, 1, 32768, 128, 1), 2),
    ((1, 4, 8192, 128, 0), 2), ((2, 8, 2048, 128, 0), 1), ((1, 32, 8192, 128, 1), 1),
    ((1, 1, 4096, 64, 0), 2), ((1, 1, 2 ** 20, 64, 1), 1), ((1, 1, 100, 64, 0), 1),
    ((0, 1, 64, 64, 0), 0), ((1, 1, 64, 96, 0), 0), ((1, 1, 64, 64, 2), 0),
])
def test_splitkv_num_splits(shape, splits):
    # doubling from 1 while B*H*ceil(N/128)*S < 512, N/(2S) >= 2048 and S < 16;
    # the first six shapes are those measured (their fastest split count)
    assert fb.splitkv_num_splits(*shape) == splits


def test_mask_tiles_bytes():
    # T = 3 tiles: words 8*2*3 -> 256, prefix 4*2*4 -> 256, list 4*2*3 -> 256
    assert fb.fa_mask_tiles_bytes(2, 130) == 768
    assert fb.fa_mask_tiles_bytes(1, 64 * 100) == 1024 + 512 + 512
    assert fb.fa_mask_tiles_bytes(0, 10) == 0 and fb.fa_mask_tiles_bytes(1, 0) == 0
    assert fb.fa_mask_tiles_bytes(1, (1 << 30) + 1) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), 1), (dict(B=0), 2), (dict(N=0), 2), (dict(N=(1 << 30) + 1), 2),
    (dict(tiles=None), 5), (dict(nb=767), 5), (dict(tiles=P + 8), 4),
])
def test_mask_tiles_rejects(kw, code):
    a = dict(mask=P, B=2, N=130, tiles=P, nb=768)
    a.update(kw)
    assert fb.fa_mask_tiles(a["mask"], a["B"], a["N"], a["tiles"], a["nb"], None) == code


@pytest.mark.parametrize("kw,code", [(dict(keep=None), 1), (dict(N=0), 2), (dict(N=(1 << 24) + 1), 2),
                                     (dict(p=1.0), 3)])
def test_dropout_mask_rejects(kw, code):
    a = dict(keep=P, B=1, H=1, N=64, p=0.5, seed=1, offset=0)
    a.update(kw)
    assert fb.fa_dropout_mask(a["keep"], a["B"], a["H"], a["N"], a["p"], a["seed"], a["offset"], None) == code


CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_client")


def test_c_client_argument_errors(tmp_path):
    """The torch-free client (built by build()) links against libfa.so and
    rejects bad invocations before any GPU call: exit 2 with a message."""
    import subprocess
    if not os.path.exists(CLIENT):
        pytest.skip("tests/c_abi_client is not built (build() compiles it)")
    res = subprocess.run([CLIENT], capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "usage" in res.stderr
    missing = str(tmp_path / "absent.bin")
    res = subprocess.run([CLIENT, missing, str(tmp_path / "o.bin"), "1", "1", "64", "64", "0", "0", "0.125"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2 and "cannot read" in res.stderr
    res = subprocess.run([CLIENT, missing, str(tmp_path / "o.bin"), "1", "0", "64", "64", "0", "0", "0.125"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2


def test_bwd_noalloc_argument_errors_and_scratch_limit():
    """fa_bwd_noalloc checks its arguments like fa_bwd, then rejects shapes
    whose workspace exceeds its static scratch (32 MiB) with
    FA_ERR_SCRATCH_LIMIT -- all before any GPU call."""
    def call(**kw):
        a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, H=2, N=128, D=64, causal=1,
                 scale=0.125, dtype=0)
        a.update(kw)
        return fb.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                                 a["B"], a["H"], a["N"], a["D"], a["causal"], a["scale"], a["dtype"], None)
    assert call(dq=None) == 1
    assert call(N=0) == 2
    assert call(D=96) == 3
    assert call(dv=P + 2) == 4
    # Delta alone: 4 bytes per query row -- 8M rows fill the scratch exactly
    assert fb.bwd_workspace_bytes(1, 64, 1 << 17, 64, 1, 0) == 32 << 20
    assert call(B=1, H=65, N=1 << 17, D=64) == 7
    # one head of 65536 rows: partial dK/dV and dQ sums of 64 MiB each
    assert fb.bwd_workspace_bytes(1, 1, 1 << 16, 128, 1, 0) > 32 << 20
    assert call(B=1, H=1, N=1 << 16, D=128) == 7
    assert "scratch" in fb.status_str(7)


def test_fwd_kernel_name_follows_the_launch_size():
    # no GPU work: the choice is made on the host from the shape alone
    assert fb.fwd_kernel_name(1, 32, 8192, 128, 1) == "fwd_d128_kernel"   # 1024 tiles of 256 queries
    assert fb.fwd_kernel_name(1, 16, 32768, 128, 1) == "fwd_d128_kernel"
    assert fb.fwd_kernel_name(1, 32, 4096, 128, 1) == "fwd_kernel"        # 512 tiles of 256 queries
    assert fb.fwd_kernel_name(1, 32, 4096, 64, 0) == "fwd_kernel"         # D = 64: never the D=128 kernel
    assert fb.fwd_kernel_name(1, 32, 1024, 128, 1) == "fwd_kernel"        # 256 tiles of 128 queries
    assert fb.fwd_kernel_name(1, 1, 32768, 128, 1) == "fwd_short_pipe_kernel"  # 256 tiles, causal, long keys
    assert fb.fwd_kernel_name(1, 1, 32768, 128, 0) == "fwd_kernel"        # the same, not causal
    assert fb.fwd_kernel_name(1, 2, 32768, 128, 1) == "fwd_kernel"        # 512 tiles
    assert fb.fwd_kernel_name(1, 32, 512, 128, 1) == "fwd_short_kernel"   # 128 tiles of 128 queries
    assert fb.fwd_kernel_name(1, 1, 256, 64, 0) == "fwd_short_kernel"
    assert fb.fwd_kernel_name(1, 1, 16384, 128, 0) == "fwd_short_pipe_kernel"  # pipelined from N = 1024
    assert fb.fwd_kernel_name(1, 16, 1024, 128, 1) == "fwd_short_pipe_kernel"
    assert fb.fwd_kernel_name(1, 8, 1000, 128, 1) == "fwd_short_kernel"
    assert fb.fwd_kernel_name(1, 1, 64, 96, 0) == ""                      # unsupported D
    assert fb.fwd_kernel_name(0, 1, 64, 64, 0) == ""
