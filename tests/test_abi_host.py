"""The C-ABI library on the host: it loads, exports what the header declares, and
rejects bad arguments before touching the GPU.

No kernel is launched here. Acceptance checks go through flash_attn_fwd_validate
(which never launches); flash_attn_fwd itself is only called with arguments that
fail validation or describe an empty problem, both of which return before any
HIP call. Fake addresses are never dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_flash_amd as fa
from exact_attention_flash_amd import _native
from exact_attention_flash_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

A = 0x10000000          # 16-byte aligned fake device addresses, 1 GiB apart
GB = 1 << 30
SMALL = 16 * 64 * 2     # bytes of one [1,1,16,64] 16-bit tensor


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(flash_attn_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_header_symbols():
    assert os.path.exists(LIB_PATH), "build the library first (__graft_entry__.build())"
    names = _declared_functions()
    assert names == ["flash_attn_abi_version", "flash_attn_bwd", "flash_attn_bwd_validate", "flash_attn_fwd",
                     "flash_attn_fwd_fp8", "flash_attn_fwd_fp8_validate", "flash_attn_fwd_kernel",
                     "flash_attn_fwd_splitkv", "flash_attn_fwd_splitkv_noalloc", "flash_attn_fwd_splitkv_plan",
                     "flash_attn_fwd_splitkv_validate",
                     "flash_attn_fwd_splitkv_workspace_size", "flash_attn_fwd_strided",
                     "flash_attn_fwd_strided_validate", "flash_attn_fwd_validate", "flash_attn_quantize_fp8",
                     "flash_attn_quantize_fp8_validate", "flash_attn_strerror"]
    lib = ctypes.CDLL(LIB_PATH)
    for n in names:
        assert hasattr(lib, n)
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (flash_attn_\w+)$", out, flags=re.M))
    assert exported == set(names)


def test_abi_version_and_strerror():
    assert fa.flash_attn_abi_version() == 9
    codes = [fa.FA_OK, fa.FA_ERR_NULL, fa.FA_ERR_SHAPE, fa.FA_ERR_HEADDIM, fa.FA_ERR_DTYPE,
             fa.FA_ERR_SCALE, fa.FA_ERR_ALIGN, fa.FA_ERR_ALIAS, fa.FA_ERR_HIP, fa.FA_ERR_ARG,
             fa.FA_ERR_WORKSPACE, fa.FA_ERR_STRIDE, fa.FA_ERR_SCRATCH]
    msgs = [fa.flash_attn_strerror(c) for c in codes]
    assert len(set(msgs)) == len(codes)
    assert fa.flash_attn_strerror(12345) == "unknown status"


def _args(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=1, H=1, N=16, d=64,
          causal=0, scale=0.125, stream=None, dtype=0):
    return (q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype)


BAD = [
    (dict(B=-1), fa.FA_ERR_SHAPE), (dict(H=-2), fa.FA_ERR_SHAPE), (dict(N=-5), fa.FA_ERR_SHAPE),
    (dict(d=32), fa.FA_ERR_HEADDIM), (dict(d=96), fa.FA_ERR_HEADDIM), (dict(d=192), fa.FA_ERR_HEADDIM),
    (dict(d=512), fa.FA_ERR_HEADDIM),
    (dict(dtype=2), fa.FA_ERR_DTYPE), (dict(dtype=-1), fa.FA_ERR_DTYPE),
    (dict(causal=2), fa.FA_ERR_ARG), (dict(causal=-1), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(scale=-0.5), fa.FA_ERR_SCALE),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE), (dict(scale=float("inf")), fa.FA_ERR_SCALE),
    (dict(q=None), fa.FA_ERR_NULL), (dict(k=None), fa.FA_ERR_NULL), (dict(v=None), fa.FA_ERR_NULL),
    (dict(o=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(q=A + 8), fa.FA_ERR_ALIGN), (dict(v=A + 2 * GB + 4), fa.FA_ERR_ALIGN),
    (dict(o=A + 3 * GB + 2), fa.FA_ERR_ALIGN), (dict(lse=A + 4 * GB + 2), fa.FA_ERR_ALIGN),
    (dict(o=A), fa.FA_ERR_ALIAS), (dict(o=A + GB + SMALL - 16), fa.FA_ERR_ALIAS),
    (dict(o=A + 2 * GB - SMALL + 16), fa.FA_ERR_ALIAS),
    (dict(lse=A + GB + 64), fa.FA_ERR_ALIAS), (dict(lse=A + 3 * GB + 64), fa.FA_ERR_ALIAS),
    (dict(lse=A + 3 * GB - 60), fa.FA_ERR_ALIAS),
    (dict(N=1 << 24, d=128), fa.FA_ERR_SHAPE), (dict(B=1 << 20, H=1 << 20, N=1 << 10), fa.FA_ERR_SHAPE),
    (dict(B=1 << 40, H=1 << 40), fa.FA_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,code", BAD)
def test_validate_rejects(kw, code):
    assert _native.validate_raw(*_args(**kw)) == code


@pytest.mark.parametrize("kw,code", BAD)
def test_fwd_rejects_before_launch(kw, code):
    """flash_attn_fwd returns the same code and launches nothing."""
    assert _native.fwd_raw(*_args(**kw)) == code


@pytest.mark.parametrize("kw", [dict(), dict(d=128, dtype=1, causal=1), dict(B=3, H=8, N=4099, d=128),
                                dict(B=1, H=32, N=16384, d=128, causal=1), dict(d=256),
                                dict(B=2, H=8, N=1000, d=256, causal=1, dtype=1)])
def test_validate_accepts(kw):
    size = kw.get("B", 1) * kw.get("H", 1) * kw.get("N", 16) * kw.get("d", 64) * 2
    assert size < GB
    assert _native.validate_raw(*_args(**kw)) == fa.FA_OK


def test_adjacent_buffers_are_not_aliases():
    # o right after v's last byte and lse right after o's last byte
    args = _args(o=A + 2 * GB + SMALL, lse=A + 2 * GB + 2 * SMALL)
    assert _native.validate_raw(*args) == fa.FA_OK


def test_inputs_may_alias_each_other():
    """q, k and v are read-only, so attention over a single buffer is allowed."""
    assert _native.validate_raw(*_args(q=A, k=A, v=A)) == fa.FA_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_empty_problem_is_a_noop_even_with_null_pointers(kw):
    args = _args(q=None, k=None, v=None, o=None, lse=None, **kw)
    assert _native.validate_raw(*args) == fa.FA_OK
    assert _native.fwd_raw(*args) == fa.FA_OK


def test_python_binding_rejects_bad_tensors_before_the_library():
    import torch

    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)                                   # CPU tensors
    with pytest.raises(ValueError):
        fa.forward(q[0], q[0], q[0])                          # not 4-D
    with pytest.raises(ValueError):
        fa.forward(q, q.half(), q)                            # dtype mismatch
    with pytest.raises(TypeError):
        fa._dtype_code(q.float())                             # fp32 is not a kernel dtype


# ------------------------------------------------------------------ backward entry point
def _bargs(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, dout=A + 4 * GB, lse=A + 5 * GB, dq=A + 6 * GB,
           dk=A + 7 * GB, dv=A + 8 * GB, delta=A + 9 * GB, B=1, H=1, N=16, d=64, causal=0, scale=0.125,
           stream=None, dtype=0):
    return (q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, N, d, causal, scale, stream, dtype)


BAD_BWD = [
    (dict(B=-1), fa.FA_ERR_SHAPE), (dict(N=-3), fa.FA_ERR_SHAPE), (dict(d=96), fa.FA_ERR_HEADDIM),
    (dict(dtype=3), fa.FA_ERR_DTYPE), (dict(causal=5), fa.FA_ERR_ARG), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(scale=float("nan")), fa.FA_ERR_SCALE),
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL), (dict(dout=None), fa.FA_ERR_NULL),
    (dict(lse=None), fa.FA_ERR_NULL), (dict(dq=None), fa.FA_ERR_NULL), (dict(dk=None), fa.FA_ERR_NULL),
    (dict(dv=None), fa.FA_ERR_NULL), (dict(delta=None), fa.FA_ERR_NULL),
    (dict(dout=A + 4 * GB + 8), fa.FA_ERR_ALIGN), (dict(dk=A + 7 * GB + 4), fa.FA_ERR_ALIGN),
    (dict(delta=A + 9 * GB + 2), fa.FA_ERR_ALIGN), (dict(lse=A + 5 * GB + 1), fa.FA_ERR_ALIGN),
    (dict(dq=A), fa.FA_ERR_ALIAS), (dict(dk=A + 4 * GB + 32), fa.FA_ERR_ALIAS),
    (dict(dv=A + 6 * GB), fa.FA_ERR_ALIAS), (dict(delta=A + 5 * GB), fa.FA_ERR_ALIAS),
    (dict(delta=A + 8 * GB + SMALL - 4), fa.FA_ERR_ALIAS), (dict(dq=A + 3 * GB - SMALL + 16), fa.FA_ERR_ALIAS),
    (dict(N=1 << 24, d=128), fa.FA_ERR_SHAPE), (dict(B=1 << 40, H=1 << 40), fa.FA_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,code", BAD_BWD)
def test_bwd_validate_rejects(kw, code):
    assert _native.validate_bwd_raw(*_bargs(**kw)) == code
    assert _native.bwd_raw(*_bargs(**kw)) == code     # returns before any launch


@pytest.mark.parametrize("kw", [dict(), dict(d=128, dtype=1, causal=1), dict(B=2, H=32, N=4096, d=128, causal=1)])
def test_bwd_validate_accepts(kw):
    assert _native.validate_bwd_raw(*_bargs(**kw)) == fa.FA_OK


def test_bwd_inputs_may_alias_and_outputs_may_touch():
    """Read-only inputs may share memory; outputs may sit right after one another."""
    assert _native.validate_bwd_raw(*_bargs(q=A, k=A, v=A, o=A + GB, dout=A + GB)) == fa.FA_OK
    assert _native.validate_bwd_raw(*_bargs(dq=A + 6 * GB, dk=A + 6 * GB + SMALL, dv=A + 6 * GB + 2 * SMALL,
                                            delta=A + 6 * GB + 3 * SMALL)) == fa.FA_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0)])
def test_bwd_empty_problem_is_a_noop(kw):
    args = _bargs(q=None, k=None, v=None, o=None, dout=None, lse=None, dq=None, dk=None, dv=None, delta=None, **kw)
    assert _native.validate_bwd_raw(*args) == fa.FA_OK
    assert _native.bwd_raw(*args) == fa.FA_OK


def test_bwd_python_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        fa.backward(q, q, q, q, lse, q)                       # CPU tensors
    with pytest.raises(ValueError):
        fa.flash_attn_bwd(q, q, q, q, q, lse.double(), q, q, q, lse)   # lse dtype


# ---- key-split forward ----

def _sargs(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=1, H=1, N=1024, d=64, causal=0,
           scale=0.125, num_splits=4, ws=A + 5 * GB, ws_bytes=GB, stream=None, dtype=0):
    return (q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, ws, ws_bytes, stream, dtype)


WS_1K = 4 * 1 * 1024 * 65 * 4   # workspace of B1 H1 N1024 d64 at 4 splits


@pytest.mark.parametrize("B,H,N,d,causal,cus,want", [
    (1, 1, 256, 64, 0, 256, 1),         # 1 item, but only 4 key tiles: too short to split
    (1, 1, 448, 64, 0, 256, 1),         # 7 tiles: still too short
    (1, 1, 512, 64, 0, 256, 8),         # 8 tiles: 8 ranges
    (1, 1, 4096, 128, 0, 256, 16),      # 16 items want 16 ranges (the cap)
    (1, 4, 4096, 128, 1, 256, 4),       # 64 items want 4; the first causal tile has 4 key tiles
    (1, 1, 4096, 128, 1, 256, 4),       # wants 16, causal first tile allows 4
    (1, 1, 100, 64, 1, 256, 1),         # 100 keys: 2 tiles, too short
    (1, 1, 600, 64, 1, 256, 4),         # causal first query tile has 4 key tiles
    (1, 1, 1, 64, 0, 256, 1),           # one key: nothing to split
    (4, 16, 1024, 64, 0, 256, 1),       # 256 items fill 256 CUs
    (2, 32, 4096, 128, 1, 256, 1),
    (1, 8, 2048, 128, 0, 256, 4),       # 64 items -> 4
    (1, 8, 2048, 128, 0, 304, 5),       # another CU count -> ceil(304 / 64) = 5
    (1, 1, 4096, 128, 0, 0, 1),         # no device information: no split
    (0, 4, 128, 64, 0, 256, 1),         # empty problem
])
def test_splitkv_plan(B, H, N, d, causal, cus, want):
    assert fa.splitkv_plan(B, H, N, d, causal, cus) == want


def test_splitkv_plan_and_size_reject_bad_shapes():
    assert _native.splitkv_plan(-1, 1, 16, 64, 0, 256) == fa.FA_ERR_SHAPE
    assert _native.splitkv_plan(1, 1, 16, 96, 0, 256) == fa.FA_ERR_HEADDIM
    assert _native.splitkv_plan(1, 1, 16, 64, 3, 256) == fa.FA_ERR_ARG
    assert _native.splitkv_workspace_size(1, 1, 16, 64, 0, 0) == fa.FA_ERR_ARG
    assert _native.splitkv_workspace_size(1, -1, 16, 64, 0, 2) == fa.FA_ERR_SHAPE
    assert _native.splitkv_workspace_size(1, 1, 16, 80, 0, 2) == fa.FA_ERR_HEADDIM


@pytest.mark.parametrize("B,H,N,d,causal,splits,want", [
    (1, 1, 1024, 64, 0, 4, WS_1K),
    (1, 1, 1024, 64, 0, 1, 0),
    (1, 1, 1024, 64, 0, 99, 16 * 1024 * 65 * 4),     # reduced to 16
    (1, 1, 1024, 64, 1, 99, 4 * 1024 * 65 * 4),      # causal: reduced to 4
    (2, 3, 100, 128, 0, 2, 2 * 6 * 100 * 129 * 4),
    (2, 3, 100, 128, 0, 5, 2 * 6 * 100 * 129 * 4),   # 100 keys: 2 tiles
    (1, 1, 0, 64, 0, 3, 0),
])
def test_splitkv_workspace_size(B, H, N, d, causal, splits, want):
    assert fa.splitkv_workspace_size(B, H, N, d, causal, splits) == want


BAD_SPLIT = [
    (dict(num_splits=-1), fa.FA_ERR_ARG),
    (dict(ws=None), fa.FA_ERR_WORKSPACE), (dict(ws=A + 5 * GB + 8), fa.FA_ERR_WORKSPACE),
    (dict(ws_bytes=WS_1K - 1), fa.FA_ERR_WORKSPACE), (dict(ws_bytes=0), fa.FA_ERR_WORKSPACE),
    (dict(ws=A), fa.FA_ERR_ALIAS), (dict(ws=A + 3 * GB - WS_1K + 16), fa.FA_ERR_ALIAS),
    (dict(ws=A + 4 * GB), fa.FA_ERR_ALIAS),
    # the forward's own checks still apply
    (dict(d=96), fa.FA_ERR_HEADDIM), (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(q=None), fa.FA_ERR_NULL),
    (dict(o=A), fa.FA_ERR_ALIAS), (dict(causal=5), fa.FA_ERR_ARG), (dict(dtype=7), fa.FA_ERR_DTYPE),
    # the forward takes d = 256; the key split does not
    (dict(d=256), fa.FA_ERR_HEADDIM),
]


@pytest.mark.parametrize("kw,code", BAD_SPLIT)
def test_splitkv_validate_rejects(kw, code):
    assert _native.validate_splitkv_raw(*_sargs(**kw)) == code


@pytest.mark.parametrize("kw,code", BAD_SPLIT)
def test_splitkv_rejects_before_launch(kw, code):
    assert _native.splitkv_raw(*_sargs(**kw)) == code


@pytest.mark.parametrize("kw", [
    dict(), dict(ws_bytes=WS_1K), dict(ws=A + 4 * GB + 1024 * 4),        # just after lse
    dict(num_splits=1, ws=None, ws_bytes=0),                             # resolves to the plain forward
    dict(N=16, num_splits=8, ws=None, ws_bytes=0),                       # 16 keys: one tile, no split
    dict(num_splits=0, ws=None, ws_bytes=0),                             # chosen at launch: not checked here
    dict(causal=1, num_splits=50, ws_bytes=WS_1K),                       # reduced to 4
])
def test_splitkv_validate_accepts(kw):
    assert _native.validate_splitkv_raw(*_sargs(**kw)) == fa.FA_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_splitkv_empty_problem_is_a_noop(kw):
    assert _native.splitkv_raw(*_sargs(q=None, k=None, v=None, o=None, lse=None, ws=None, ws_bytes=0,
                                       **kw)) == fa.FA_OK


# ---- key-split forward without a workspace ----
# Only calls that fail a check (or describe an empty problem) are made: they return
# before any HIP call. num_splits = 0 would query the device, so it is not used here.

def _nargs(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=1, H=1, N=1024, d=64, causal=0,
           scale=0.125, num_splits=4, stream=None, dtype=0):
    return (q, k, v, o, lse, B, H, N, d, causal, scale, num_splits, stream, dtype)


def test_noalloc_boundary_sizes():
    assert fa.splitkv_workspace_size(1, 16, 1024, 64, 0, 16) == fa.FA_SPLITKV_SCRATCH_BYTES
    assert fa.splitkv_workspace_size(1, 16, 1025, 64, 0, 16) > fa.FA_SPLITKV_SCRATCH_BYTES


def test_noalloc_scratch_size_matches_header_and_covers_the_planned_split():
    text = open(HEADER).read()
    m = re.search(r"#define FA_SPLITKV_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == fa.FA_SPLITKV_SCRATCH_BYTES
    # every split the planner picks for a 256-compute-unit device fits, at both head sizes
    worst = 0
    for d in (64, 128):
        for causal in (0, 1):
            for B, H in ((1, 1), (1, 2), (1, 3), (1, 5), (2, 3), (1, 8), (3, 7), (1, 64), (4, 32)):
                for N in (449, 512, 1000, 1024, 2047, 4096, 8191, 16384, 65536):
                    s = fa.splitkv_plan(B, H, N, d, causal, 256)
                    worst = max(worst, fa.splitkv_workspace_size(B, H, N, d, causal, s))
    assert 0 < worst <= fa.FA_SPLITKV_SCRATCH_BYTES


BAD_NOALLOC = [
    (dict(num_splits=-1), fa.FA_ERR_ARG), (dict(d=96), fa.FA_ERR_HEADDIM), (dict(scale=0.0), fa.FA_ERR_SCALE),
    (dict(d=256), fa.FA_ERR_HEADDIM), (dict(d=256, num_splits=2), fa.FA_ERR_HEADDIM),
    (dict(q=None), fa.FA_ERR_NULL), (dict(o=A), fa.FA_ERR_ALIAS), (dict(causal=5), fa.FA_ERR_ARG),
    (dict(dtype=7), fa.FA_ERR_DTYPE), (dict(B=-1), fa.FA_ERR_SHAPE), (dict(lse=A + 4 * GB + 2), fa.FA_ERR_ALIGN),
    # 2 splits of B1 H64 N4096 d128 need 2 * 64 * 4096 * 129 * 4 bytes (258 MiB)
    (dict(H=64, N=4096, d=128, num_splits=2), fa.FA_ERR_SCRATCH),
    # 16 splits of B1 H16 d64 need exactly 65 MiB at N = 1024; one more row does not fit
    (dict(H=16, N=1025, d=64, num_splits=16), fa.FA_ERR_SCRATCH),
]


@pytest.mark.parametrize("kw,code", BAD_NOALLOC)
def test_noalloc_rejects_before_launch(kw, code):
    assert _native.splitkv_noalloc_raw(*_nargs(**kw)) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_noalloc_empty_problem_is_a_noop(kw):
    assert _native.splitkv_noalloc_raw(*_nargs(q=None, k=None, v=None, o=None, lse=None, **kw)) == fa.FA_OK


# ---- strided forward ----
# B2 H3 N100 d80 views; contiguous strides unless overridden (elements)

def _cstr(H=3, N=100, d=80):
    return (H * N * d, N * d, d)


def _targs(q=A, k=A + GB, v=A + 2 * GB, o=A + 3 * GB, lse=A + 4 * GB, B=2, H=3, N=100, d=80, qs="c", ks="c",
           vs="c", os_="c", ls="c", causal=0, scale=0.1, stream=None, dtype=0):
    c = _cstr(H, N, d)
    pick = lambda x: c if x == "c" else x
    return (q, k, v, o, lse, B, H, N, d, pick(qs), pick(ks), pick(vs), pick(os_), (H * N, N) if ls == "c" else ls,
            causal, scale, stream, dtype)


BAD_STRIDED = [
    (dict(d=12), fa.FA_ERR_HEADDIM), (dict(d=0), fa.FA_ERR_HEADDIM), (dict(d=264), fa.FA_ERR_HEADDIM),
    (dict(d=4), fa.FA_ERR_HEADDIM), (dict(d=260), fa.FA_ERR_HEADDIM), (dict(d=512), fa.FA_ERR_HEADDIM),
    (dict(qs=(24000, 8000, 79)), fa.FA_ERR_STRIDE),          # row stride below d and not a multiple of 8
    (dict(ks=(24000, 8000, 72)), fa.FA_ERR_STRIDE),          # row stride below d
    (dict(vs=(24000, 8004, 80)), fa.FA_ERR_STRIDE),          # head stride not a multiple of 8
    (dict(qs=(-24000, 8000, 80)), fa.FA_ERR_STRIDE),
    (dict(os_=(24000, 8000, 1 << 23)), fa.FA_ERR_STRIDE),    # row stride too large
    (dict(N=20000, qs=(0, 0, 65536)), fa.FA_ERR_STRIDE),     # slice spans >= 2 GiB
    (dict(os_=(24000, 0, 80)), fa.FA_ERR_STRIDE),            # heads of o overlap
    (dict(os_=(24000, 4000, 80)), fa.FA_ERR_STRIDE),         # o's head stride inside a head's rows
    (dict(ls=(300, 50)), fa.FA_ERR_STRIDE),                  # lse heads overlap
    (dict(ls=(-1, 100)), fa.FA_ERR_STRIDE),
    (dict(qs=None), fa.FA_ERR_NULL), (dict(ls=None), fa.FA_ERR_NULL), (dict(o=None), fa.FA_ERR_NULL),
    (dict(q=A + 8), fa.FA_ERR_ALIGN), (dict(lse=A + 4 * GB + 2), fa.FA_ERR_ALIGN),
    (dict(o=A + 16), fa.FA_ERR_ALIAS),                       # o inside q's span
    (dict(lse=A + 2 * GB + 4000), fa.FA_ERR_ALIAS),          # lse inside v's span
    (dict(dtype=3), fa.FA_ERR_DTYPE), (dict(causal=2), fa.FA_ERR_ARG), (dict(scale=-1.0), fa.FA_ERR_SCALE),
    (dict(B=-1), fa.FA_ERR_SHAPE),
]


@pytest.mark.parametrize("kw,code", BAD_STRIDED)
def test_strided_validate_rejects(kw, code):
    assert _native.validate_strided_raw(*_targs(**kw)) == code


@pytest.mark.parametrize("kw,code", BAD_STRIDED)
def test_strided_rejects_before_launch(kw, code):
    assert _native.strided_raw(*_targs(**kw)) == code


@pytest.mark.parametrize("kw", [
    dict(), dict(d=8), dict(d=128), dict(d=64), dict(d=120), dict(d=136), dict(d=200), dict(d=256),
    dict(qs=(100 * 3 * 3 * 80, 80, 3 * 3 * 80), ks=(100 * 3 * 3 * 80, 80, 3 * 3 * 80)),   # packed qkv rows
    dict(ks=(8000, 0, 80), vs=(8000, 0, 80)),                   # one K/V head shared by all heads
    dict(ks=(0, 0, 80), vs=(0, 0, 80)),                         # one K/V slice shared by everything
    dict(os_=(100 * 3 * 80, 80, 3 * 80)),                       # o as [B, N, H, d]
    dict(os_=(3 * 100 * 96, 100 * 96, 96)),                     # padded o rows
    dict(ls=(3 * 128, 128)), dict(ls=(1, 2), B=2, H=1, N=1),    # padded lse rows; tiny
    dict(o=A + 16, q=A + 3 * GB),                               # swapped places, still disjoint
])
def test_strided_validate_accepts(kw):
    assert _native.validate_strided_raw(*_targs(**kw)) == fa.FA_OK


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0)])
def test_strided_empty_problem_is_a_noop(kw):
    args = _targs(q=None, k=None, v=None, o=None, lse=None, qs=None, ks=None, vs=None, os_=None, ls=None, **kw)
    assert _native.strided_raw(*args) == fa.FA_OK


# ---- FP8 ----

def _qargs(x=A, x8=A + GB, se=A + 2 * GB, B=1, H=2, N=100, d=128, layout=0, stream=None, dtype=0, fmt=0):
    return (x, x8, se, B, H, N, d, layout, stream, dtype, fmt)


BAD_QUANT = [
    (dict(d=96), fa.FA_ERR_HEADDIM), (dict(layout=2), fa.FA_ERR_ARG), (dict(dtype=5), fa.FA_ERR_DTYPE),
    (dict(fmt=2), fa.FA_ERR_ARG), (dict(fmt=-1), fa.FA_ERR_ARG),
    (dict(N=-1), fa.FA_ERR_SHAPE), (dict(x=None), fa.FA_ERR_NULL), (dict(se=None), fa.FA_ERR_NULL),
    (dict(x8=A + GB + 8), fa.FA_ERR_ALIGN), (dict(se=A + 2 * GB + 2), fa.FA_ERR_ALIGN),
    (dict(x8=A + 16), fa.FA_ERR_ALIAS), (dict(se=A + GB + 64), fa.FA_ERR_ALIAS),
    (dict(se=A + GB + 2 * 100 * 128 - 4), fa.FA_ERR_ALIAS),
    (dict(se=A + GB + 2 * 2 * 128 * 64 - 4, layout=1), fa.FA_ERR_ALIAS),   # keys-transposed output is larger
]


@pytest.mark.parametrize("kw,code", BAD_QUANT)
def test_quantize_rejects(kw, code):
    assert _native.validate_quantize_raw(*_qargs(**kw)) == code
    assert _native.quantize_raw(*_qargs(**kw)) == code


@pytest.mark.parametrize("kw", [dict(), dict(layout=1), dict(d=64, dtype=1), dict(se=A + GB + 2 * 100 * 128),
                                dict(fmt=fa.FA_FP8_E5M2), dict(fmt=fa.FA_FP8_E5M2, layout=1)])
def test_quantize_accepts(kw):
    assert _native.validate_quantize_raw(*_qargs(**kw)) == fa.FA_OK


def test_quantize_empty_is_a_noop():
    assert _native.quantize_raw(*_qargs(x=None, x8=None, se=None, N=0)) == fa.FA_OK


def _fargs(q8=A, k8=A + GB, v8t=A + 2 * GB, qs=A + 3 * GB, ks=A + 3 * GB + 4096, vs=A + 3 * GB + 8192,
           o=A + 4 * GB, lse=A + 5 * GB, B=1, H=2, N=100, d=128, causal=0, scale=0.1, stream=None, dtype=0,
           fmt=0):
    return (q8, k8, v8t, qs, ks, vs, o, lse, B, H, N, d, causal, scale, stream, dtype, fmt)


BAD_FP8 = [
    (dict(d=96), fa.FA_ERR_HEADDIM), (dict(d=256), fa.FA_ERR_HEADDIM), (dict(dtype=2), fa.FA_ERR_DTYPE),
    (dict(causal=3), fa.FA_ERR_ARG),
    (dict(fmt=7), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_SCALE), (dict(B=-1), fa.FA_ERR_SHAPE),
    (dict(v8t=None), fa.FA_ERR_NULL), (dict(ks=None), fa.FA_ERR_NULL), (dict(lse=None), fa.FA_ERR_NULL),
    (dict(q8=A + 4), fa.FA_ERR_ALIGN), (dict(vs=A + 3 * GB + 8194), fa.FA_ERR_ALIGN),
    (dict(o=A + 16), fa.FA_ERR_ALIAS), (dict(lse=A + 3 * GB + 4096), fa.FA_ERR_ALIAS),
    (dict(lse=A + 4 * GB + 64), fa.FA_ERR_ALIAS),
]


@pytest.mark.parametrize("kw,code", BAD_FP8)
def test_fp8_rejects(kw, code):
    assert _native.validate_fp8_raw(*_fargs(**kw)) == code
    assert _native.fp8_raw(*_fargs(**kw)) == code


def test_fp8_accepts_and_empty():
    assert _native.validate_fp8_raw(*_fargs()) == fa.FA_OK
    assert _native.validate_fp8_raw(*_fargs(causal=1, dtype=1)) == fa.FA_OK
    assert _native.validate_fp8_raw(*_fargs(fmt=fa.FA_FP8_E5M2)) == fa.FA_OK
    assert _native.validate_fp8_raw(*_fargs(d=64)) == fa.FA_OK
    assert _native.fp8_raw(*_fargs(q8=None, k8=None, v8t=None, qs=None, ks=None, vs=None, o=None, lse=None,
                                   H=0)) == fa.FA_OK


# (N, d, causal, kernel): the ping-pong kernel for d <= 64, 97..128 and 129..256,
# the pipelined kernel for d in 65..96, at any N and mask
PIPE, PING = _native.FA_FWD_KERNEL_PIPELINED, _native.FA_FWD_KERNEL_PINGPONG


@pytest.mark.parametrize("N,d,causal,want", [
    (0, 64, 0, PING), (256, 64, 0, PING), (4096, 128, 0, PING), (4096, 128, 1, PING), (16384, 128, 1, PING),
    (65536, 128, 0, PING), (1024, 56, 0, PING), (300, 72, 1, PIPE), (300, 80, 0, PIPE), (300, 88, 1, PIPE),
    (300, 96, 0, PIPE), (16384, 96, 1, PIPE), (300, 104, 0, PING), (8192, 8, 0, PING), (300, 136, 1, PING),
    (4096, 256, 0, PING)])
def test_fwd_kernel_choice(monkeypatch, N, d, causal, want):
    monkeypatch.delenv("FLASH_ATTN_FWD_KERNEL", raising=False)
    assert _native.fwd_kernel(N, d, causal) == want
    assert fa.flash_attn_fwd_kernel(N, d, bool(causal)) == ("pipelined" if want == PIPE else "pingpong")


def test_fwd_kernel_forced_and_rejects(monkeypatch):
    monkeypatch.setenv("FLASH_ATTN_FWD_KERNEL", "pingpong")
    assert _native.fwd_kernel(16384, 128, 1) == PING
    assert _native.fwd_kernel(300, 80, 0) == PING
    monkeypatch.setenv("FLASH_ATTN_FWD_KERNEL", "pipelined")
    assert _native.fwd_kernel(256, 64, 0) == PIPE
    assert _native.fwd_kernel(256, 192, 0) == PING   # no pipelined instance above 128
    monkeypatch.setenv("FLASH_ATTN_FWD_KERNEL", "other")   # unknown names are ignored
    assert _native.fwd_kernel(256, 64, 0) == PING and _native.fwd_kernel(256, 80, 0) == PIPE
    monkeypatch.delenv("FLASH_ATTN_FWD_KERNEL")
    assert _native.fwd_kernel(-1, 64, 0) == fa.FA_ERR_SHAPE
    for d in (0, 7, 12, 252, 264, 512):
        assert _native.fwd_kernel(256, d, 0) == fa.FA_ERR_HEADDIM
    assert _native.fwd_kernel(256, 64, 2) == fa.FA_ERR_ARG
    with pytest.raises(fa.FlashAttnError):
        fa.flash_attn_fwd_kernel(256, 12)
