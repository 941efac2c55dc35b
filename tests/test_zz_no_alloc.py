"""flash_attn_fwd_splitkv_noalloc (partials in the library's fixed device array)
against flash_attn_fwd_splitkv with a caller workspace, through the C ABI.

Both run the same kernels with the same split count, so o and lse must agree
bitwise. The calls without a workspace come two in a row, the second on a
smaller problem (the array then still holds the first call's partials, which the
second must not read), then once more with the split chosen by the library.
"""
import math
import sys

import numpy as np
import pytest

from exact_attention_flash_amd import _native, inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _problem(shape, dtype, seed):
    dev = torch.device("cuda:0")
    B, H, N, d = shape
    q, k, v = (inputs.to_torch(x, dtype, dev) for x in inputs.draw_qkv(shape, dtype, 1.0, seed))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=dev)
    return q, k, v, o, lse


def _code(dtype):
    return _native.FA_FP16 if dtype == inputs.FP16 else _native.FA_BF16


def _with_workspace(q, k, v, shape, dtype, causal, splits):
    B, H, N, d = shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=q.device)
    nbytes = _native.splitkv_workspace_size(B, H, N, d, causal, splits)
    assert nbytes > 0
    ws = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=q.device)
    st = _native.splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                             causal, 1.0 / math.sqrt(d), splits, ws.data_ptr(), nbytes,
                             torch.cuda.current_stream().cuda_stream, _code(dtype))
    assert st == _native.FA_OK, _native.strerror(st)
    return o, lse


def _noalloc(q, k, v, o, lse, shape, dtype, causal, splits):
    B, H, N, d = shape
    st = _native.splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H,
                                     N, d, causal, 1.0 / math.sqrt(d), splits,
                                     torch.cuda.current_stream().cuda_stream, _code(dtype))
    assert st == _native.FA_OK, _native.strerror(st)


def _same(a, b):
    x, y = a.cpu(), b.cpu()
    assert not torch.isnan(x).any()
    assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                       y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32))


# (shape, dtype, causal, splits): the first needs 4 * 8 * 2048 * 129 * 4 bytes (33 MiB)
# of partials, the second 3 * 2 * 700 * 65 * 4 (1 MiB)
CALLS = [((1, 8, 2048, 128), inputs.BF16, 1, 4), ((1, 2, 700, 64), inputs.FP16, 0, 3)]


def test_noalloc_matches_workspace_call_twice_in_a_row():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    probs = [_problem(shape, dt, 11 + i) for i, (shape, dt, _, _) in enumerate(CALLS)]
    refs = []
    for (shape, dt, causal, splits), (q, k, v, _, _) in zip(CALLS, probs):
        _log(f"workspace call {shape} causal={causal} splits={splits}")
        refs.append(_with_workspace(q, k, v, shape, dt, causal, splits))
    torch.cuda.synchronize()
    for (shape, dt, causal, splits), (q, k, v, o, lse) in zip(CALLS, probs):
        _log(f"noalloc call {shape} causal={causal} splits={splits}")
        _noalloc(q, k, v, o, lse, shape, dt, causal, splits)
    torch.cuda.synchronize()
    for (o_ref, lse_ref), (_, _, _, o, lse) in zip(refs, probs):
        _same(o, o_ref)
        _same(lse, lse_ref)


def test_noalloc_planned_split_matches():
    shape, dt, causal = (2, 4, 1536, 128), inputs.BF16, 1
    B, H, N, d = shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = _native.splitkv_plan(B, H, N, d, causal, cus)
    _log(f"planned noalloc {shape} splits={splits} cus={cus}")
    assert splits > 1
    q, k, v, o, lse = _problem(shape, dt, 5)
    o_ref, lse_ref = _with_workspace(q, k, v, shape, dt, causal, splits)
    _noalloc(q, k, v, o, lse, shape, dt, causal, 0)
    torch.cuda.synchronize()
    _same(o, o_ref)
    _same(lse, lse_ref)
