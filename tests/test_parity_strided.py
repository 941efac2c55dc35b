"""GPU parity of flash_attn_fwd_strided: strided views and head dimensions that are
not 64 or 128, against the float64 oracle (tolerances of tests/_parity.py).

* Head dimensions d in {8, 24, 40, 56, 72, 80, 96, 120} (multiples of 8, masked up to
  the 64- or 128-wide kernel as "6.1 FlashAttention V1 in detail", §8.3 masks
  BLOCK_D > D), both dtypes and masks, ragged N, through both forward kernels.
* Head dimensions above 128 (136, 192, 200, 256) on the 256-wide instance, which runs
  once per 128 columns of V and O and loads Q straight into registers: ragged and
  multi-item shapes compared in full, NaN in the padding past d, packed QKV, the
  headline shape at d = 256 on sampled heads, and the contiguous call.
* Layouts: q, k, v as views of one packed [B, N, 3, H, d] projection output; o written
  into a [B, N, H, d] tensor; padded rows whose padding holds NaN (never read: a read
  would poison the result); padded output rows and lse rows whose padding must keep
  its sentinel; one K/V head shared by all heads (head stride 0).
* The contiguous call through the strided entry equals flash_attn_fwd bitwise.
"""
import math
import sys

import numpy as np
import pytest

from exact_attention_flash_amd import inputs
from oracle.dense import attention as oracle_attention
from tests._parity import assert_parity, metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_flash_amd as fa_mod

    fa_mod._native.lib()
    return fa_mod


def _scale(d):
    return float(np.float32(1.0 / math.sqrt(d)))


def _tdtype(dtype):
    return torch.bfloat16 if dtype == inputs.BF16 else torch.float16


def _dev_from_bits(bits, dtype):
    return inputs.to_torch(bits, dtype, torch.device("cuda:0"))


def _o64(t, dtype):
    return inputs.bits_to_f64(inputs.from_torch_bits(t.contiguous()), dtype)


def _oracle(bits, dtype, causal, scale):
    q, k, v = (inputs.bits_to_f64(x, dtype) for x in bits)
    return oracle_attention(q, k, v, scale, causal=causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("d", [8, 24, 40, 56, 72, 80, 88, 96, 120])
def test_head_dims(fa, fwd_kernel, d, dtype, causal):
    shape = (2, 2, 300, d)
    scale = _scale(d)
    bits = inputs.draw_qkv(shape, dtype, 1.0, 700 + d + (1 if causal else 0))
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)   # contiguous, d not 64/128: strided entry
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"strided {fwd_kernel} d={d} {dtype} causal={causal}: {m}")
    assert_parity(m, f"d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 80, 128])
def test_packed_qkv_and_bnhd_output(fa, d, causal):
    """q, k, v are views of one [B, N, 3, H, d] tensor; o is a [B, N, H, d] tensor."""
    B, H, N, dtype = 2, 3, 517, inputs.BF16
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 800 + d + (1 if causal else 0))
    q0, k0, v0 = (_dev_from_bits(x, dtype) for x in bits)
    packed = torch.stack([t.permute(0, 2, 1, 3) for t in (q0, k0, v0)], dim=2).contiguous()   # [B, N, 3, H, d]
    q, k, v = (packed[:, :, i].permute(0, 2, 1, 3) for i in range(3))                         # [B, H, N, d] views
    assert not q.is_contiguous() and q.stride() == (N * 3 * H * d, d, 3 * H * d, 1)
    o_bnhd = torch.empty((B, N, H, d), dtype=_tdtype(dtype), device="cuda:0")
    o = o_bnhd.permute(0, 2, 1, 3)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    fa.flash_attn_fwd_strided(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"packed qkv d={d} causal={causal}: {m}")
    assert_parity(m, f"packed d={d} causal={causal}")


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("d", [40, 64, 96])
def test_padding_is_never_read_or_written(fa, d, dtype):
    """Inputs with row stride d + 24 whose padding holds NaN; o and lse with padded rows
    holding a sentinel that must survive."""
    B, H, N, pad = 1, 2, 333, 24
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 900 + d)
    dev = torch.device("cuda:0")
    views = []
    for x in bits:
        full = torch.full((B, H, N, d + pad), float("nan"), dtype=_tdtype(dtype), device=dev)
        full[..., :d] = _dev_from_bits(x, dtype)
        views.append(full[..., :d])
    o_full = torch.full((B, H, N, d + pad), 7.0, dtype=_tdtype(dtype), device=dev)
    lse_full = torch.full((B, H, N + 5), -3.0, dtype=torch.float32, device=dev)
    o, lse = o_full[..., :d], lse_full[..., :N]
    fa.flash_attn_fwd_strided(*views, o, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, True, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    assert_parity(m, f"padded d={d} {dtype}")
    assert torch.all(o_full[..., d:] == 7.0).item(), "output padding was written"
    assert torch.all(lse_full[..., N:] == -3.0).item(), "lse padding was written"


@pytest.mark.parametrize("causal", [False, True])
def test_shared_kv_head(fa, causal):
    """Head stride 0 for K and V: every query head attends the one K/V head."""
    B, H, N, d, dtype = 2, 4, 260, 80, inputs.FP16
    scale = _scale(d)
    qb, _, _ = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 950)
    _, kb, vb = inputs.draw_qkv((B, 1, N, d), dtype, 1.0, 951)
    q = _dev_from_bits(qb, dtype)
    k1, v1 = _dev_from_bits(kb, dtype), _dev_from_bits(vb, dtype)
    k, v = k1.expand(B, H, N, d), v1.expand(B, H, N, d)
    assert k.stride(1) == 0
    o = torch.empty((B, H, N, d), dtype=_tdtype(dtype), device="cuda:0")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    fa.flash_attn_fwd_strided(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    kfull = np.broadcast_to(kb, (B, H, N, d))
    vfull = np.broadcast_to(vb, (B, H, N, d))
    ro, rl = _oracle((qb, kfull, vfull), dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    assert_parity(m, f"shared kv causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_contiguous_strided_equals_plain(fa, d, causal):
    shape, dtype = (2, 3, 400, d), inputs.BF16
    bits = inputs.draw_qkv(shape, dtype, 1.0, 960 + d)
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o1, l1 = fa.forward(q, k, v, causal=causal, scale=0.1)
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    fa.flash_attn_fwd_strided(q, k, v, o2, l2, causal=causal, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [80, 96])
def test_head_dims_multi_item_workgroups(fa, fwd_kernel, d, causal):
    """The 80- and 96-wide instances with several items per workgroup (4*32 slices of
    three 256-row query tiles, the last ragged: 384 items on at most 256 workgroups),
    compared in full."""
    shape, dtype = (4, 32, 600, d), inputs.BF16
    scale = _scale(d)
    bits = inputs.draw_qkv(shape, dtype, 1.0, 800 + d + (1 if causal else 0))
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"strided {fwd_kernel} d={d} multi-item causal={causal}: {m}")
    assert_parity(m, f"d={d} multi-item causal={causal}")


def test_workload_shape_d80(fa):
    """B2 H32 N4096 at d = 80 (a non-power-of-2 head dimension at the headline shape),
    causal bf16; sampled heads against the oracle."""
    B, H, N, d, dtype = 2, 32, 4096, 80, inputs.BF16
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 970)
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    heads = [0, 33, 63]
    sel = lambda x: x.reshape(B * H, N, d)[heads]
    ro, rl = _oracle(tuple(sel(x) for x in bits), dtype, True, scale)
    og = _o64(o, dtype).reshape(B * H, N, d)[heads]
    lg = lse.double().cpu().numpy().reshape(B * H, N)[heads]
    m = metrics(og, lg, ro, rl, dtype)
    _log(f"d=80 headline shape heads {heads}: {m}")
    assert_parity(m, "d=80 headline shape")


# ---- head dimensions above 128: the 256-wide instance ----

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("d", [136, 192, 200, 256])
def test_wide_head_dims(fa, d, dtype, causal):
    """Ragged N (two 256-row query tiles, the second partial), compared in full."""
    shape = (2, 2, 300, d)
    scale = _scale(d)
    bits = inputs.draw_qkv(shape, dtype, 1.0, 1700 + d + (1 if causal else 0))
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"wide d={d} {dtype} causal={causal}: {m}")
    assert_parity(m, f"wide d={d} {dtype} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [192, 256])
def test_wide_multi_item_workgroups(fa, d, causal):
    """8 x 32 slices of three 256-row query tiles (the last ragged): 768 items, at least
    three per workgroup, so every workgroup loads a later item's Q into registers while
    the item before drains; compared in full."""
    shape, dtype = (8, 32, 600, d), inputs.BF16
    scale = _scale(d)
    bits = inputs.draw_qkv(shape, dtype, 1.0, 1750 + d + (1 if causal else 0))
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"wide d={d} multi-item causal={causal}: {m}")
    assert_parity(m, f"wide d={d} multi-item causal={causal}")


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("d", [136, 200])
def test_wide_padding_is_never_read_or_written(fa, d, dtype):
    """Row stride d + 24 with NaN in the padding of q, k and v (a read of any masked
    column would poison the result); o and lse padding keep their sentinels."""
    B, H, N, pad = 1, 2, 333, 24
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 1800 + d)
    dev = torch.device("cuda:0")
    views = []
    for x in bits:
        full = torch.full((B, H, N, d + pad), float("nan"), dtype=_tdtype(dtype), device=dev)
        full[..., :d] = _dev_from_bits(x, dtype)
        views.append(full[..., :d])
    o_full = torch.full((B, H, N, d + pad), 7.0, dtype=_tdtype(dtype), device=dev)
    lse_full = torch.full((B, H, N + 5), -3.0, dtype=torch.float32, device=dev)
    o, lse = o_full[..., :d], lse_full[..., :N]
    fa.flash_attn_fwd_strided(*views, o, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, True, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    assert_parity(m, f"wide padded d={d} {dtype}")
    assert torch.all(o_full[..., d:] == 7.0).item(), "output padding was written"
    assert torch.all(lse_full[..., N:] == -3.0).item(), "lse padding was written"


@pytest.mark.parametrize("causal", [False, True])
def test_wide_packed_qkv_and_bnhd_output(fa, causal):
    """d = 256 with q, k, v views of one [B, N, 3, H, d] tensor and o a [B, N, H, d] tensor."""
    B, H, N, d, dtype = 2, 3, 517, 256, inputs.FP16
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 1850 + (1 if causal else 0))
    q0, k0, v0 = (_dev_from_bits(x, dtype) for x in bits)
    packed = torch.stack([t.permute(0, 2, 1, 3) for t in (q0, k0, v0)], dim=2).contiguous()
    q, k, v = (packed[:, :, i].permute(0, 2, 1, 3) for i in range(3))
    o_bnhd = torch.empty((B, N, H, d), dtype=_tdtype(dtype), device="cuda:0")
    o = o_bnhd.permute(0, 2, 1, 3)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    fa.flash_attn_fwd_strided(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"wide packed qkv causal={causal}: {m}")
    assert_parity(m, f"wide packed causal={causal}")


def test_wide_contiguous_strided_equals_plain(fa):
    shape, dtype = (2, 3, 400, 256), inputs.BF16
    bits = inputs.draw_qkv(shape, dtype, 1.0, 1900)
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o1, l1 = fa.forward(q, k, v, causal=True, scale=0.1)   # flash_attn_fwd at d = 256
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    fa.flash_attn_fwd_strided(q, k, v, o2, l2, causal=True, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_wide_headline_shape_d256(fa):
    """B2 H32 N4096 at d = 256, causal bf16: one row of every (slice, 256-row query
    tile) work item (the in-tile row varies by slice so every 32-row wave block is
    hit) plus three whole slices, against the oracle."""
    B, H, N, d, dtype = 2, 32, 4096, 256, inputs.BF16
    scale = _scale(d)
    bits = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 1950)
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    og_all = _o64(o, dtype).reshape(B * H, N, d)
    lg_all = lse.double().cpu().numpy().reshape(B * H, N)
    heads = [0, 33, 63]
    sel = lambda x: x.reshape(B * H, N, d)[heads]
    ro, rl = _oracle(tuple(sel(x) for x in bits), dtype, True, scale)
    m = metrics(og_all[heads], lg_all[heads], ro, rl, dtype)
    _log(f"d=256 headline shape, whole slices {heads}: {m}")
    assert_parity(m, "d=256 headline shape")
    # one row per work item, every slice
    qf, kf, vf = (inputs.bits_to_f64(x, dtype).reshape(B * H, N, d) for x in bits)
    rows = np.array([[t * 256 + (37 * s + 5 * t) % 256 for t in range(N // 256)] for s in range(B * H)])
    worst = []
    for s in range(B * H):
        r = rows[s]
        ref_o, ref_l = oracle_attention(qf[s], kf[s], vf[s], scale, causal=True, rows=r)
        mm = metrics(og_all[s, r], lg_all[s, r], ref_o, ref_l, dtype)
        assert_parity(mm, f"d=256 headline shape slice {s}")
        worst.append(mm["o_max_excess"])
    _log(f"d=256 headline shape, one row of each of {rows.size} work items: worst O excess {max(worst):.2e}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,dtype,sigma", [
    ((1, 1, 1, 256), inputs.BF16, 1.0),      # one query, one key
    ((1, 1, 64, 256), inputs.FP16, 1.0),     # exactly one key tile
    ((1, 3, 257, 192), inputs.BF16, 1.0),    # B*H = 3: no XCD grouping; one row past a query tile
    ((2, 4, 130, 256), inputs.FP16, 8.0),    # sigma 8: extreme logits
    ((1, 2, 700, 136), inputs.FP16, 8.0),
])
def test_wide_edge_shapes(fa, shape, dtype, sigma, causal):
    d = shape[-1]
    scale = _scale(d)
    bits = inputs.draw_qkv(shape, dtype, sigma, 2000 + shape[2] + d + (1 if causal else 0))
    q, k, v = (_dev_from_bits(x, dtype) for x in bits)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = _oracle(bits, dtype, causal, scale)
    m = metrics(_o64(o, dtype), lse.double().cpu().numpy(), ro, rl, dtype)
    _log(f"wide edge {shape} {dtype} sigma={sigma} causal={causal}: {m}")
    assert_parity(m, f"wide edge {shape} causal={causal}")
