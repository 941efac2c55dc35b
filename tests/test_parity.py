"""GPU parity: the HIP kernels behind the C ABI against the float64 oracle.

Every case draws seeded inputs (exact_attention_flash_amd.inputs), runs
flash_attn_fwd on the GPU through the C ABI (via the thin Python binding), widens
the 16-bit outputs exactly and compares element by element with oracle.dense on
the same bytes, with the tolerances of tests/_parity.py.

* Small shapes: full outputs, sizes that span several 128-row query tiles and
  64-row key tiles, with ragged tails, N = 1 and N = 3, both dtypes, both masks,
  each through both forward kernels (FLASH_ATTN_FWD_KERNEL forces one).
* The five workloads at full size, in the same launch configuration the
  benchmark times: complete outputs where the oracle is quick (the 256- and
  1024-token workloads) and otherwise sampled rows of every (batch, head) --
  first/last rows, tile and wave boundaries, the ragged end and random rows --
  plus complete heads; each with the workload seed and seed + 100 through the
  kernel the call picks, and with the workload seed through the other kernel.
* Properties: the worked example of the tokenlab note zero-padded to d = 64,
  V = 1, Q = 0, the causal prefix property (bitwise), determinism, a side stream,
  empty problems and very large logits.
"""
import math
import os
import sys
import time

import numpy as np
import pytest

from exact_attention_flash_amd import inputs
from oracle.dense import attention as oracle_attention
from tests import _golden
from tests._parity import assert_parity, half_ulp, metrics

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fa():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_attention_flash_amd as fa_mod

    fa_mod._native.lib()  # raises if the HIP library is not built
    return fa_mod


def _run_gpu(fa, qb, kb, vb, dtype, causal, scale, stream=None):
    dev = torch.device("cuda:0")
    q, k, v = (inputs.to_torch(x, dtype, dev) for x in (qb, kb, vb))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return inputs.bits_to_f64(inputs.from_torch_bits(o), dtype), lse.double().cpu().numpy()


def _oracle(qb, kb, vb, dtype, causal, scale, rows=None, heads=None):
    if heads is not None:  # select (batch, head) slices before widening to float64
        qb, kb, vb = (x.reshape(-1, *x.shape[-2:])[heads] for x in (qb, kb, vb))
    q, k, v = (inputs.bits_to_f64(x, dtype) for x in (qb, kb, vb))
    return oracle_attention(q, k, v, scale, causal=causal, rows=rows)


# N spans one to three 256-row query tiles and up to 11 64-key tiles, with ragged ends
SMALL_SHAPES = [(1, 1, 1, 64), (1, 1, 3, 128), (1, 2, 63, 64), (1, 1, 64, 128), (2, 3, 130, 64),
                (1, 2, 200, 128), (1, 1, 257, 128), (2, 2, 384, 64), (1, 1, 511, 128), (1, 2, 700, 64),
                (2, 1, 640, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
def test_small_shapes_full(fa, fwd_kernel, shape, dtype, causal):
    seed = 1000 + 7 * SMALL_SHAPES.index(shape) + (3 if causal else 0) + (1 if dtype == inputs.FP16 else 0)
    qb, kb, vb = inputs.draw_qkv(shape, dtype, 1.0, seed)
    scale = inputs.default_scale(shape[-1])
    o, lse = _run_gpu(fa, qb, kb, vb, dtype, causal, scale)
    ro, rl = _oracle(qb, kb, vb, dtype, causal, scale)
    m = metrics(o, lse, ro, rl, dtype)
    _log(f"small {fwd_kernel} {shape} {dtype} causal={causal}: {m}")
    assert_parity(m, f"{shape} {dtype} causal={causal}")


def _sample_rows(n, count, rng):
    fixed = [0, 1, 31, 32, 63, 64, 95, 127, 128, 129, 255, 256, n // 2, n - 129, n - 128, n - 65, n - 64,
             n - 33, n - 32, n - 2, n - 1]
    rows = set(r for r in fixed if 0 <= r < n)
    rows.update(rng.integers(0, n, size=count).tolist())
    return np.array(sorted(rows))


def _item_rows(n, h, rng):
    """One row of every 256-row query tile of slice h (the kernels' work item is a
    (slice, 256-row query tile) pair), at an in-tile offset that walks the eight
    32-row blocks the eight waves of a workgroup own as the slice and tile change,
    plus the tile and wave boundaries and a few random rows."""
    tiles = (n + 255) // 256
    rows = set()
    for t in range(tiles):
        blk = (h + t) % 8
        r = 256 * t + 32 * blk + (7 * h + 13 * t) % 32
        rows.add(min(r, n - 1))
    rows.update(_sample_rows(n, 8, rng).tolist())
    return np.array(sorted(rows))


CASES = [(name, c) for name, w in inputs.WORKLOADS.items() for c in w.causal]
# the headline shape without the mask: long items that cross into the next item of
# the same workgroup with every wave active (not one of the measured workloads)
EXTRA = {"llama7b_b2_h32_n4096_d128_noncausal": inputs.Workload(
    "llama7b_b2_h32_n4096_d128_noncausal", 2, 32, 4096, 128, inputs.BF16, 1.0, (False,), 3)}
CASES += [(name, c) for name, w in EXTRA.items() for c in w.causal]


@pytest.mark.parametrize("seed_offset,kernel", [(0, "picked"), (100, "picked"), (0, "other")])
@pytest.mark.parametrize("name,causal", CASES)
def test_workload_parity(fa, monkeypatch, name, causal, seed_offset, kernel):
    """Full size, in the launch configuration the benchmark times (the kernel the
    call picks), and through the other forward kernel: complete outputs where the
    oracle is quick, otherwise at least one row of every work item (slice, 256-row
    query tile) of every slice, plus complete slices."""
    w = inputs.WORKLOADS[name] if name in inputs.WORKLOADS else EXTRA[name]
    monkeypatch.delenv("FLASH_ATTN_FWD_KERNEL", raising=False)
    picked = fa._native.fwd_kernel(w.N, w.d, causal)
    assert picked in (fa._native.FA_FWD_KERNEL_PIPELINED, fa._native.FA_FWD_KERNEL_PINGPONG)
    if kernel == "other":
        monkeypatch.setenv("FLASH_ATTN_FWD_KERNEL",
                           "pingpong" if picked == fa._native.FA_FWD_KERNEL_PIPELINED else "pipelined")
    _log(f"workload {name} causal={causal}: kernel {kernel} (picked {picked})")
    t0 = time.time()
    qb, kb, vb = inputs.workload_qkv(w, seed_offset)
    scale = inputs.default_scale(w.d)
    _log(f"workload {name} causal={causal} seed={w.seed + seed_offset}: inputs ready {time.time() - t0:.1f}s")
    o, lse = _run_gpu(fa, qb, kb, vb, w.dtype, causal, scale)
    bh = w.B * w.H
    o = o.reshape(bh, w.N, w.d)
    lse = lse.reshape(bh, w.N)
    _log(f"  gpu done {time.time() - t0:.1f}s")
    if w.N * w.N * bh <= 1024 * 1024 * 64:
        ro, rl = _oracle(qb, kb, vb, w.dtype, causal, scale)
        m = metrics(o, lse, ro.reshape(bh, w.N, w.d), rl.reshape(bh, w.N), w.dtype)
        _log(f"  full oracle {time.time() - t0:.1f}s: {m}")
        assert_parity(m, name)
        return
    rng = np.random.default_rng(w.seed + seed_offset)
    go, gl, ro_all, rl_all = [], [], [], []
    n_rows = 0
    for h in range(bh):
        rows = _item_rows(w.N, h, rng)
        n_rows += len(rows)
        ro, rl = _oracle(qb, kb, vb, w.dtype, causal, scale, rows=rows, heads=[h])
        go.append(o[h, rows])
        gl.append(lse[h, rows])
        ro_all.append(ro[0])
        rl_all.append(rl[0])
    m = metrics(np.concatenate(go), np.concatenate(gl), np.concatenate(ro_all), np.concatenate(rl_all), w.dtype)
    _log(f"  {n_rows} rows covering every (slice, 256-row query tile) of {bh} slices {time.time() - t0:.1f}s: {m}")
    assert_parity(m, f"{name} sampled rows")
    # complete slices: the first and last (batch, head) slice, and one slice of the
    # long-context workload
    full_heads = [0, bh - 1] if w.N <= 4099 else [bh // 2]
    for h in full_heads:
        ro, rl = _oracle(qb, kb, vb, w.dtype, causal, scale, heads=[h])
        m = metrics(o[h], lse[h], ro[0], rl[0], w.dtype)
        _log(f"  full slice {h} {time.time() - t0:.1f}s: {m}")
        assert_parity(m, f"{name} slice {h}")


# Several work items per workgroup (the persistent grid has one workgroup per
# compute unit): the tile stream and the pipeline run across item boundaries.
MULTI_ITEM_SHAPES = [(8, 32, 512, 128), (16, 32, 512, 64), (6, 32, 704, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
@pytest.mark.parametrize("shape", MULTI_ITEM_SHAPES)
def test_multi_item_workgroups_full(fa, fwd_kernel, shape, dtype, causal):
    seed = 2000 + 11 * MULTI_ITEM_SHAPES.index(shape) + (3 if causal else 0) + (1 if dtype == inputs.FP16 else 0)
    qb, kb, vb = inputs.draw_qkv(shape, dtype, 1.0, seed)
    scale = inputs.default_scale(shape[-1])
    o, lse = _run_gpu(fa, qb, kb, vb, dtype, causal, scale)
    ro, rl = _oracle(qb, kb, vb, dtype, causal, scale)
    m = metrics(o, lse, ro, rl, dtype)
    _log(f"multi-item {fwd_kernel} {shape} {dtype} causal={causal}: {m}")
    assert_parity(m, f"{shape} {dtype} causal={causal}")


@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
def test_worked_example_padded(fa, dtype):
    """Scores [2,1,0] and values [1,3,5] (tokenlab note), as d = 64 with zeros elsewhere."""
    g = _golden.worked_example()
    n, d = 3, 64
    q = np.zeros((1, 1, n, d), np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    q[..., 0] = 1.0
    k[0, 0, :, 0] = g["scores"]
    v[0, 0, :, 0] = g["values"]
    qb, kb, vb = (inputs.to_bits(x, dtype) for x in (q, k, v))
    o, lse = _run_gpu(fa, qb, kb, vb, dtype, False, 1.0)
    # the printed value has 6 decimals; the output is that value rounded to the dtype
    tol = half_ulp(g["u_over_l"], dtype) + 1e-5
    assert np.all(np.abs(o[0, 0, :, 0] - g["u_over_l"]) <= tol)
    assert np.all(o[0, 0, :, 1:] == 0.0)
    assert np.allclose(lse, math.log(math.exp(2) + math.exp(1) + 1), atol=1e-5)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_and_zero_queries(fa, causal):
    B, H, N, d = 1, 2, 300, 128
    qb, kb, vb = inputs.draw_qkv((B, H, N, d), inputs.BF16, 1.0, 77)
    ones = inputs.to_bits(np.ones((B, H, N, d), np.float32), inputs.BF16)
    o, _ = _run_gpu(fa, qb, kb, ones, inputs.BF16, causal, inputs.default_scale(d))
    assert np.all(np.abs(o - 1.0) <= 2.0 ** -7)   # sum of rounded weights over the fp32 sum
    zeros = inputs.to_bits(np.zeros((B, H, N, d), np.float32), inputs.BF16)
    o, lse = _run_gpu(fa, zeros, kb, vb, inputs.BF16, causal, inputs.default_scale(d))
    v = inputs.bits_to_f64(vb, inputs.BF16)
    cnt = (np.arange(N) + 1) if causal else np.full(N, N)
    mean = (np.cumsum(v, axis=2) / cnt[:, None]) if causal else np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
    assert np.max(np.abs(o - mean)) <= 1e-2
    assert np.max(np.abs(lse - np.log(cnt))) <= 1e-5


def test_causal_prefix_is_bitwise_independent_of_later_rows(fa):
    """Rows < 4096 of a causal N = 4099 problem equal the N = 4096 problem exactly."""
    dtype = inputs.FP16
    qb, kb, vb = inputs.draw_qkv((1, 2, 4099, 128), dtype, 8.0, 55)
    o1, l1 = _run_gpu(fa, qb, kb, vb, dtype, True, inputs.default_scale(128))
    o2, l2 = _run_gpu(fa, qb[:, :, :4096].copy(), kb[:, :, :4096].copy(), vb[:, :, :4096].copy(),
                      dtype, True, inputs.default_scale(128))
    assert np.array_equal(o1[:, :, :4096], o2) and np.array_equal(l1[:, :, :4096], l2)


def test_deterministic_and_side_stream(fa):
    w = inputs.WORKLOADS["mha_b4_h16_n1024_d64"]
    qb, kb, vb = inputs.workload_qkv(w)
    a = _run_gpu(fa, qb, kb, vb, w.dtype, False, inputs.default_scale(w.d))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = _run_gpu(fa, qb, kb, vb, w.dtype, False, inputs.default_scale(w.d), stream=s)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_problem_touches_nothing(fa):
    q = torch.empty((2, 3, 0, 64), dtype=torch.bfloat16, device="cuda:0")
    o, lse = fa.forward(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)


@pytest.mark.parametrize("causal", [False, True])
def test_very_large_logits(fa, causal):
    """Logits in the thousands: no overflow; the result follows the largest scores."""
    B, H, N, d = 1, 2, 190, 64
    dtype = inputs.FP16
    qb, kb, vb = inputs.draw_qkv((B, H, N, d), dtype, 8.0, 91)
    scale = 2.0
    o, lse = _run_gpu(fa, qb, kb, vb, dtype, causal, scale)
    ro, rl = _oracle(qb, kb, vb, dtype, causal, scale)
    m = metrics(o, lse, ro, rl, dtype)
    _log(f"large logits causal={causal}: {m}")
    assert m["finite"]
    # the scores reach ~1e4 in magnitude; the LSE bound is relative to them
    assert np.max(np.abs(lse - rl) / np.maximum(1.0, np.abs(rl))) <= 1e-6
    assert m["o_max_excess"] <= 1e-2 and m["o_mean_abs"] <= 1e-3


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_large_values_bf16_scale_exactly(fa, causal, split):
    """bf16 values up to |v| ~ 2^99 at N = 1024 (2^96 times values below 8), inside the documented limit
    N * max|v| < 2^113 (probabilities reach 2^15 before normalisation). The value
    path is linear in V, and a power-of-two scale is exact in bf16 and fp32 while
    nothing overflows, so O(2^E V) must equal 2^E O(V) bit for bit and the LSE must
    not move; O(V) itself is checked against the oracle (inputs drawn like the bf16
    workloads, sigma = 1). The key-split path (four ranges and the merge) obeys the
    same contract."""
    B, H, N, d = 1, 2, 1024, 128
    dtype = inputs.BF16
    qb, kb, vb = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 57)
    scale = inputs.default_scale(d)

    def run(vbits):
        if not split:
            return _run_gpu(fa, qb, kb, vbits, dtype, causal, scale)
        dev = torch.device("cuda:0")
        q, k, v = (inputs.to_torch(x, dtype, dev) for x in (qb, kb, vbits))
        o_, lse_, used = fa.forward_splitkv(q, k, v, causal=causal, scale=scale, num_splits=4)
        torch.cuda.synchronize()
        assert used == 4
        return inputs.bits_to_f64(inputs.from_torch_bits(o_), dtype), lse_.double().cpu().numpy()

    o, lse = run(vb)
    ro, rl = _oracle(qb, kb, vb, dtype, causal, scale)
    m = metrics(o, lse, ro, rl, dtype)
    _log(f"large values causal={causal} split={split} base: {m}")
    assert_parity(m, "large values base")
    v64 = inputs.bits_to_f64(vb, dtype)
    assert np.max(np.abs(v64)) < 2.0 ** 3
    for e in (40, 80, 96):
        big = np.ldexp(v64, e)
        vb_big = inputs.to_bits(big.astype(np.float32), dtype)
        assert np.array_equal(inputs.bits_to_f64(vb_big, dtype), big)
        ob, lb = run(vb_big)
        _log(f"large values causal={causal} split={split} 2^{e}: max|O| {np.max(np.abs(ob)):.3e}")
        assert np.all(np.isfinite(ob))
        assert np.array_equal(ob, np.ldexp(o, e))
        assert np.array_equal(lb, lse)


def test_launch_log_names_the_instance():
    """FLASH_ATTN_LOG=1 (read once per process, hence a child process): every launch
    prints its kernel instance and grid to stderr."""
    import os
    import subprocess

    code = (
        "import os, torch, exact_attention_flash_amd as fa\n"
        "q = torch.randn(1, 8, 300, 128, device='cuda', dtype=torch.bfloat16)\n"
        "o, lse = fa.forward(q, q, q, causal=True)\n"
        "os.environ['FLASH_ATTN_FWD_KERNEL'] = 'pipelined'\n"
        "o, lse = fa.forward(q, q, q, causal=True)\n"
        "fa.backward(q, q, q, o, lse, torch.randn_like(q), causal=True)\n"
        "torch.cuda.synchronize()\n")
    env = dict(os.environ, FLASH_ATTN_LOG="1")
    env.pop("FLASH_ATTN_FWD_KERNEL", None)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stderr[-2000:]
    _log(res.stderr.strip())
    lines = [l for l in res.stderr.splitlines() if l.startswith("flash_attn: ")]
    # d = 128: the ping-pong kernel; then the pipelined one, forced
    assert lines[0].startswith("flash_attn: fwd_pingpong<bf16, 128, causal, whole> grid "), lines
    assert lines[1].startswith("flash_attn: fwd_sp<bf16, 128, causal> grid 16 x 512, 16 items"), lines
    assert any("bwd_dkdv<bf16, 128, causal>" in l for l in lines[2:]), lines


@pytest.mark.parametrize("pattern", ["rising", "first_spike"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [inputs.BF16, inputs.FP16])
def test_reference_changes(fa, dtype, causal, pattern):
    """Row maxima that move a long way between key tiles.

    "rising": key tile j is scaled by 1 + j/2, so with scale 2 every tile's scores
    exceed the previous tile's reference by far more than the kept-reference slack
    (2^15 in probability) and the reference must be replaced many times. "first_spike": key 0 is scaled by 8, so the
    first tile's reference stays far above every later score and later
    probabilities are tiny against it.
    """
    B, H, N, d = 1, 2, 700, 64
    qb, kb, vb = inputs.draw_qkv((B, H, N, d), dtype, 1.0, 17)
    k = inputs.bits_to_f64(kb, dtype)
    if pattern == "rising":
        k = k * (1.0 + 0.5 * (np.arange(N) // 64))[None, None, :, None]
    else:
        k[:, :, 0, :] *= 8.0
    kb = inputs.to_bits(k.astype(np.float32), dtype)
    scale = 2.0
    o, lse = _run_gpu(fa, qb, kb, vb, dtype, causal, scale)
    ro, rl = _oracle(qb, kb, vb, dtype, causal, scale)
    m = metrics(o, lse, ro, rl, dtype)
    _log(f"reference changes {pattern} {dtype} causal={causal}: {m}")
    assert m["finite"]
    assert np.max(np.abs(lse - rl) / np.maximum(1.0, np.abs(rl))) <= 1e-6
    assert m["o_max_excess"] <= 1e-2 and m["o_mean_abs"] <= 1e-3
