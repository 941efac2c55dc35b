"""Parity metrics between the GPU output and the float64 oracle.

Tolerances (written here once, used by every GPU parity test):

* O: mean absolute error <= 1e-3, and the maximum absolute error in excess of
  half a unit in the last place of the output dtype at the oracle's value,
  max(|O_gpu - O_ref| - ulp(O_ref)/2, 0), <= 1e-2. The plain maximum is also
  computed and reported. The excess form is needed because the output is
  stored in bf16/fp16: with N(0, 8^2) inputs |O| reaches ~47, where one fp16 ulp
  is 2^-5, so even the exact result rounded once is up to 1.56e-2 away from
  itself -- no 16-bit output could meet a literal 1e-2 there.
* LSE (fp32 output): maximum absolute error <= 1e-3.
"""
import numpy as np

from exact_attention_flash_amd import inputs

O_MAX_EXCESS = 1e-2
O_MEAN = 1e-3
LSE_MAX = 1e-3

_MANT = {inputs.BF16: 7, inputs.FP16: 10}
_MIN_EXP = {inputs.BF16: -126, inputs.FP16: -14}


def half_ulp(x, dtype):
    """Half the spacing of `dtype` numbers at |x| (subnormal spacing near 0)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(ax))
    e = np.maximum(np.where(np.isfinite(e), e, _MIN_EXP[dtype]), _MIN_EXP[dtype])
    return np.ldexp(0.5, (e - _MANT[dtype]).astype(np.int64))


def metrics(o_gpu, lse_gpu, o_ref, lse_ref, dtype):
    err = np.abs(o_gpu - o_ref)
    excess = np.maximum(err - half_ulp(o_ref, dtype), 0.0)
    return {
        "o_max_abs": float(err.max()) if err.size else 0.0,
        "o_max_excess": float(excess.max()) if err.size else 0.0,
        "o_mean_abs": float(err.mean()) if err.size else 0.0,
        "lse_max_abs": float(np.abs(lse_gpu - lse_ref).max()) if lse_ref.size else 0.0,
        "finite": bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))),
    }


def assert_parity(m, label=""):
    assert m["finite"], f"{label}: non-finite output"
    assert m["o_max_excess"] <= O_MAX_EXCESS, f"{label}: O max excess {m['o_max_excess']:.3e}"
    assert m["o_mean_abs"] <= O_MEAN, f"{label}: O mean abs {m['o_mean_abs']:.3e}"
    assert m["lse_max_abs"] <= LSE_MAX, f"{label}: LSE max abs {m['lse_max_abs']:.3e}"
