"""Tolerance helpers shared by the GPU parity tests.

Two checks per output element, both against the oracle's float64 result:

* rounded: |gpu - RNE_dtype(oracle)| <= max(tol, ulp_dtype(oracle)).  Both
  sides are rounded to the output dtype; a value whose unrounded result lands
  on the other side of a rounding boundary than the oracle's differs from the
  rounded reference by exactly one unit in the last place, however accurate
  it is, so one ulp is accepted where it exceeds tol (bf16 outputs of
  magnitude >= 0.5).
* unrounded: |gpu - oracle| <= tol + ulp_dtype / 2 (+ extra).  The GPU's own
  rounding to the output dtype costs at most half an ulp, so any drift of the
  unrounded GPU result beyond tol shows here even where the rounded check's
  one-ulp allowance would hide it.  `extra` carries roundings the method
  itself prescribes before the final one: the two-phase decode stores every
  partition's output in the output dtype (page "paged_attention_v2_pytorch.py",
  the partition-output store into tmp_output, read back by the
  cross-partition reduction), so the combined output carries
  sum_p (w_p / W) * ulp(o_p) / 2 on top (tmp_rounding_budget).
"""
import numpy as np
import torch

MANTISSA_BITS = {torch.float32: 23, torch.float16: 10, torch.bfloat16: 7}


def ulp(x, dtype):
    """Unit in the last place of `dtype` at |x| (normal range; tiny values get the smallest normal's)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - MANTISSA_BITS[dtype])


def rne(a, dtype):
    """Round float64 values to `dtype` (nearest, ties to even) and widen back."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype).double().numpy()


def allowed_error(ref_rounded, dtype, tol):
    return np.maximum(tol, ulp(ref_rounded, dtype))


def tmp_rounding_budget(max_logits, exp_sums, tmp_output, dtype):
    """sum_p (w_p / W) * ulp_dtype(o_p) / 2 per head-dim element, from the
    oracle's float64 statistics of one (sequence, head): the error the pages'
    rounding of each partition output to the output dtype can add to phase 2's
    weighted mean (w_p = exp(m_p - M) l_p, W = sum_p w_p)."""
    m = np.asarray(max_logits, dtype=np.float64)
    w = np.exp(m - m.max()) * np.asarray(exp_sums, dtype=np.float64)
    w = w / w.sum()
    # ulp of the value rounded up to the next binade where it sits at the top of one
    o = np.abs(np.asarray(tmp_output, dtype=np.float64)) * (1.0 + 2.0 ** -MANTISSA_BITS[dtype])
    return (w[:, None] * 0.5 * ulp(o, dtype)).sum(axis=0)


def check(got, ref64, dtype, tol, what="", extra=0.0):
    """Both checks for one array; returns the max error against the rounded reference."""
    got = np.asarray(got, dtype=np.float64)
    ref64 = np.asarray(ref64, dtype=np.float64)
    r = rne(ref64, dtype)
    err = np.abs(got - r)
    assert (err <= allowed_error(r, dtype, tol)).all(), f"{what}: max err {err.max():.3g} vs rounded oracle (tol {tol:.3g})"
    eu = np.abs(got - ref64)
    bound = tol + 0.5 * ulp(np.maximum(np.abs(got), np.abs(ref64)), dtype) + extra
    assert (eu <= bound).all(), \
        f"{what}: max err {eu.max():.3g} vs unrounded oracle beyond tol + ulp/2 (worst excess {(eu - bound).max():.3g})"
    return float(err.max()) if err.size else 0.0
