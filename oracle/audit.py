"""Plain fp64 CPU oracle of the expert-weight audit: exact-zero count and the
robust spread sigma_rob of a weight tensor, per slice (e.g. per expert) and
over the whole tensor.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU baseline may import or run this module; the library path never calls it
and shares no code with it.

Source: the model-hub discussion "singular matrices in Qwen3.8-2.4T-A95B":
its table of expert tensors with their share of zero entries ("zer%"), and
its definition of the robust spread,
    sigma_rob = 1.4826 * median(|w_i - median(w)|),
the median absolute deviation scaled by 1.4826 ~ 1 / Phi^-1(3/4), so that it
estimates the standard deviation of normally distributed weights.

Readings where the page leaves a step open (listed in the design notes):
  * the median of an even number of values is the mean of the two middle
    ones (both medians, the inner and the outer);
  * the constant is 1.4826 as printed, not 1 / Phi^-1(3/4) to more digits;
  * a zero is a value equal to 0 (both signed zeros count);
  * a NaN anywhere in a slice makes its median, MAD and sigma_rob NaN (the
    median of a set containing NaN is undefined); an empty slice has NaN
    statistics;
  * the inputs are bf16 tensors (the page's proposed recheck on the BF16
    files), read exactly into fp64.
"""
from __future__ import annotations

import numpy as np

SIGMA_ROB_SCALE = 1.4826


def audit_values(w: np.ndarray) -> dict:
    """Statistics of one flat set of weights (any shape, read as fp64)."""
    v = np.asarray(w, dtype=np.float64).reshape(-1)
    n = int(v.size)
    n_nan = int(np.isnan(v).sum())
    n_zero = int((v == 0.0).sum())
    if n == 0 or n_nan:
        med = mad = np.nan
    else:
        with np.errstate(invalid="ignore"):  # inf - inf where the median is infinite: NaN, as defined
            med = float(np.median(v))
            mad = float(np.median(np.abs(v - med)))
    sig = SIGMA_ROB_SCALE * mad
    return {"n": n, "n_zero": n_zero, "n_nan": n_nan, "median": med, "mad": mad, "sigma_rob": sig,
            "zero_frac": n_zero / n if n else np.nan}


def audit(w: np.ndarray, slices: int) -> tuple[list, dict]:
    """w holds `slices` equal slices one after another (e.g. [E, I, H] with one
    slice per expert).  Returns (per-slice statistics, whole-tensor statistics)."""
    v = np.asarray(w, dtype=np.float64).reshape(slices, -1)
    return [audit_values(v[s]) for s in range(slices)], audit_values(v)
