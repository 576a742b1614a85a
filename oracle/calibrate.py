"""Per-layer K/V scale calibration, float64 reference.

The pages require one finite, positive K scale and one V scale per attention
layer, produced offline and refused when missing, non-finite or non-positive
("Integrate calibrated E4M3 QSA KV capacity path", Changes and Validation
boundary; "Calibrated E4M3 KV cache for Qwen4Exp QSA with MTP", Status and
history). They do not state the calibration rule. Reading used here: the
scale maps the tensor's largest magnitude onto the largest E4M3 value,
scale = fl32(amax / 448), with amax the maximum |x| over the calibration set.
"""

import numpy as np

STATUS_OK = 0
STATUS_BAD_SCALE = 2
STATUS_NONFINITE_INPUT = 3


def quotient_f32(num, den) -> np.ndarray:
    """Correctly rounded float32 quotient of float32 operands.

    The float64 quotient rounded once to float32 equals the correctly rounded
    float32 quotient: double rounding is innocuous for division when the wide
    format has at least 2p + 2 bits of precision (53 >= 2 * 24 + 2; Figueroa,
    "When is double rounding innocuous?", 1995).
    """
    n = np.asarray(num, dtype=np.float32).astype(np.float64)
    d = np.asarray(den, dtype=np.float32).astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        return (n / d).astype(np.float32)


def calibrate_amax(x_f16):
    """amax and scale of each row of an fp16 [n_tensors, n_elems] array.

    Returns (amax float32[n], scale float32[n], status). amax is the exact
    maximum magnitude (an fp16 value, exact in float32). A row holding any
    non-finite element gets NaN for both outputs and the call reports
    NONFINITE_INPUT (3); otherwise a row whose amax is zero gets amax = scale
    = 0 and the call reports BAD_SCALE (2); otherwise status is OK (0).
    """
    x = np.asarray(x_f16, dtype=np.float16)
    if x.ndim == 1:
        x = x[None, :]
    finite = np.isfinite(x).all(axis=1)
    mag = np.abs(x.astype(np.float64))
    mag[~np.isfinite(mag)] = 0.0
    amax = mag.max(axis=1) if x.shape[1] else np.zeros(x.shape[0])
    amax32 = amax.astype(np.float32)
    scale = quotient_f32(amax32, np.float32(448.0))
    amax32[~finite] = np.float32(np.nan)
    scale[~finite] = np.float32(np.nan)
    if not finite.all():
        status = STATUS_NONFINITE_INPUT
    elif (amax32 == 0).any():
        status = STATUS_BAD_SCALE
    else:
        status = STATUS_OK
    return amax32, scale, status
