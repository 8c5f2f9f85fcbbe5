"""Shared helpers of the test suite: tolerance rules and GPU availability.

Tolerance rules (applied per output tensor, comparing the GPU result upcast to
float64 with the fp64 oracle):
  * fp32 inputs: max|gpu - ref| / max|ref| <= 1e-4.
  * bf16 inputs: every element within 2e-2 * RMS(ref), plus, for outputs
    stored in bf16, the half-ulp of that element's own bf16 rounding
    (2^-8 * |ref|):  |gpu - ref| <= 2e-2 * RMS(ref) + 2^-8 * |ref|.
    The allowance exists because rounding an exact result to bf16 can by
    itself exceed 2e-2 * RMS: KDA outputs are heavy-tailed (max|o|/RMS ~ 14 on
    the synthetic workloads), and a bf16 rounding costs up to 2^-8 * |o|.
    The fp32 final state gets no allowance.
"""
import math

import numpy as np
import torch

FP32_MAX_REL = 1e-4
BF16_RMS_REL = 2e-2
BF16_HALF_ULP = 2.0 ** -8


def gpu_available() -> bool:
    try:
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def np64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").to(torch.float64).numpy()


def error_metrics(gpu, ref, stored_bf16: bool):
    gpu = np64(gpu)
    ref = np64(ref)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    rms = math.sqrt(float(np.mean(ref * ref))) if ref.size else 0.0
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    excess = err - (BF16_HALF_ULP * np.abs(ref) if stored_bf16 else 0.0)
    return dict(
        max_abs=float(err.max()) if err.size else 0.0,
        max_rel=float(err.max()) / mx if mx > 0 else float(err.max() if err.size else 0.0),
        max_over_rms=float(err.max()) / rms if rms > 0 else 0.0,
        excess_over_rms=float(excess.max()) / rms if rms > 0 else 0.0,
        rms_over_rms=math.sqrt(float(np.mean(err * err))) / rms if rms > 0 else 0.0,
        finite=bool(np.all(np.isfinite(gpu))),
    )


def assert_close(gpu, ref, io_dtype, stored_in_io_dtype: bool, what: str = ""):
    """Assert the tolerance rule above; returns the metrics."""
    m = error_metrics(gpu, ref, stored_bf16=(io_dtype == torch.bfloat16 and stored_in_io_dtype))
    assert m["finite"], "%s: non-finite values" % what
    if io_dtype == torch.float32:
        assert m["max_rel"] <= FP32_MAX_REL, "%s: max rel err %.3e > %.0e (%s)" % (
            what, m["max_rel"], FP32_MAX_REL, m)
    else:
        assert m["excess_over_rms"] <= BF16_RMS_REL, "%s: error %.3e RMS beyond the bf16 allowance (%s)" % (
            what, m["excess_over_rms"], m)
    return m
