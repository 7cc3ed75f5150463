"""Tolerance checks shared by the GPU parity tests.

Two metrics, both from the stated bar for this path:
* relative L2 error ||y - y_ref|| / ||y_ref||, evaluated per slice (every
  (batch, head) for retention outputs, the whole tensor for the layer) so that
  heads with small outputs are not hidden by large ones; the worst slice counts;
* max-abs error on unit-normalised outputs: both y and y_ref divided by the
  RMS of y_ref over the same slice.

fp32 paths: rel-L2 <= 1e-4.  bf16-input / fp32-accumulate paths:
rel-L2 <= 2e-2 and unit-normalised max-abs <= 5e-2.
"""
import numpy as np

FP32_REL_L2 = 1e-4
BF16_REL_L2 = 2e-2
BF16_MAX_ABS = 5e-2


def to_np(x):
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype in (torch.bfloat16, torch.float16):
            x = x.float()
        x = x.double().numpy()
    return np.asarray(x, dtype=np.float64)


def errors(y, ref, slice_dims=2):
    """(worst rel-L2, worst unit-normalised max-abs) over slices made of the
    leading `slice_dims` axes."""
    y, ref = to_np(y), to_np(ref)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    lead = int(np.prod(y.shape[:slice_dims])) if slice_dims else 1
    y2, r2 = y.reshape(lead, -1), ref.reshape(lead, -1)
    diff = y2 - r2
    nref = np.linalg.norm(r2, axis=1)
    rel = np.linalg.norm(diff, axis=1) / np.maximum(nref, 1e-300)
    rms = np.sqrt((r2 ** 2).mean(axis=1))
    mabs = np.abs(diff).max(axis=1) / np.maximum(rms, 1e-300)
    if not np.all(np.isfinite(y2)):
        return float("inf"), float("inf")
    return float(rel.max()), float(mabs.max())


def assert_fp32(y, ref, slice_dims=2, tol=FP32_REL_L2, what=""):
    rel, _ = errors(y, ref, slice_dims)
    assert rel <= tol, f"{what}: rel-L2 {rel:.3e} > {tol:.1e}"
    return rel


def assert_bf16(y, ref, slice_dims=2, what=""):
    rel, mabs = errors(y, ref, slice_dims)
    assert rel <= BF16_REL_L2 and mabs <= BF16_MAX_ABS, \
        f"{what}: rel-L2 {rel:.3e} (<= {BF16_REL_L2}), unit max-abs {mabs:.3e} (<= {BF16_MAX_ABS})"
    return rel, mabs
