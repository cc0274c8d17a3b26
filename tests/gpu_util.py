"""Helpers for the GPU parity tests: device copies of seeded inputs and the
error metrics and tolerances the comparisons use."""

from __future__ import annotations

import numpy as np

# Tolerances for O (bf16) and LSE (fp32) against the fp64 oracle.
O_REL_L2 = 5e-3
O_MAX_ABS = 2e-2
LSE_MAX_ABS = 1e-3


def to_device(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on the GPU."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    """GPU tensor (bf16 or fp32) -> float64 numpy array."""
    import torch

    return t.detach().to("cpu", dtype=torch.float64).numpy()


def bits_of(t) -> np.ndarray:
    import torch

    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def errors(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray):
    """(relative L2 of O, max |O - O_ref|, max |LSE - LSE_ref|)."""
    diff = o_gpu - o_ref
    rel = float(np.linalg.norm(diff.ravel()) / max(np.linalg.norm(o_ref.ravel()), 1e-300))
    return rel, float(np.max(np.abs(diff))), float(np.max(np.abs(lse_gpu - lse_ref)))


def assert_close(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    rel, mx, lmx = errors(o_gpu, lse_gpu, o_ref, lse_ref)
    print(f"[parity] {what}: rel_l2={rel:.3e} max_abs={mx:.3e} lse_abs={lmx:.3e}", flush=True)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), f"{what}: non-finite"
    assert rel <= O_REL_L2, f"{what}: O relative L2 {rel:.3e} > {O_REL_L2}"
    assert mx <= O_MAX_ABS, f"{what}: O max abs {mx:.3e} > {O_MAX_ABS}"
    assert lmx <= LSE_MAX_ABS, f"{what}: LSE max abs {lmx:.3e} > {LSE_MAX_ABS}"
    return rel, mx, lmx
