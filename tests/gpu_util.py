"""Helpers for the GPU parity tests: bf16 bits <-> device tensors, and the
parity bar.

Parity bar (fixed for this path): for every output tensor,
    max |gpu - ref| <= 1e-2 * max |ref| + 1e-3,
with ref the fp64 oracle computed from the same bf16-rounded inputs.
"""
import numpy as np
import torch

import datagen

DEV = torch.device("cuda:0")


def to_dev(bits: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    if dtype == torch.bfloat16:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(bits)).to(DEV)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64_of_bits(bits: np.ndarray) -> np.ndarray:
    return datagen.bf16_to_f32(bits).astype(np.float64)


def f64_of(t: torch.Tensor) -> np.ndarray:
    return f64_of_bits(bits_of(t))


def tol_of(ref: np.ndarray) -> float:
    return 1e-2 * float(np.max(np.abs(ref))) + 1e-3 if ref.size else 1e-3


def assert_parity(gpu: torch.Tensor, ref: np.ndarray, what: str = "") -> float:
    if gpu.dtype == torch.float32:
        got = gpu.detach().cpu().numpy().astype(np.float64).reshape(ref.shape)
    else:
        got = f64_of(gpu).reshape(ref.shape)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    tol = tol_of(ref)
    print(f"  parity {what}: max|gpu-ref| = {err:.3e}  tol = {tol:.3e}", flush=True)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= tol, f"{what}: max|gpu-ref| = {err:.3e} > tol {tol:.3e}"
    return err


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def rand_bf16(rng, shape, scale=1.0, kind="normal"):
    if kind == "normal":
        return datagen.rne_bf16((rng.standard_normal(shape) * scale).astype(np.float32))
    return datagen.rne_bf16((rng.uniform(-scale, scale, shape)).astype(np.float32))
