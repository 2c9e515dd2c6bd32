"""Helpers shared by the GPU parity tests: moving seeded inputs between torch
and the oracle's float64 world, and the comparison rules.

Tolerances (normwise relative error, ||got - ref||_F / ||ref||_F):
  fp32 1e-5, bf16 / fp16 5e-3.
"""
import sys

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-5, "f16": 5e-3, "bf16": 5e-3}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def log(msg):
    """Name the case on stdout before a GPU step (flushed, survives a crash)."""
    print(msg, flush=True)
    sys.stdout.flush()


def raw(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU or GPU tensor: float32 array, or uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.int8:
        return t.numpy().astype(np.float64)
    raise TypeError(t.dtype)


def f64(t: torch.Tensor, dtype: str) -> np.ndarray:
    """float64 values of a tensor, decoded by the oracle's own format routines."""
    if t.dtype == torch.int8:
        return t.detach().cpu().numpy().astype(np.float64)
    return oracle.decode_dtype(raw(t), dtype)


def dev(t, device="cuda"):
    return None if t is None else t.to(device)


def assert_close(got_t, ref64, dtype, what=""):
    got = f64(got_t, dtype)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = oracle.normwise_rel_error(got, ref64)
    assert err <= TOL[dtype], f"{what}: normwise rel err {err:.3e} > {TOL[dtype]:.1e}"
    return err


def assert_bits_equal(a: torch.Tensor, b, what=""):
    ra = raw(a)
    rb = raw(b) if isinstance(b, torch.Tensor) else b
    if ra.dtype == np.float32:
        ra = ra.view(np.uint32)
        rb = rb.view(np.uint32) if rb.dtype == np.float32 else rb
    bad = np.nonzero(ra.reshape(-1) != rb.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} elements differ (first at flat index {bad[0]})"


def encode_dtype(x64, dtype):
    """Storage bits the oracle assigns to float64 values."""
    if dtype == "f32":
        return oracle.round_f32(x64).astype(np.float32)
    return oracle.encode(x64, dtype)
