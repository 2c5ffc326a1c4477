"""Shared helpers for the GPU parity tests (comparison against the oracle)."""

from __future__ import annotations

import numpy as np
import torch

import oracle as O
from global_gqa_rope_amd import api
from global_gqa_rope_amd.workloads import LayerShape

# Tolerances for this path: bf16 I/O max |err| <= 2e-2 and relative L2 <= 5e-3;
# fp32 I/O both <= 1e-5.
TOL = {torch.bfloat16: (2e-2, 5e-3), torch.float32: (1e-5, 1e-5)}


def oracle_layer(shape: LayerShape) -> O.OracleLayer:
    return O.OracleLayer(shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.window,
                         shape.kv_shared, shape.rope_theta, shape.rope_fraction, shape.norm_eps)


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got: torch.Tensor, want: np.ndarray) -> tuple[float, float]:
    g = to64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert np.isfinite(g).all(), "non-finite values in the GPU output"
    diff = g - want
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    rel = float(np.linalg.norm(diff) / max(np.linalg.norm(want), 1e-30))
    return max_abs, rel


def assert_close(got: torch.Tensor, want: np.ndarray, dtype: torch.dtype, what: str) -> None:
    max_abs, rel = errors(got, want)
    tol_abs, tol_rel = TOL[dtype]
    print(f"[parity] {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}", flush=True)
    assert max_abs <= tol_abs and rel <= tol_rel, f"{what}: max_abs={max_abs:.3e} rel={rel:.3e}"


def device() -> torch.device:
    return torch.device("cuda", 0)


def api_layer(shape: LayerShape, dtype) -> api.Layer:
    return api.Layer.from_shape(shape, dtype)
