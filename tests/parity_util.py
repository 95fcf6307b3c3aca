"""Shared helpers of the GPU parity tests: tensor -> exact fp64 numpy copies,
the tolerance metric, and oracle calls on sub-batches."""
import numpy as np
import torch

# Tolerances by storage dtype of the compared tensor: relative L2 error per
# unit (request x head, or sequence x head), maximised over units.
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a float tensor (bf16 and fp32 convert without loss)."""
    return t.detach().to(torch.float32).cpu().to(torch.float64).numpy()


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "fp32", torch.bfloat16: "bf16"}[t.dtype]


def rel_err_units(got, ref, unit_dims: int) -> float:
    """max over units of ||got - ref||_2 / ||ref||_2, where a unit is an index
    into the first `unit_dims` axes."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n_units = int(np.prod(got.shape[:unit_dims]))
    g = got.reshape(n_units, -1)
    r = ref.reshape(n_units, -1)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def assert_close_units(got, ref, unit_dims, dtype, what):
    err = rel_err_units(got, ref, unit_dims)
    tol = TOL[dtype]
    assert err <= tol, f"{what}: max per-unit relative L2 error {err:.3e} > {tol:.0e}"
    return err
