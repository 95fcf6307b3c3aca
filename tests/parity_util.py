"""Shared helpers of the GPU parity tests: tensor -> exact fp64 numpy copies,
the tolerance metric, and oracle calls on sub-batches.

The bar has two parts, both at the tolerance of the compared tensor's
storage dtype (1e-4 for fp32, 2e-2 for bf16):
  * per unit (request x head for decode tokens, sequence x head for the
    outputs of a prefill call, slot x head for states):
    ||got - ref||_2 / ||ref||_2, maximised over units;
  * per element: |got - ref| / max(|ref|, rms of the element's unit),
    maximised over elements, so a single wrong element fails even inside a
    128 x 128 state head.  A unit whose reference is all zeros takes the
    rms of the whole reference tensor as its floor; where that is zero too,
    the element must match exactly.
Every check prints both figures and the largest absolute difference.

One derived exception: in the prefill's bf16x3 mode every matrix-core
product is formed from operands split into bf16 hi + lo, which carries about
16 significant bits (the dropped lo x lo term and the rounding of each lo
part bound a product's error by about 3 * 2^-18 |a b|).  An fp32 output or
state element is a sum of 128 to 192 such products of random sign, so its
error against the unit's rms reaches ~1e-4 at the worst elements of long
resumed sequences, while the errors average out over a unit (~1.5e-5).  For
fp32 tensors produced in that mode the element bar is ELEM_TOL_SPLIT; the
per-unit bar stays 1e-4, and the fp32 mode keeps 1e-4 for both.
"""
import numpy as np
import torch

TOL = {"fp32": 1e-4, "bf16": 2e-2}
ELEM_TOL_SPLIT = 3e-4


def elem_tol(dtype: str, split_products: bool) -> float:
    """The per-element bar of a tensor of `dtype`, computed with bf16-split
    matrix-core products or not."""
    return ELEM_TOL_SPLIT if split_products and dtype == "fp32" else TOL[dtype]


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a float tensor (bf16 and fp32 convert without loss)."""
    return t.detach().to(torch.float32).cpu().to(torch.float64).numpy()


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "fp32", torch.bfloat16: "bf16"}[t.dtype]


def _units(got, ref, unit_dims):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    n_units = int(np.prod(got.shape[:unit_dims]))
    return got.reshape(n_units, -1), ref.reshape(n_units, -1)


def rel_err_units(got, ref, unit_dims: int) -> float:
    """max over units of ||got - ref||_2 / ||ref||_2, where a unit is an index
    into the first `unit_dims` axes."""
    g, r = _units(got, ref, unit_dims)
    num = np.linalg.norm(g - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if len(num) else 0.0


def elem_err(got, ref, unit_dims: int):
    """(max over elements of |got - ref| / max(|ref|, unit rms), max |got - ref|)."""
    g, r = _units(got, ref, unit_dims)
    if g.size == 0:
        return 0.0, 0.0
    diff = np.abs(g - r)
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    floor = np.where(rms > 0, rms, np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), floor)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(den > 0, diff / np.where(den > 0, den, 1.0),
                         np.where(diff > 0, np.inf, 0.0))
    return float(np.max(ratio)), float(np.max(diff))


def assert_close_units(got, ref, unit_dims, dtype, what, etol=None):
    err = rel_err_units(got, ref, unit_dims)
    el, mabs = elem_err(got, ref, unit_dims)
    tol = TOL[dtype]
    etol = tol if etol is None else etol
    print(f"[parity] {what}: unit rel L2 {err:.2e}, element {el:.2e}, max abs {mabs:.2e} "
          f"(tol {tol:.0e}, element {etol:.0e})", flush=True)
    assert err <= tol, f"{what}: max per-unit relative L2 error {err:.3e} > {tol:.0e}"
    assert el <= etol, (f"{what}: max element error {el:.3e} (|got - ref| over max(|ref|, "
                        f"unit rms)) > {etol:.0e}")
    return err


def assert_close_seqs(got, ref, cu_seqlens, dtype, what, etol=None):
    """The bar of assert_close_units over prefill outputs [T, H, d] with the
    unit (sequence, head): the tokens cu_seqlens[n] .. cu_seqlens[n+1] - 1 of
    one head.  A single token's output is a poor unit under strong decay:
    it is then about (q_t . k_t) beta_t v_t, and when q_t . k_t nearly
    cancels no fixed-precision evaluation stays within a relative bound of
    it (a plain fp32 token-by-token evaluation of the definition misses
    1e-4 there; tests/test_tolerance_units.py)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    cu = np.asarray(cu_seqlens).astype(np.int64)
    tol = TOL[dtype]
    etol = tol if etol is None else etol
    errs, els, mabss = [0.0], [0.0], [0.0]  # np.max keeps a NaN (Python's max would drop it)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            continue
        g = np.swapaxes(got[a:b], 0, 1)  # [H, tokens, d]: one unit per head
        r = np.swapaxes(ref[a:b], 0, 1)
        errs.append(rel_err_units(g, r, 1))
        e, m = elem_err(g, r, 1)
        els.append(e)
        mabss.append(m)
    err, el, mabs = float(np.max(errs)), float(np.max(els)), float(np.max(mabss))
    print(f"[parity] {what}: unit (sequence, head) rel L2 {err:.2e}, element {el:.2e}, "
          f"max abs {mabs:.2e} (tol {tol:.0e}, element {etol:.0e})", flush=True)
    assert err <= tol, f"{what}: max per-unit relative L2 error {err:.3e} > {tol:.0e}"
    assert el <= etol, (f"{what}: max element error {el:.3e} (|got - ref| over max(|ref|, "
                        f"unit rms)) > {etol:.0e}")
    return err
