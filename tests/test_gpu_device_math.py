"""Error bounds of the device math the kernels use (la_device.h), measured
on the GPU against fp64 libm through a probe library (tests/devmath):

* exp_acc (chunked prefill): within 3 ulp of exp(x) for every x whose
  result is a normal fp32 number, and within 2^-126 absolutely below that;
* fast_exp (decode, verify, commit, conv): relative error within
  1.25 |x| 2^-24 + 4 ulp: the fp32 product t = x log2(e) is off by up to
  |t| 2^-24, which 2^t turns into a relative error of |t| 2^-24 ln 2 =
  |x| 2^-24; log2(e) rounded to fp32 is 0.22 ulp low, another 0.22 |x| 2^-24;
  then the hardware exp2 and the rounding of its result;
* silu(y) = y / (1 + e^-y) with a hardware reciprocal: the same bound in
  |y| (e^-y carries it where it dominates the sum).
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "devmath", "libdevmath.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        from devmath import build_probe
        build_probe.build()
    lib = ctypes.CDLL(LIB)
    lib.devmath_eval.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
    lib.devmath_eval.restype = ctypes.c_int
    return lib


def run(lib, x, which, dev):
    xd = torch.from_numpy(x.astype(np.float32)).to(dev)
    yd = torch.empty_like(xd)
    assert lib.devmath_eval(ctypes.c_void_p(xd.data_ptr()), ctypes.c_void_p(yd.data_ptr()),
                            xd.numel(), which) == 0
    return yd.cpu().numpy().astype(np.float64)


def ulp32(v):
    """Spacing of fp32 numbers at |v| (normal range)."""
    return np.spacing(np.abs(v).astype(np.float32)).astype(np.float64)


def inputs():
    rng = np.random.default_rng(5)
    grid = np.linspace(-104.0, 0.0, 400001)
    return np.concatenate([grid, rng.uniform(-160, 88, 200000), -rng.exponential(1.0, 100000),
                           [0.0, -1e-30, -87.3, -88.0, -103.9]]).astype(np.float32)


def test_exp_acc_within_3_ulp(probe, dev):
    x = inputs()
    y = run(probe, x, 0, dev)
    ref = np.exp(x.astype(np.float64))
    normal = ref >= 2.0 ** -126
    err = np.abs(y - ref)
    ulps = err[normal] / ulp32(ref[normal])
    print(f"exp_acc: max {ulps.max():.2f} ulp over {normal.sum()} normal results; "
          f"max abs error below normal {err[~normal].max() if (~normal).any() else 0:.2e}")
    assert ulps.max() <= 3.0
    assert (~normal).sum() == 0 or err[~normal].max() <= 2.0 ** -126


def test_fast_exp_error_grows_with_the_product_rounding(probe, dev):
    rng = np.random.default_rng(6)
    x = np.concatenate([np.linspace(-30.0, 30.0, 200001), rng.normal(0, 1, 100000)]).astype(np.float32)
    y = run(probe, x, 1, dev)
    ref = np.exp(x.astype(np.float64))
    rel = np.abs(y - ref) / ref
    bound = 1.25 * np.abs(x.astype(np.float64)) * 2.0 ** -24 + 4 * 2.0 ** -24
    print(f"fast_exp: max relative error {rel.max():.2e}, max ratio to bound {(rel / bound).max():.2f}")
    assert np.all(rel <= bound)


def test_silu_relative_error(probe, dev):
    y_in = np.concatenate([np.linspace(-30.0, 30.0, 300001),
                           np.random.default_rng(7).normal(0, 2, 100000)]).astype(np.float32)
    y = run(probe, y_in, 2, dev)
    v = y_in.astype(np.float64)
    ref = v / (1.0 + np.exp(-v))
    nz = np.abs(ref) > 1e-30
    rel = np.abs(y[nz] - ref[nz]) / np.abs(ref[nz])
    bound = 1.25 * np.abs(v[nz]) * 2.0 ** -24 + 4 * 2.0 ** -24
    print(f"silu: max relative error {rel.max():.2e}, max ratio to bound {(rel / bound).max():.2f}")
    assert np.all(rel <= bound)
