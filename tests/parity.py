"""Normwise comparison used by the parity tests.

For a tensor pair (got, ref): max|got - ref| / max|ref| and
mean|got - ref| / mean|ref|.  Elementwise relative errors are ill-posed where
ref crosses zero, so the tolerances are normwise per tensor.
Tolerances: fp32 runs 1e-4 (max); bf16-in / fp32-accumulate runs 2e-2 (max)
and 1e-2 (mean).
"""
import numpy as np

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}


def errors(got, ref, allowance=None):
    """Normwise (max, mean) relative errors.  `allowance` (same shape) is an
    absolute error that output storage alone may introduce (half an ulp of the
    stored value); it is subtracted from |got - ref| before the norms."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    d = np.abs(got - ref)
    if allowance is not None:
        d = np.maximum(d - allowance, 0.0)
    mx = np.max(np.abs(ref))
    mn = np.mean(np.abs(ref))
    return (np.max(d) / mx if mx > 0 else np.max(d)), (np.mean(d) / mn if mn > 0 else np.mean(d))


def half_ulp(stored, dtype):
    """Half an ulp of values stored in `dtype` (bf16: 8 significant bits,
    fp32: 24): the rounding a correct result suffers when it is written out."""
    bits = 8 if dtype == "bf16" else 24
    return np.abs(np.asarray(stored, dtype=np.float64)) * 2.0 ** -bits


def check(name, got, ref, dtype, allowance=None):
    tmax, tmean = TOL[dtype]
    emax, emean = errors(got, ref, allowance)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert emax <= tmax and emean <= tmean, f"{name}: max-rel {emax:.3e} (tol {tmax}), mean-rel {emean:.3e} (tol {tmean})"
    return emax, emean
