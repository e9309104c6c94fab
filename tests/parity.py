"""Comparison helpers shared by the GPU parity tests.

The bar: relative Frobenius error per output tensor, ||G - O||_F / ||O||_F,
at most 1e-5 for fp32 storage and 2e-2 for bf16 storage (fp32 accumulate);
an all-zero reference requires an all-zero result.  Every element must also
lie within 4*tol*(|O| + rms(O)) of the oracle, which no rounding of the
stated arithmetic approaches but a wrong tile, row or column does.
"""
import numpy as np

import oracle

TOL = {0: 1e-5, 1: 2e-2}   # by storage type: TP_F32, TP_BF16


def rel_frob(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    nr = np.linalg.norm(ref)
    if nr == 0:
        return 0.0 if not np.any(got) else float("inf")
    return float(np.linalg.norm(got - ref) / nr)


def assert_close(name, got, ref, tol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    r = rel_frob(got, ref)
    assert r <= tol, f"{name}: relative Frobenius error {r:.3e} > {tol:.1e}"
    if ref.size:
        rms = np.sqrt(np.mean(ref * ref))
        bound = 4 * tol * (np.abs(ref) + rms)
        bad = np.abs(got - ref) > bound
        if np.any(bad):
            i = np.argwhere(bad)[0]
            raise AssertionError(f"{name}: element {tuple(i)} = {got[tuple(i)]:.6g}, "
                                 f"oracle {ref[tuple(i)]:.6g}")
    return r


def f64(a):
    """Host storage array (uint16 bf16 bits or float32) -> float64."""
    return oracle.to_f64(a)


def sample_idx(n: int, k: int):
    """k fixed indices spread over [0, n), always including the last one."""
    if n <= k:
        return np.arange(n)
    idx = sorted(set([(j * n) // k for j in range(k)] + [n - 1]))
    return np.array(idx, dtype=np.int64)
