"""Pass/fail rule shared by the parity tests.

|gpu - ref| <= 1e-3·sqrt(K) + 2^-10·|ref| elementwise, ref in fp64.  The
absolute term covers fp32 accumulation over K terms of size <= 1; the relative
term covers the final rounding to fp16 (at most 2^-11·|ref|).
"""
import numpy as np


def bound(K, ref):
    return 1e-3 * np.sqrt(max(int(K), 1)) + 2.0 ** -10 * np.abs(ref)


def check_close(out, ref, K, what=""):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    err = np.abs(out - ref)
    lim = bound(K, ref)
    bad = ~(err <= lim)          # NaN in out counts as a failure
    if bad.any():
        idx = np.argwhere(bad)[:5]
        details = ", ".join(f"{tuple(i)}: got {out[tuple(i)]!r} ref {ref[tuple(i)]!r}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} entries out of tolerance "
                             f"(max err {np.nanmax(err):.3g}); first: {details}")
    return float(err.max()) if err.size else 0.0
