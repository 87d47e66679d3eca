"""Derivation of the normal-CDF polynomial used by the bf16 LUT build.

Phi(u) - 1/2 is odd, so on [-4, 4] it is fitted by
    P(s) = s * (c0 + c1 s^2 + ... + c9 s^18),  s = u / 4,
by least squares on 4000 Chebyshev nodes of [-4, 4] (fp64).  Beyond |u| = 4
the kernel clamps Phi to 0 or 1 (1 - Phi(4) = 3.2e-5).  Prints the fp32
coefficients pasted into build_lut.hip and the fit's maximum error (about
8e-7 for Phi, i.e. far below the 2^-9 relative rounding of the bf16 hidden
activations the build stores).

    python mixture_lookup_experts_amd/csrc/gelu_poly_fit.py
"""
import numpy as np
from scipy.special import ndtr

L, NTERM = 4.0, 10


def fit():
    x = np.cos(np.pi * (np.arange(4000) + 0.5) / 4000) * L
    s = x / L
    basis = np.stack([s ** (2 * k + 1) for k in range(NTERM)], axis=1)
    c, *_ = np.linalg.lstsq(basis, ndtr(x) - 0.5, rcond=None)
    return c.astype(np.float32)


def phi_poly(u, c):
    u = np.clip(np.asarray(u, np.float64), -L, L)
    s = u / L
    s2 = s * s
    p = np.zeros_like(s)
    for k in range(NTERM - 1, -1, -1):
        p = p * s2 + c[k]
    return np.clip(0.5 + s * p, 0.0, 1.0)


if __name__ == "__main__":
    c = fit()
    xx = np.linspace(-8, 8, 400001)
    err = np.max(np.abs(phi_poly(xx, c.astype(np.float64)) - ndtr(xx)))
    print("coefficients (fp32):")
    for k, v in enumerate(c):
        print("  c%d = %.9e" % (k, v))
    print("max |Phi_poly - Phi| on [-8, 8]: %.3e" % err)
