"""Accuracy and throughput bookkeeping for F^H D results.

Accuracy (page "Chapter 17: MRI Reconstruction", section 17.3 step 3, which
judges the reduced-accuracy trig by PSNR without giving a formula):

* rel_l2  = ||rho - ref||_2 / ||ref||_2 over the complex vector (the gate);
* psnr_db = 20 log10( max_n |ref_n| / sqrt(mean_n |rho_n - ref_n|^2) ), with
  complex magnitudes over the compared voxels (reported, not gated).

Work accounting per voxel-sample term, a fixed convention since the pages
give none: 13 FLOP (phase 3 mul + 2 add, complex multiply-accumulate 4 mul +
4 add, an FMA counted as 2) and 2 transcendentals (sin, cos).
"""
from __future__ import annotations

import numpy as np

FLOP_PER_TERM = 13
TRANS_PER_TERM = 2


def _c(re, im) -> np.ndarray:
    return np.asarray(re, np.float64) + 1j * np.asarray(im, np.float64)


def rel_l2(re, im, ref_re, ref_im) -> float:
    a, b = _c(re, im), _c(ref_re, ref_im)
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    return float(num / den) if den > 0 else float(num)


def max_abs_err(re, im, ref_re, ref_im) -> float:
    return float(np.max(np.abs(_c(re, im) - _c(ref_re, ref_im)), initial=0.0))


def rms(re, im) -> float:
    a = _c(re, im)
    return float(np.sqrt(np.mean(np.abs(a) ** 2))) if a.size else 0.0


def psnr_db(re, im, ref_re, ref_im) -> float:
    a, b = _c(re, im), _c(ref_re, ref_im)
    mse = float(np.mean(np.abs(a - b) ** 2))
    peak = float(np.max(np.abs(b), initial=0.0))
    if mse == 0.0:
        return float("inf")
    return float(20.0 * np.log10(peak / np.sqrt(mse)))


def terms_per_s(N: int, M: int, seconds: float) -> float:
    return float(N) * float(M) / seconds


def gflops(N: int, M: int, seconds: float) -> float:
    return FLOP_PER_TERM * terms_per_s(N, M, seconds) / 1e9
