"""Parity tolerances of the GPU tests and the rounding bound of the forward output.

The O, LSE and gradient bars are those stated for bf16 inputs: O max-abs 1e-2, LSE
relative 1e-3, gradients max-norm-relative 2e-2.  ``rounding_bound`` is the error the
forward's own rounding steps can produce for one output element (the rounding reading:
probabilities rounded to bf16 before the P.V product, fp32 accumulation, output rounded
to bf16); the synthetic edge cases, whose rows attend to one or a few keys so that |O|
reaches 2-4, are held to max(1e-2, rounding bound).  ``tests/test_tolerance_model.py``
checks on the CPU that an emulation of those rounding steps stays inside the bound.
"""
from __future__ import annotations

import numpy as np

O_ATOL = 1e-2
LSE_RTOL = 1e-3
LSE_ATOL = 1e-5          # absolute floor of the LSE bound, for |LSE| < 1e-2
GRAD_RTOL = 2e-2
P_ROUND = 2.0 ** -8      # bf16 unit roundoff of each probability before the P.V product
ACC_ROUND = 2.0 ** -12   # fp32 accumulation and exp2 error, relative to sum_j P_ij |V_jc|


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def rounding_bound(Oref, Aabs):
    """Bound on |O - O*| per element from the forward's rounding steps.

    Aabs = sum_j P_ij |V_jc| (the attention output for the values |V|).  Each rounded
    probability is off by at most 2^-8 of itself, which moves O_ic by at most
    2^-8 Aabs_ic; fp32 accumulation adds far less than 2^-12 Aabs_ic; the final rounding
    to bf16 adds half an ulp of the (so perturbed) result.
    """
    model = (P_ROUND + ACC_ROUND) * Aabs
    return 0.5 * bf16_ulp(np.abs(Oref) + model) + model
