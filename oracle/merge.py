"""Oracle: merge of two partial attention results.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Ring Attention glossary page ("Como funciona la atencion en anillo") combines the
partial results of the key blocks with the cumulative softmax: each device keeps a
running sum of the exponentiated scores and of the weighted values and divides one
by the other at the end.  A partial result over a key subset A is carried as
(O_A, LSE_A) with O_A = num_A / den_A and LSE_A = ln den_A (natural log), so
num_A = e^{LSE_A} O_A and den_A = e^{LSE_A}.  Adding the sums of two disjoint subsets
and dividing again gives

    LSE = ln(e^{LSE_A} + e^{LSE_B})
    O   = (e^{LSE_A} O_A + e^{LSE_B} O_B) / e^{LSE}

A subset with no visible key is (O = 0, LSE = -inf), the identity of the merge.
Written with the larger LSE factored out so that no exponential overflows.
"""

import numpy as np


def lse_merge(o_a, lse_a, o_b, lse_b):
    """o [S][H][D], lse [H][S] (float64) -> merged (o, lse)."""
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    mx = np.maximum(lse_a, lse_b)
    empty = ~np.isfinite(mx)
    mx_safe = np.where(empty, 0.0, mx)
    den_a = np.exp(lse_a - mx_safe)          # e^{LSE_A} / e^{mx}; 0 when LSE_A = -inf
    den_b = np.exp(lse_b - mx_safe)
    den = den_a + den_b
    lse = np.where(empty, -np.inf, mx_safe + np.log(np.where(empty, 1.0, den)))
    wa = np.where(empty, 0.0, den_a / np.where(empty, 1.0, den))   # [H][S]
    wb = np.where(empty, 0.0, den_b / np.where(empty, 1.0, den))
    o = wa.T[:, :, None] * o_a + wb.T[:, :, None] * o_b
    return o, lse
