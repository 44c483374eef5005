"""Float64 restatement of the update -- TEST INFRASTRUCTURE (pins the C oracle).

Computes the same mathematics as FA-ja "この演算子を使用する理由" (RUDA docs
page "実験的なデバイス上の融合 AdamW / AMSGrad") entirely in float64 from the
FP32 inputs, with exact-as-float64 coefficients (Python float powers), no
FP32 casts anywhere.  It is written independently of ``radamw_oracle.c`` and
serves as the "true value" the FP32 oracle must approach within a few ulps.
"""
from __future__ import annotations

import numpy as np


def step64(p, g_stored, m, v, vmax, t, lr, beta1, beta2, eps, weight_decay,
           amsgrad, maximize, gradient_scale):
    """Return (p, m, v, vmax) after update t, all float64 arrays.

    ``g_stored`` holds the stored gradient values already widened to float
    (their exact values); ``m, v, vmax`` are the previous moments (zeros for
    t == 1)."""
    p = np.asarray(p, np.float64)
    grad = np.asarray(g_stored, np.float64) / float(gradient_scale)
    if maximize:
        grad = -grad
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * grad
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * grad * grad
    if amsgrad:
        vmax = np.maximum(np.asarray(vmax, np.float64), v)
        second = vmax
    else:
        second = v
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = second / (1.0 - beta2 ** t)
    p = p * (1.0 - lr * weight_decay) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v, (vmax if amsgrad else None)
