"""Plain fp64 oracle for the AdamW step applied beside Muon to 1-D and embedding parameters.

TEST INFRASTRUCTURE ONLY (same rules as the rest of ``oracle``): imported by ``tests/`` only,
and it shares nothing with the HIP library.

Source: "Moonlight 16B Guide: Scalable MoE & Muon Optimizer", section "The Coordinate-Wise
Limitation of AdamW" (first and second moment estimates and the update with decoupled weight
decay) and section "The Hybrid Optimization Strategy" (AdamW for RMSNorm scales, biases,
router projections and token embeddings; Muon for the 2-D matrices).

The guide's update is
    m_t = beta1 m_{t-1} + (1 - beta1) g_t
    v_t = beta2 v_{t-1} + (1 - beta2) g_t^2
    theta_{t+1} = theta_t - lr m_t / (sqrt(v_t) + eps) - lr wd theta_t
with eps outside the square root and no bias correction. Readings: the displayed equation
governs (the guide's ASCII diagram puts eps inside the square root; the equation is the
plainer statement), and the optional bias correction (m_t / (1 - beta1^t), v_t / (1 - beta2^t),
the usual Adam form the guide does not print) is available as a switch, off by default.
"""
from __future__ import annotations

import numpy as np


def adamw_step(theta, g, m, v, lr: float, beta1: float, beta2: float, eps: float, wd: float,
               step: int = 1, bias_correction: bool = False):
    """One AdamW step on flat fp64 arrays; returns (theta_next, m_next, v_next)."""
    theta = np.asarray(theta, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    mh, vh = m, v
    if bias_correction:
        mh = m / (1.0 - beta1 ** step)
        vh = v / (1.0 - beta2 ** step)
    theta_next = theta - lr * mh / (np.sqrt(vh) + eps) - lr * wd * theta
    return theta_next, m, v
