"""fp64 AdamW for the token embedding E and the LM head U.

TEST INFRASTRUCTURE ONLY (same rules as gpt_oracle: tests, the smoke check and
the benchmark's CPU baseline may use it; the product path never does).

The nanochat articles hand the embeddings and the LM head to AdamW and the 2-D
block matrices to Muon (the table of parameter types in section "2. Muon
Optimize Edici" of the Turkish dev.to page, and the same table in its Arabic
translation).  They print neither AdamW's formula nor its hyperparameters, so
the plainest reading is taken: Adam's bias-corrected first and second moments
(Kingma & Ba, "Adam: A Method for Stochastic Optimization", Algorithm 1) with the
weight decay decoupled from the gradient and applied to the weight before the
step (Loshchilov & Hutter, "Decoupled Weight Decay Regularization", Algorithm 2
with the schedule multiplier fixed at 1).  Learning rate, betas, epsilon and
decay are arguments.  For the t-th call (t = 1, 2, ...) with gradient g:

    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    w <- w - lr wd w - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
"""
from __future__ import annotations

import numpy as np


def adamw_step(w, g, m, v, t, lr, beta1, beta2, eps, wd):
    """One AdamW step on one tensor (t counts from 1); returns new (w, m, v) in fp64."""
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    w = w - lr * wd * w - lr * m_hat / (np.sqrt(v_hat) + eps)
    return w, m, v
