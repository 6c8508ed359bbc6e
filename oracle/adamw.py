"""Plain fp64 CPU oracle of the AdamW step for the parameters Muon does not update.

TEST INFRASTRUCTURE ONLY, like ``oracle/muon.py``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may call it, and it
shares no code with the HIP library.

Source: the MuonX article (Baidu Baige, damodev.csdn.net), section 2 "why fewer but slower
steps": AdamW adjusts every element on its own from running averages of the gradient and
of its square, and in practice the hidden 2-D weight matrices go to Muon while embeddings,
biases and similar parameters stay with AdamW.

The pages print no AdamW formula. Reading (the usual decoupled-decay AdamW, element by
element, at step t = 1, 2, ...):

    W  <- W * (1 - lr * wd)
    m  <- beta1 * m + (1 - beta1) * g
    v  <- beta2 * v + (1 - beta2) * g^2
    W  <- W - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

Pins (``tests/test_oracle.py``): the first step from m = v = 0 reduces to
``W(1 - lr wd) - lr g / (|g| + eps)``; a constant gradient gives the geometric-series
state in closed form; torch.optim.AdamW on the CPU (an implementation of its own) agrees
over several steps.
"""

from __future__ import annotations

import numpy as np


def adamw_step(W, G, m, v, t, *, lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0):
    """One AdamW step at step number ``t`` (1-based). All arrays are read as float64;
    returns ``(W', m', v')`` as new float64 arrays."""
    if t < 1:
        raise ValueError("step numbers start at 1")
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    W = W * (1.0 - lr * wd)                                   # decoupled weight decay
    m = beta1 * m + (1.0 - beta1) * G                         # first moment
    v = beta2 * v + (1.0 - beta2) * G * G                     # second moment
    m_hat = m / (1.0 - beta1 ** t)                            # bias corrections
    v_hat = v / (1.0 - beta2 ** t)
    W = W - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W, m, v
