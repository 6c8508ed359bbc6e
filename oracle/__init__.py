"""fp64 CPU oracle of the per-matrix Muon update (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may
import this package; the HIP library and its binding never do and share no code with it.
"""

from .muon import (DEFAULT_COEFFS, DEFAULT_SEGMENTS, frobenius_normalise, momentum,
                   muon_step, newton_schulz_gram, newton_schulz_plain, ns_round, orient,
                   orthogonalise, weight_update)
from .flop_model import dense_flops, product_counts

__all__ = [
    "DEFAULT_COEFFS", "DEFAULT_SEGMENTS", "momentum", "orient", "frobenius_normalise",
    "ns_round", "newton_schulz_plain", "newton_schulz_gram", "weight_update",
    "orthogonalise", "muon_step", "dense_flops", "product_counts",
]
