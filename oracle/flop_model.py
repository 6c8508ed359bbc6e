"""Matrix-multiply FLOP model of one NS update, as the MuonX article counts it.

TEST INFRASTRUCTURE ONLY (see ``oracle/muon.py``): used by tests and by the bench's
baseline leg, never by the product path; the library carries its own, independent count.

MuonX article (Baidu Baige, damodev.csdn.net), section 3.2 "Gram NS: fewer long matrix
products": for one 2560 x 9728 momentum matrix, plain NS does 10 long products and 5
small square ones; Gram NS split 2 + 2 + 1 does 6 long and 11 square ones, and the
theoretical matmul work falls from 1.443 to 1.134 TFLOPs (about -21.4%).

Counting rule (the plainest reading that reproduces those numbers): with the short side
m' and the long side n', a long product (X X^T, or an m' x m' matrix times X) costs
``2 m'^2 n'`` FLOPs and a square m' x m' product costs ``2 m'^3``. The counts below follow
the operation sequence of ``oracle.muon``: a plain round is X X^T, A^2 and B X (two long,
one square); a Gram segment of s rounds is one X X^T and one Q X (two long) plus one
square product in its first round (R^2) and four in each later round (Q R, (Q R) Q^T,
A^2, P Q).
"""

from __future__ import annotations


def product_counts(mode: str, segments=(2, 2, 1), rounds=None):
    """Return ``(long, square)`` product counts for one NS update."""
    if mode == "plain":
        r = int(sum(segments)) if rounds is None else int(rounds)
        return 2 * r, r
    if mode == "gram":
        longs = 2 * len(segments)
        squares = sum(1 + 4 * (int(s) - 1) for s in segments)
        return longs, squares
    raise ValueError(f"unknown mode {mode!r}")


def dense_flops(rows: int, cols: int, mode: str, segments=(2, 2, 1), rounds=None) -> float:
    """Dense matmul FLOPs of one NS update of a rows x cols matrix (short side m')."""
    m, n = min(rows, cols), max(rows, cols)
    n_long, n_square = product_counts(mode, segments, rounds)
    return float(n_long) * 2.0 * m * m * n + float(n_square) * 2.0 * m * m * m
