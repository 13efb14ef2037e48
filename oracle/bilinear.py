"""Bilinear block schemes for matrix multiplication — TEST INFRASTRUCTURE ONLY (part
of the oracle package; only the tests, the smoke check and bench.py's CPU baseline
use it).

A scheme <mb, kb, nb; R> splits op(A) into mb x kb blocks, op(B) into kb x nb
blocks and C into mb x nb blocks, and forms R block products

    P_r = (sum_a U[r, a] A_a) (sum_b V[r, b] B_b),     C_c = sum_r W[c, r] P_r

(FalconGEMM page, Methodology item 1: Strassen-like, Winograd-based and
tensor-decomposition low-complexity algorithms).  Block a = (i, j) of A has index
i*kb + j, block b = (j, l) of B index j*nb + l, block c = (i, l) of C index i*nb + l.
A scheme computes the product exactly in exact arithmetic iff its tables satisfy the
Brent equations: sum_r U[r, (i, j)] V[r, (j', l)] W[(i', l'), r] equals 1 when
j = j', i = i' and l = l', and 0 otherwise (`brent_ok` checks every one, in integers).

Schemes here:
  S69        <2,2,2;7>   Strassen (1969)
  WINOGRAD   <2,2,2;7>   Winograd's form (its chained sums expanded)
  R223       <2,2,3;11>  rectangular: Strassen (1969) on the first two column blocks
                         of B and C, and the four block products of the third
                         (C13 = A11 B13 + A12 B23, C23 = A21 B13 + A22 B23); eleven is
                         the smallest rank of the <2,2,3> product.
"""
from __future__ import annotations

import numpy as np


def _scheme(mb, kb, nb, products, outputs):
    """products: list of (dict A-block -> coefficient, dict B-block -> coefficient), with
    blocks named 'A11'.. and 'B11'..; outputs: dict C-block name -> dict product index
    (1-based) -> coefficient."""
    R = len(products)
    U = np.zeros((R, mb * kb), dtype=np.int64)
    V = np.zeros((R, kb * nb), dtype=np.int64)
    W = np.zeros((mb * nb, R), dtype=np.int64)
    for r, (ua, vb) in enumerate(products):
        for name, c in ua.items():
            U[r, (int(name[1]) - 1) * kb + int(name[2]) - 1] = c
        for name, c in vb.items():
            V[r, (int(name[1]) - 1) * nb + int(name[2]) - 1] = c
    for name, terms in outputs.items():
        for p, c in terms.items():
            W[(int(name[1]) - 1) * nb + int(name[2]) - 1, p - 1] = c
    return {"mb": mb, "kb": kb, "nb": nb, "U": U, "V": V, "W": W}


S69 = _scheme(2, 2, 2, [
    ({"A11": 1, "A22": 1}, {"B11": 1, "B22": 1}),
    ({"A21": 1, "A22": 1}, {"B11": 1}),
    ({"A11": 1}, {"B12": 1, "B22": -1}),
    ({"A22": 1}, {"B21": 1, "B11": -1}),
    ({"A11": 1, "A12": 1}, {"B22": 1}),
    ({"A21": 1, "A11": -1}, {"B11": 1, "B12": 1}),
    ({"A12": 1, "A22": -1}, {"B21": 1, "B22": 1}),
], {"C11": {1: 1, 4: 1, 5: -1, 7: 1}, "C12": {3: 1, 5: 1}, "C21": {2: 1, 4: 1},
    "C22": {1: 1, 2: -1, 3: 1, 6: 1}})

# Winograd's form: S1 = A21 + A22, S2 = S1 - A11, S3 = A11 - A21, S4 = A12 - S2;
# T1 = B12 - B11, T2 = B22 - T1, T3 = B22 - B12, T4 = T2 - B21; P1 = A11 B11,
# P2 = A12 B21, P3 = S4 B22, P4 = A22 T4, P5 = S1 T1, P6 = S2 T2, P7 = S3 T3;
# C11 = P1 + P2, C12 = P1 + P6 + P5 + P3, C21 = P1 + P6 + P7 - P4, C22 = P1 + P6 + P7 + P5.
WINOGRAD = _scheme(2, 2, 2, [
    ({"A11": 1}, {"B11": 1}),
    ({"A12": 1}, {"B21": 1}),
    ({"A12": 1, "A21": -1, "A22": -1, "A11": 1}, {"B22": 1}),
    ({"A22": 1}, {"B22": 1, "B12": -1, "B11": 1, "B21": -1}),
    ({"A21": 1, "A22": 1}, {"B12": 1, "B11": -1}),
    ({"A21": 1, "A22": 1, "A11": -1}, {"B22": 1, "B12": -1, "B11": 1}),
    ({"A11": 1, "A21": -1}, {"B22": 1, "B12": -1}),
], {"C11": {1: 1, 2: 1}, "C12": {1: 1, 6: 1, 5: 1, 3: 1}, "C21": {1: 1, 6: 1, 7: 1, 4: -1},
    "C22": {1: 1, 6: 1, 7: 1, 5: 1}})

R223 = _scheme(2, 2, 3, [
    ({"A11": 1, "A22": 1}, {"B11": 1, "B22": 1}),
    ({"A21": 1, "A22": 1}, {"B11": 1}),
    ({"A11": 1}, {"B12": 1, "B22": -1}),
    ({"A22": 1}, {"B21": 1, "B11": -1}),
    ({"A11": 1, "A12": 1}, {"B22": 1}),
    ({"A21": 1, "A11": -1}, {"B11": 1, "B12": 1}),
    ({"A12": 1, "A22": -1}, {"B21": 1, "B22": 1}),
    ({"A11": 1}, {"B13": 1}),
    ({"A12": 1}, {"B23": 1}),
    ({"A21": 1}, {"B13": 1}),
    ({"A22": 1}, {"B23": 1}),
], {"C11": {1: 1, 4: 1, 5: -1, 7: 1}, "C12": {3: 1, 5: 1}, "C21": {2: 1, 4: 1},
    "C22": {1: 1, 2: -1, 3: 1, 6: 1}, "C13": {8: 1, 9: 1}, "C23": {10: 1, 11: 1}})

SCHEMES = {"S69": S69, "WINOGRAD": WINOGRAD, "R223": R223}


def brent_ok(s) -> bool:
    """Every Brent equation of the scheme, in exact integer arithmetic."""
    mb, kb, nb, U, V, W = s["mb"], s["kb"], s["nb"], s["U"], s["V"], s["W"]
    for i in range(mb):
        for j in range(kb):
            for j2 in range(kb):
                for l in range(nb):
                    for i2 in range(mb):
                        for l2 in range(nb):
                            t = int(np.sum(U[:, i * kb + j] * V[:, j2 * nb + l] *
                                           W[i2 * nb + l2, :]))
                            want = 1 if (j == j2 and i == i2 and l == l2) else 0
                            if t != want:
                                return False
    return True


def blocks(X, rows: int, cols: int):
    """The rows x cols blocks of X in row-major block order (equal sizes)."""
    h, w = X.shape[0] // rows, X.shape[1] // cols
    return [X[i * h:(i + 1) * h, j * w:(j + 1) * w] for i in range(rows) for j in range(cols)]


def apply(A, B, s):
    """op(A) op(B) through the scheme, fp64, from fp64 operands (dimensions divisible by
    the block counts): the operand sums, the R products (library matmul as a step),
    the output combinations."""
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    mb, kb, nb, U, V, W = s["mb"], s["kb"], s["nb"], s["U"], s["V"], s["W"]
    if A.shape[1] != B.shape[0] or A.shape[0] % mb or A.shape[1] % kb or B.shape[1] % nb:
        raise ValueError("shapes do not split into the scheme's blocks")
    Ab, Bb = blocks(A, mb, kb), blocks(B, kb, nb)
    P = []
    for r in range(U.shape[0]):
        S = sum(U[r, a] * Ab[a] for a in range(mb * kb) if U[r, a])
        T = sum(V[r, b] * Bb[b] for b in range(kb * nb) if V[r, b])
        P.append(S @ T)
    C = np.empty((A.shape[0], B.shape[1]))
    h, w = A.shape[0] // mb, B.shape[1] // nb
    for c in range(mb * nb):
        i, l = divmod(c, nb)
        C[i * h:(i + 1) * h, l * w:(l + 1) * w] = sum(W[c, r] * P[r] for r in range(U.shape[0])
                                                      if W[c, r])
    return C
