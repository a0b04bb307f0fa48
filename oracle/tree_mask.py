"""CPU oracle of the tree-verify visibility bitmask (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; it shares no code with the HIP library.

What it computes: tree node i may attend tree node j exactly when j is i or an
ancestor of i -- the visibility the verify attention applies to the tree block
("The GPU That Wasn't There", The Native Engine Thesis; "The Moment of
Certainty", The Path Forward: From Diagnosis to Solution). The pages do not
spell out the parent-array encoding; the reading taken here: parent[i] in
[-1, i) with -1 for a root, and any other value read as -1 (a malformed entry
starts a new root rather than reaching outside the tree).

Method: the plain definition of reachability, written as a closure of the
boolean "is parent of" relation. A[i, j] = 1 iff j = parent(i); the
ancestor-or-self relation is R = I + A + A^2 + ... + A^(N-1), formed by
repeated boolean products until it stops changing. Bits are then packed into
W = ceil(N/32) little-endian 32-bit words per node (bit j & 31 of word j >> 5),
the layout the attention reads.
"""
from __future__ import annotations

import numpy as np


def parent_relation(parents: np.ndarray) -> np.ndarray:
    """Boolean [B, N, N] matrix A with A[b, i, j] = (j is the parent of i)."""
    parents = np.asarray(parents, dtype=np.int64)
    B, N = parents.shape
    A = np.zeros((B, N, N), dtype=bool)
    for b in range(B):
        for i in range(N):
            p = int(parents[b, i])
            if 0 <= p < i:  # -1 and malformed values: a root, no edge
                A[b, i, p] = True
    return A


def ancestor_or_self(parents: np.ndarray) -> np.ndarray:
    """Boolean [B, N, N] matrix R with R[b, i, j] = (j == i or j is an ancestor of i)."""
    A = parent_relation(parents)
    B, N, _ = A.shape
    eye = np.broadcast_to(np.eye(N, dtype=bool), (B, N, N))
    R = eye.copy()
    while True:
        # one more step up the tree from every node already reached
        step = np.matmul(R.astype(np.int64), A.astype(np.int64)) > 0
        nxt = R | step
        if np.array_equal(nxt, R):
            return R
        R = nxt


def pack_bits(R: np.ndarray) -> np.ndarray:
    """[B, N, N] booleans -> uint32 [B, N, W] words, bit j & 31 of word j >> 5."""
    B, N, _ = R.shape
    W = (N + 31) // 32
    out = np.zeros((B, N, W), dtype=np.uint64)
    for j in range(N):
        out[:, :, j >> 5] |= R[:, :, j].astype(np.uint64) << np.uint64(j & 31)
    return out.astype(np.uint32)


def tree_mask(parents: np.ndarray) -> np.ndarray:
    """The bitmask mla_tree_verify takes as tree_mask, uint32 [B, N, W]."""
    return pack_bits(ancestor_or_self(parents))
