"""CPU oracle of the KV-row moves after a verify step (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module; it shares no code with the HIP library.

Tier-0 keeps each request's KV rows contiguous in the pool ("The Moment of
Reckoning: A User's Challenge That Reshaped a Long-Context Inference
Investigation", Output Knowledge Created by This Message), while the verify
block's tree nodes sit at scattered slots ("The Moment of Certainty", The User
Provides the Final Piece). The pages give no more than that; the readings taken
(stated with the library's entry points):

commit  -- for sequence b with S = seq_len clamped to [N, max_kv], t0 = S - N
           and L = accept_len clamped to [0, N], accepted node n_k = path[k]
           (clamped to [0, N)) moves from slot table[t0 + n_k] to
           base + t0 + k, and table[t0 + k] becomes that slot. All of a
           sequence's sources are read before any of its destinations is
           written.
defrag  -- positions [0, S) (S clamped to [0, max_kv]) move from their table
           slots to base + p and the table becomes base + p; destinations do
           not overlap sources, so every source is read before any write.
Slots read are clamped to [0, P); a destination outside the pool is skipped
and its table entry kept.

Rows are compared as raw 16-bit patterns: a move is exact.
"""
from __future__ import annotations

import numpy as np


def _clamp(v, lo, hi):
    return max(lo, min(hi, int(v)))


def kv_commit(pool: np.ndarray, table: np.ndarray, seq_lens, num_nodes: int, accept_len,
              accept_path, region_base):
    """Returns (pool', table') after the commit; inputs are not modified."""
    pool = np.array(pool, copy=True)
    table = np.array(table, copy=True)
    P = pool.shape[0]
    B, max_kv = table.shape
    N = int(num_nodes)
    for b in range(B):
        S = _clamp(seq_lens[b], N, max_kv)
        t0 = S - N
        L = _clamp(accept_len[b], 0, N)
        src = [_clamp(table[b, t0 + _clamp(accept_path[b][k], 0, N - 1)], 0, P - 1) for k in range(L)]
        rows = [pool[s].copy() for s in src]  # every source read first
        for k in range(L):
            d = int(region_base[b]) + t0 + k
            if 0 <= d < P:
                pool[d] = rows[k]
                table[b, t0 + k] = d
    return pool, table


def kv_defrag(pool: np.ndarray, table: np.ndarray, seq_lens, region_base):
    """Returns (pool', table') after moving every sequence to its run."""
    pool = np.array(pool, copy=True)
    table = np.array(table, copy=True)
    P = pool.shape[0]
    B, max_kv = table.shape
    moves = []
    for b in range(B):
        S = _clamp(seq_lens[b], 0, max_kv)
        for p in range(S):
            s = _clamp(table[b, p], 0, P - 1)
            moves.append((b, p, pool[s].copy()))  # every source read first
    for b, p, row in moves:
        d = int(region_base[b]) + p
        if 0 <= d < P:
            pool[d] = row
            table[b, p] = d
    return pool, table
