"""Plain reference of draft-tree marshaling (verify order, parent array,
ancestor masks, draft slot entries).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The verify step needs the draft nodes of a request in an order where parents
come first, the tree mask, and the draft tokens' slots after the prefix in
the slot table ("The Execution Phase: From Plan to 3-6x Decode Speedup on
Blackwell Consumer GPUs", section "The Methodology: Evidence-Driven
Engineering", where these are built on the host as tree build and mask
build).  Written out step by step: each node's depth is the length of its
parent chain; the verify order sorts nodes by (depth, raw index); a node's
mask holds itself and every node on its parent chain.
"""
from __future__ import annotations

import numpy as np

BAD_PARENT = 1
BAD_TABLE = 2


def marshal_one(raw_parent):
    """One request: returns (perm, parent, anc, bits)."""
    T = len(raw_parent)
    depth = [0] * T
    bits = 0
    for j in range(T):
        x, d, ok = int(raw_parent[j]), 0, True
        while x != -1:
            if x < -1 or x >= T or d > T:
                ok = False
                break
            d += 1
            x = int(raw_parent[x])
        if not ok or d > T:
            bits |= BAD_PARENT
        depth[j] = d
    order = sorted(range(T), key=lambda j: (depth[j], j))
    pos = {j: i for i, j in enumerate(order)}
    perm = np.array(order, dtype=np.int32)
    parent = np.array([-1 if raw_parent[j] == -1 else pos[int(raw_parent[j])] for j in order]
                      if not bits else [-1] * T, dtype=np.int32)
    anc = np.zeros(T, dtype=np.uint64)
    if not bits:
        for i, j in enumerate(order):
            m, x = 0, j
            while x != -1:
                m |= 1 << pos[x]
                x = int(raw_parent[x])
            anc[i] = m
    return perm, parent, anc, bits


def marshal(num_tree, raw_parent, raw_slot, prefix_len, slot_indptr, slot_table):
    """All requests.  Returns (perm, parent, anc, status, new_table)."""
    table = np.array(slot_table, dtype=np.int32, copy=True)
    perm_all, parent_all, anc_all, status = [], [], [], []
    t0 = 0
    for r, T in enumerate(num_tree):
        rp = list(raw_parent[t0:t0 + T])
        perm, parent, anc, bits = marshal_one(rp)
        for i in range(T):
            e = int(slot_indptr[r]) + int(prefix_len[r]) + i
            # only inside the request's own range [slot_indptr[r], slot_indptr[r+1])
            if max(0, int(slot_indptr[r])) <= e < min(len(table), int(slot_indptr[r + 1])):
                table[e] = raw_slot[t0 + perm[i]]
            else:
                bits |= BAD_TABLE
        perm_all.append(perm)
        parent_all.append(parent)
        anc_all.append(anc)
        status.append(bits)
        t0 += T
    return (np.concatenate(perm_all), np.concatenate(parent_all), np.concatenate(anc_all),
            np.array(status, dtype=np.uint32), table)
