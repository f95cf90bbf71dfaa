"""Pins for the draft-tree marshaling reference (oracle/tree.py)."""
import os

import numpy as np
import pytest

import oracle
from oracle import tree as ot
from speculative_tree_verify_mla_amd import inputs
from conftest import ROOT


def _golden():
    cases, cur = [], None
    for line in open(os.path.join(ROOT, "tests", "golden", "marshal.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, rest = line.split(None, 1)
        if key == "tree":
            cur = {"name": rest, "anc": {}}
            cases.append(cur)
        elif key == "anc":
            i, vals = rest.split(":")
            cur["anc"][int(i)] = [int(v) for v in vals.split()]
        else:
            cur[key] = [int(v) for v in rest.split()]
    return cases


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_marshaling(case):
    perm, parent, anc, bits = ot.marshal_one(case["raw_parent"])
    assert bits == 0
    assert perm.tolist() == case["perm"]
    assert parent.tolist() == case["parent"]
    for i, pos in case["anc"].items():
        assert int(anc[i]) == sum(1 << k for k in pos), i


@pytest.mark.parametrize("bad", [[0], [-1, 1], [1, 0], [-1, 5], [2, 0, 1], [-2]])
def test_cycles_and_out_of_range_parents_are_flagged(bad):
    assert ot.marshal_one(bad)[3] & ot.BAD_PARENT


@pytest.mark.parametrize("seed", range(6))
def test_marshaled_tree_attends_like_the_raw_tree(seed):
    """End to end: shuffle a random tree's node numbering, marshal it, run
    the verify oracle on the marshaled inputs, and compare each row with plain
    attention over the raw node's prefix and raw ancestors (oracle.attend,
    computed without any tree mask code)."""
    rng = np.random.default_rng(seed)
    H, T, L = 2, int(rng.integers(1, 33)), int(rng.integers(0, 40))
    wl = inputs.make_workload("mar", H, [T], [L], 512, seed=seed)
    # raw numbering: a random relabeling of the (topological) generated tree
    sigma = rng.permutation(T)                  # raw id of generated node g
    raw_parent = np.empty(T, np.int32)
    raw_slot = np.empty(T, np.int32)
    q_raw = np.empty_like(wl.q)
    for g in range(T):
        pg = wl.parent[g]
        raw_parent[sigma[g]] = -1 if pg == -1 else sigma[pg]
        raw_slot[sigma[g]] = wl.slot_table[L + g]
        q_raw[sigma[g]] = wl.q[g]
    table = wl.slot_table.copy()
    table[L:] = -7                               # draft entries come from the marshaling
    perm, parent, anc, status, table2 = ot.marshal([T], raw_parent, raw_slot, [L], [0, L + T],
                                                   table)
    assert status[0] == 0 and np.all(parent < np.arange(T))
    out, lse = oracle.verify_attn(H, [T], [L], q_raw[perm], wl.kv_pool, table2, wl.slot_indptr,
                                  parent, wl.sm_scale)
    kv = inputs.bf16_to_f32(wl.kv_pool).astype(np.float64)
    for i in range(T):
        j = perm[i]
        chain, x = [], j
        while x != -1:
            chain.append(raw_slot[x])
            x = raw_parent[x]
        slots = np.concatenate([wl.slot_table[:L], np.array(chain, np.int32)])
        for h in range(H):
            o, l, _ = oracle.attend(inputs.bf16_to_f32(q_raw[j, h]), wl.kv_pool, slots,
                                    wl.sm_scale)
            np.testing.assert_allclose(out[i, h], o, rtol=0, atol=1e-12)
            assert abs(lse[i, h] - l) <= 1e-12
        m = int(anc[i])
        assert bin(m).count("1") == len(chain)


def test_draft_entries_stay_inside_the_request_range():
    """Each request's draft entries go to slot_indptr[r] + prefix_len[r] + i
    only while that index lies in [slot_indptr[r], slot_indptr[r+1]): a
    negative prefix length of request 1 flags it and leaves request 0's
    range exactly as a valid batch leaves it."""
    num_tree = [3, 4]
    raw_parent = np.array([-1, 0, 0, -1, 0, 1, 1], np.int32)
    raw_slot = np.arange(7, dtype=np.int32) + 500
    indptr = [0, 10, 20]
    table = np.arange(20, dtype=np.int32)
    ok = ot.marshal(num_tree, raw_parent, raw_slot, [7, 6], indptr, table)
    bad = ot.marshal(num_tree, raw_parent, raw_slot, [7, -2], indptr, table)
    assert ok[3].tolist() == [0, 0]
    assert bad[3][0] == 0 and bad[3][1] & ot.BAD_TABLE
    # request 0: prefix 0..6 untouched, its drafts at 7..9 in breadth-first order
    assert bad[4][:10].tolist() == list(range(7)) + [500, 501, 502]
    np.testing.assert_array_equal(bad[4][:10], ok[4][:10])
    # request 1: entry 10 + (-2) + i is inside its range for i >= 2 only
    assert bad[4][10:12].tolist() == [505, 506]
    assert bad[4][12:].tolist() == list(range(12, 20))
