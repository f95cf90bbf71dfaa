"""Pins for the slot-compaction reference (oracle/compact.py)."""
import os

import numpy as np
import pytest

import oracle
from oracle import compact as oc
from speculative_tree_verify_mla_amd import inputs
from conftest import ROOT


def _golden():
    cases, cur = [], None
    for line in open(os.path.join(ROOT, "tests", "golden", "compact.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0], "moves": []}
            cases.append(cur)
        elif key == "move":
            cur["moves"].append((int(vals[0]), int(vals[1])))
        elif key in ("dst", "budget", "expect_copied"):
            cur[key] = int(vals[0])
        else:
            cur[key] = [int(v) for v in vals]
    return cases


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_compactions(case):
    rng = np.random.default_rng(0)
    pool = inputs.normal_bf16(rng, (40, 576))
    t, p, c = oc.compact(case["table"], pool, case["dst"], case["budget"])
    assert c == case["expect_copied"]
    assert t.tolist() == case["expect_table"]
    expect_pool = pool.copy()
    for src, dst in case["moves"]:
        expect_pool[dst] = pool[src]
    np.testing.assert_array_equal(p, expect_pool)


@pytest.mark.parametrize("table_kind", ["runs_mixed", "scattered"])
def test_full_compaction_is_contiguous_and_leaves_attention_unchanged(table_kind):
    """Relocating rows and rewriting the table is a permutation of storage:
    the verify oracle must give the same bits, and the table must end as one
    run."""
    L, T = 600, 12
    wl = inputs.make_workload("cmp", 4, [T], [L], 4096, seed=5, table=table_kind)
    n = L + T
    pool = np.concatenate([wl.kv_pool, np.zeros((n, 576), np.uint16)])
    dst = 4096                                      # the free run appended to the pool
    t2, p2, c = oc.compact(wl.slot_table, pool, dst, n)
    assert c == n and oc.runs(t2) == 1 and oc.runs(wl.slot_table) > 1
    np.testing.assert_array_equal(t2, dst + np.arange(n))
    a = oracle.verify_attn_workload(wl)
    b = oracle.verify_attn(wl.num_heads, wl.num_tree, wl.prefix_len, wl.q, p2, t2,
                           wl.slot_indptr, wl.parent, wl.sm_scale)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_budget_moves_the_first_rows_in_logical_order():
    rng = np.random.default_rng(3)
    pool = inputs.normal_bf16(rng, (400, 576))
    table = rng.permutation(200)[:120].astype(np.int32)
    table[[0, 7, 8]] = [200, 207, 208]             # already in place for dst = 200
    t, p, c = oc.compact(table, pool, 200, 50)
    assert c == 50
    moved = np.flatnonzero(t != table)
    need = np.flatnonzero(table != 200 + np.arange(120))
    np.testing.assert_array_equal(moved, need[:50])
    assert oc.runs(t[:53]) == 1                     # 50 moves (positions 1-6, 9-52) + 3 in place
    assert t[53] == table[53]
    np.testing.assert_array_equal(p[200 + moved], pool[table[moved]])
    untouched = np.setdiff1d(np.arange(400), 200 + moved)
    np.testing.assert_array_equal(p[untouched], pool[untouched])
