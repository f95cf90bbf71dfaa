"""The seeded input generators: reproducible, well-formed, and shaped like
the verify-step workloads (scattered page_size=1 slots, random draft trees)."""
import numpy as np
import pytest
import torch

from speculative_tree_verify_mla_amd import inputs


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, -3.5e-5, 65504.0],
                                 dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(inputs.bf16_bits(x), ref)
    back = inputs.bf16_to_f32(ref)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_seeds_reproduce_bitwise():
    a = inputs.make_workload("a", 2, [5, 3], [40, 7], 512, seed=9, table="interleaved")
    b = inputs.make_workload("a", 2, [5, 3], [40, 7], 512, seed=9, table="interleaved")
    for f in ("q", "kv_pool", "slot_table", "slot_indptr", "parent"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = inputs.make_workload("a", 2, [5, 3], [40, 7], 512, seed=10, table="interleaved")
    assert not np.array_equal(a.kv_pool, c.kv_pool)


@pytest.mark.parametrize("T", [1, 2, 16, 32, 64])
def test_random_tree_is_topological_with_bounded_depth(T):
    rng = np.random.default_rng(T)
    for _ in range(20):
        p = inputs.random_tree(rng, T, max_depth=6)
        assert p[0] == -1
        assert all(-1 <= p[i] < i for i in range(T))
        assert inputs.tree_depths(p).max() <= 6


def test_random_tree_reaches_depth_and_branching():
    rng = np.random.default_rng(1)
    depths, roots = [], []
    for _ in range(50):
        p = inputs.random_tree(rng, 16)
        depths.append(inputs.tree_depths(p).max())
        roots.append((p == -1).sum())
    assert max(depths) >= 4 and max(roots) >= 2


@pytest.mark.parametrize("table", ["permutation", "scattered", "runs_mixed", "contiguous"])
def test_tables_hold_distinct_in_range_slots(table):
    rng = np.random.default_rng(3)
    n_slots, L, T = 4096, 1000, 16
    if table == "permutation":
        t = inputs.table_permutation(rng, n_slots, L + T)
    elif table == "scattered":
        t = inputs.table_scattered(rng, n_slots, L + T)
    elif table == "runs_mixed":
        t = inputs.table_runs_mixed(rng, n_slots, L, T)
    else:
        t = inputs.table_contiguous(5, L + T)
    assert t.shape == (L + T,) and t.dtype == np.int32
    assert len(np.unique(t)) == L + T
    assert t.min() >= 0 and t.max() < n_slots


def test_runs_mixed_has_half_the_prefix_in_runs():
    rng = np.random.default_rng(4)
    L, T = 65536, 16
    t = inputs.table_runs_mixed(rng, 262144, L, T)
    prefix = t[:L]
    step = np.diff(prefix) == 1
    # entries that continue a run of consecutive slots
    frac = step.mean()
    assert 0.40 < frac < 0.52
    assert len(np.unique(t)) == L + T


def test_interleaved_tables_are_disjoint_and_fragmented():
    rng = np.random.default_rng(5)
    lens = [1024 + 32, 16384 + 32, 65536 + 32, 131072 + 32]
    tabs = inputs.tables_interleaved(rng, 524288, lens)
    assert [len(t) for t in tabs] == lens
    allt = np.concatenate(tabs)
    assert len(np.unique(allt)) == len(allt)
    for t in tabs[1:]:
        runs = 1 + (np.diff(t) != 1).sum()
        assert 1.0 < len(t) / runs < 64.0


def test_config_one_shapes():
    wl = inputs.make_config(1)
    assert wl.q.shape == (4, 8, 576) and wl.kv_pool.shape == (1024, 576)
    assert list(wl.parent) == [-1, 0, 1, 2]
    assert wl.num_keys == 260 and wl.kv_bytes() == 260 * 1152
    assert wl.slot_indptr.tolist() == [0, 260]
    assert abs(wl.sm_scale - 1 / np.sqrt(192)) < 1e-15
    v = inputs.bf16_to_f32(wl.kv_pool)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
