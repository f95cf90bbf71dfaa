"""Seeded random shapes against the CPU fp64 oracle, fused and split-verify.

Each case draws the batch size, head count, tree sizes and shapes, prefix
lengths (0 and values at tile and split edges included) and the slot-table
layout from one seed, runs the HIP path through the C ABI and compares every
output row with the oracle (max abs error 1e-2 beyond the bf16 rounding of
the exact value, 1e-3 on the LSE)."""
import numpy as np
import pytest

from speculative_tree_verify_mla_amd import inputs
from test_parity import check, run_gpu, say
from test_split_verify import run_split

pytestmark = pytest.mark.gpu

EDGE_L = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 575, 576, 577, 1023, 1024]


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 5))
    H = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 32]))
    max_rows = 512
    T = []
    for _ in range(B):
        t_hi = max(1, min(64, max_rows // (H * B)))
        T.append(int(rng.integers(1, t_hi + 1)))
    L = [int(rng.choice(EDGE_L)) if rng.random() < 0.4 else int(rng.integers(0, 3000))
         for _ in range(B)]
    tree = str(rng.choice(["random", "chain", "star"]))
    table = str(rng.choice(["scattered", "interleaved", "contiguous"]))
    slots = int(2 * (sum(L) + sum(T)) + 64)
    wl = inputs.make_workload(f"rand{seed}", H, T, L, slots, seed=seed, tree=tree, table=table,
                              max_depth=int(rng.integers(1, 9)))
    return wl, dict(B=B, H=H, T=T, L=L, tree=tree, table=table)


@pytest.mark.parametrize("seed", range(16))
def test_random_shape_matches_the_oracle(seed):
    wl, desc = random_case(seed)
    say(f"random case {seed}: {desc}")
    out, lse, status, plan = run_gpu(wl)
    assert status == 0
    check(wl, out, lse, what=f"fused nsplit={plan.splits()}")


@pytest.mark.parametrize("seed", range(16, 24))
def test_random_shape_split_verify_matches_the_oracle(seed):
    wl, desc = random_case(seed)
    say(f"random case {seed} (split-verify): {desc}")
    out, lse, status, plan = run_split(wl)
    assert status == 0
    check(wl, out, lse, what=f"split nsplit={plan.splits()}")
