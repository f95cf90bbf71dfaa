"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the plan (pure host code) sizes work and workspace as
documented, and argument errors are caught on the host before any launch."""
import ctypes
import os
import re

import numpy as np
import pytest

import speculative_tree_verify_mla_amd as va
from speculative_tree_verify_mla_amd import binding
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "verify_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(verify_attn_\w+)\s*\(", text)))


def test_header_declarations_match_binding_list():
    assert _declared_functions() == sorted(binding.EXPORTS)


def test_library_loads_and_exports_every_declared_symbol():
    lib = va.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.verify_attn_plan_struct_size() == ctypes.sizeof(binding.VaPlan)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        binding.load_library(tmp_path / "nope.so")


def test_error_strings():
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8]:
        s = va.verify_attn_error_string(code)
        assert s and s != "unknown error code"
    assert va.verify_attn_error_string(-99) == "unknown error code"


# --------------------------------------------------------------------------- plan
def _plan(H, L, T, cus=256):
    return va.verify_attn_plan(H, L, T, num_cus=cus)


def test_plan_long_prefix_h8_t16():
    p = _plan(8, [65536], [16])
    assert p.magic == binding.VA_PLAN_MAGIC and p.rows_per_group == 64 and p.tile_keys == 64
    assert p.num_groups[0] == 2                     # 128 rows / 64
    # prefix keys x groups spread over 256 CUs: 2 * 65536 / 256 = 512 keys (8
    # tiles) per work item, 128 splits; the 16 draft keys go with the last
    assert p.nsplit[0] == 128
    assert p.total_work == 256
    assert p.total_tree == 16 and p.total_rows == 128
    o = 256 * 64 * 512 * 2                          # fp16 partial outputs
    assert p.lse_offset == o
    assert p.status_offset == o + 256 * 64 * 8
    assert p.workspace_bytes == o + 256 * 64 * 8 + 1024


def test_plan_full_heads_and_ragged_batch():
    # 16 x 64 = 1024 rows: 128-row blocks, 8 row pairs; 8 * 200000 / 256 =
    # 6250 keys per block, rounded up to 6272 (whole tiles) -> 32 splits of
    # 8 blocks = 256 blocks, 512 work items of 64 rows
    p = _plan(64, [200000], [16])
    assert p.groups_per_block == 2
    assert p.num_groups[0] == 16 and p.nsplit[0] == 32 and p.total_work == 512
    p = va.verify_attn_plan(64, [200000], [16], num_cus=256, rows=64)
    assert p.groups_per_block == 1
    assert p.num_groups[0] == 16 and p.nsplit[0] == 16 and p.total_work == 256
    p = va.verify_attn_plan(16, [1024, 16384, 65536, 131072], [32] * 4, num_cus=256, rows=64)
    assert [p.num_groups[r] for r in range(4)] == [8] * 4
    keys = [1024 + 32, 16384 + 32, 65536 + 32, 131072 + 32]
    per = -(-8 * sum(keys) // 256)
    # the first split length rounds up to [1, 3, 10, 20] = 272 items for 256
    # CUs; splits are lengthened (by max(32, per / 64) keys a step) until the
    # items fit
    while 8 * sum(-(-k // per) for k in keys) > 256:
        per += max(32, per // 64)
    assert p.splits() == [-(-k // per) for k in keys] == [1, 3, 9, 18]
    assert p.work_begin[4] == p.total_work == 8 * sum(p.splits()) == 248
    assert [p.tree_begin[r] for r in range(5)] == [0, 32, 64, 96, 128]
    # by default 128-row blocks: 4 row pairs per request, prefix keys x pairs
    # over 256 CUs = 3344 keys per block, whole tiles 3392 -> [1, 5, 20, 39]
    # = 260 blocks; lengthened to 3456 -> [1, 5, 19, 38] = 252 blocks
    p = _plan(16, [1024, 16384, 65536, 131072], [32] * 4)
    assert p.groups_per_block == 2
    assert p.splits() == [1, 5, 19, 38]
    assert p.work_begin[4] == p.total_work == 8 * sum(p.splits()) == 504


def test_plan_small_inputs_keep_a_minimum_split_length():
    p = _plan(8, [256], [4])
    assert p.num_groups[0] == 1 and p.nsplit[0] == 2      # 256 prefix keys, >= 128 per split
    p = _plan(8, [4096], [16])
    assert p.num_groups[0] == 2 and p.nsplit[0] == 32     # 4096 prefix keys in splits of >= 128
    p = _plan(1, [0], [1])
    assert p.nsplit[0] == 1 and p.total_work == 1 and p.total_rows == 1


def test_plan_split_count_is_capped():
    p = _plan(1, [10_000_000], [1], cus=100000)
    assert p.nsplit[0] == binding.VA_MAX_SPLITS


def test_plan_env_override(monkeypatch):
    monkeypatch.setenv("VA_NSPLIT", "7")
    p = _plan(8, [65536], [16])
    assert p.nsplit[0] == 7 and p.total_work == 14
    monkeypatch.setenv("VA_NSPLIT", "100000")
    p = _plan(8, [100], [16])
    assert p.nsplit[0] == 4                                # capped at ceil(116 / 32) tiles


@pytest.mark.parametrize("H,L,T", [(0, [10], [4]), (8, [10], [0]), (8, [10], [65]),
                                   (8, [-1], [4]), (2000, [10], [4])])
def test_plan_rejects_bad_shapes(H, L, T):
    with pytest.raises(va.VerifyAttnError) as e:
        _plan(H, L, T)
    assert e.value.code == -2


def test_plan_rejects_too_many_requests_and_nulls():
    with pytest.raises(va.VerifyAttnError) as e:
        _plan(8, [10] * 65, [4] * 65)
    assert e.value.code == -2
    lib = va.load_library()
    plan = binding.VaPlan()
    assert lib.verify_attn_plan(1, 8, None, None, 256, ctypes.byref(plan), None) == -1


# --------------------------------------------------------------------------- host-side run checks
def _fake(addr):
    return ctypes.c_void_p(addr)


def _run(lib, plan, q=4096, kv=8192, num_slots=100, stride=576, tab=64, ind=64, pl=64, par=64,
         ws=1 << 20, ws_bytes=None, sm_scale=0.1):
    ws_bytes = plan.workspace_bytes if ws_bytes is None else ws_bytes
    return lib.verify_attn_run(ctypes.byref(plan), _fake(q), _fake(kv), num_slots, stride,
                               _fake(tab), 1000, _fake(ind), _fake(pl), _fake(par), sm_scale,
                               _fake(ws), ws_bytes, None)


def test_run_argument_errors_are_caught_before_launch():
    lib = va.load_library()
    plan = _plan(8, [100], [4])
    assert _run(lib, plan, q=0) == -1
    assert _run(lib, plan, tab=0) == -1
    assert _run(lib, plan, q=4098) == -3                  # misaligned q
    assert _run(lib, plan, kv=8200) == -3                 # misaligned pool
    assert _run(lib, plan, stride=580) == -3              # stride not a multiple of 8
    assert _run(lib, plan, stride=512) == -2              # stride below 576
    assert _run(lib, plan, num_slots=0) == -2
    assert _run(lib, plan, sm_scale=float("nan")) == -2
    assert _run(lib, plan, sm_scale=float("inf")) == -2
    assert _run(lib, plan, sm_scale=0.0) == -2             # masking needs a positive scale
    assert _run(lib, plan, sm_scale=-0.1) == -2
    assert _run(lib, plan, ws=0) == -4
    assert _run(lib, plan, ws=(1 << 20) + 16) == -4       # not 256-byte aligned
    assert _run(lib, plan, ws_bytes=plan.workspace_bytes - 1) == -4
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    bad.magic = 0
    assert _run(lib, bad) == -5
    assert lib.verify_attn_reduce(ctypes.byref(bad), _fake(1 << 20), _fake(4096), _fake(4096),
                                  None) == -5
    assert lib.verify_attn_reduce(ctypes.byref(plan), _fake(1 << 20), _fake(4100), _fake(4096),
                                  None) == -3
    assert lib.verify_attn_gather_rows(_fake(4096), 10, 576, _fake(64), -1, _fake(4096),
                                       None) == -2
    assert lib.verify_attn_gather_rows(_fake(4096), 10, 576, _fake(64), 0, _fake(4096),
                                       None) == 0
    # the read-ceiling helper: checks before any launch; 0 bytes launches nothing
    assert lib.verify_attn_stream_read(None, 1024, _fake(4096), 1, None) == -1
    assert lib.verify_attn_stream_read(_fake(4096), 1024, None, 1, None) == -1
    assert lib.verify_attn_stream_read(_fake(4096), 1000, _fake(4096), 1, None) == -2
    assert lib.verify_attn_stream_read(_fake(4096), -16, _fake(4096), 1, None) == -2
    assert lib.verify_attn_stream_read(_fake(4096), 1024, _fake(4096), 0, None) == -2
    assert lib.verify_attn_stream_read(_fake(4104), 1024, _fake(4096), 1, None) == -3
    assert lib.verify_attn_stream_read(_fake(4096), 0, _fake(4096), 1, None) == 0


@pytest.mark.parametrize("field,value", [("nsplit", 0), ("nsplit", 257), ("num_groups", 2),
                                         ("work_begin", 5), ("num_tree", 65), ("total_work", 2),
                                         ("workspace_bytes", 4096), ("lse_offset", 0),
                                         ("num_heads", 0), ("total_rows", 1)])
def test_tampered_plans_are_rejected_before_launch(field, value):
    """The kernels index through the plan's derived tables; a plan that does
    not satisfy the planner's invariants is refused (no launch, so no GPU)."""
    lib = va.load_library()
    plan = _plan(8, [100], [4])
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    f = getattr(bad, field)
    if isinstance(f, int):
        setattr(bad, field, value)
    else:
        f[1 if field == "work_begin" else 0] = value
    assert _run(lib, bad, ws_bytes=1 << 30) == -5
    assert lib.verify_attn_reduce(ctypes.byref(bad), _fake(1 << 20), _fake(4096), _fake(4096),
                                  None) == -5


@pytest.mark.parametrize("parent,ok", [([-1], True), ([-1, 0, 1, 0, -1], True), ([0], False),
                                       ([-1, 1], False), ([-1, -2], False), ([-1] * 65, False)])
def test_check_tree(parent, ok):
    assert (va.verify_attn_check_tree(parent) == 0) == ok


# --------------------------------------------------------------------------- split-verify plans
def test_plan_ex_without_flags_is_the_fused_plan():
    a = _plan(8, [65536], [16])
    lib = va.load_library()
    b = binding.VaPlan()
    pl = np.array([65536], np.int32)
    nt = np.array([16], np.int32)
    assert lib.verify_attn_plan_ex(1, 8, pl.ctypes.data_as(ctypes.c_void_p),
                                   nt.ctypes.data_as(ctypes.c_void_p), 256, 0,
                                   ctypes.byref(b), None) == 0
    assert bytes(a) == bytes(b)
    assert a.mode == binding.VA_MODE_FUSED and a.version == binding.VA_PLAN_VERSION


def test_plan_split_tree_adds_one_tree_split_per_request():
    p = va.verify_attn_plan(8, [65536], [16], num_cus=256, split_tree=True)
    assert p.mode == binding.VA_MODE_SPLIT_TREE
    # prefix keys x groups over the 254 CUs the 2 tree-block items leave:
    # ceil(2 * 65536 / 254) = 517 keys per prefix split, rounded up to whole
    # tiles (576) -> ceil(65536 / 576) = 114 prefix splits
    assert p.nsplit[0] == 114 + 1
    assert p.total_work == 2 * 115
    o = 2 * 115 * 64 * 512 * 2
    assert p.workspace_bytes == o + 2 * 115 * 64 * 8 + 1024
    q = va.verify_attn_plan(4, [0, 100, 5000], [3, 64, 9], num_cus=256, split_tree=True)
    assert all(ns >= 2 for ns in q.splits())                 # L = 0 keeps one (empty) prefix split
    assert q.work_begin[3] == sum(q.num_groups[r] * q.nsplit[r] for r in range(3))


def test_plan_split_tree_env_override_counts_prefix_splits(monkeypatch):
    monkeypatch.setenv("VA_NSPLIT", "7")
    p = va.verify_attn_plan(8, [65536], [16], num_cus=256, split_tree=True)
    assert p.nsplit[0] == 8


def test_plan_ex_rejects_unknown_flags_and_bad_modes():
    lib = va.load_library()
    b = binding.VaPlan()
    pl = np.array([100], np.int32)
    nt = np.array([4], np.int32)
    assert lib.verify_attn_plan_ex(1, 8, pl.ctypes.data_as(ctypes.c_void_p),
                                   nt.ctypes.data_as(ctypes.c_void_p), 256, 6,
                                   ctypes.byref(b), None) == -2
    plan = _plan(8, [100], [4])
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    bad.mode = 7
    assert _run(lib, bad) == -5
    bad.mode = binding.VA_MODE_SPLIT_TREE           # a split-tree plan needs >= 2 splits
    bad.nsplit[0] = 1
    assert _run(lib, bad) == -5


def test_plan_block_size_rule_and_flags(monkeypatch):
    """128-row blocks for one request in the fused mode with at least two row
    groups when a block's share of the prefix, ceil(groups / 2) * L / CUs,
    is at least 2048 keys; the flags force either size where it applies and
    are refused where it does not."""
    gpb = lambda H, L, T, cus=256: _plan(H, L, T, cus).groups_per_block
    assert gpb(8, [65536], [16]) == 1             # 1 row pair: 256 keys per block
    assert gpb(32, [65536], [16]) == 1            # 4 pairs: 1024
    assert gpb(64, [16384], [16]) == 1            # 8 pairs: 512
    assert gpb(64, [65536], [16]) == 2            # 8 pairs: 2048
    assert gpb(32, [200000], [16]) == 2           # 4 pairs: 3125
    assert gpb(64, [200000], [16]) == 2
    assert gpb(32, [65536], [16], cus=128) == 2   # the same rows on fewer CUs: 2048
    assert gpb(1, [200000], [64]) == 1            # one row group
    assert gpb(64, [200000, 200000], [16, 16]) == 2    # two requests: 2 x 8 pairs x 200000
    assert gpb(64, [200000, 200000], [16, 1]) == 1     # a request with one row group
    assert gpb(16, [1024, 16384, 65536, 131072], [32] * 4) == 2   # 4 x 4 pairs x 214016 keys
    assert va.verify_attn_plan(64, [200000], [16], num_cus=256,
                               split_tree=True).groups_per_block == 1
    monkeypatch.setenv("VA_NSPLIT", "200")        # a forced split count does not decide it
    assert gpb(64, [200000], [16]) == 2 and gpb(64, [16384], [16]) == 1
    monkeypatch.delenv("VA_NSPLIT")
    p = va.verify_attn_plan(8, [65536], [16], num_cus=256, rows=128)
    # one row pair: 65536 / 256 = 256 keys per block -> 256 splits
    assert p.groups_per_block == 2 and p.nsplit[0] == 256 and p.total_work == 512
    assert va.verify_attn_plan(64, [200000], [16], num_cus=256, rows=64).groups_per_block == 1
    lib = va.load_library()
    b = binding.VaPlan()
    p = va.verify_attn_plan(8, [100, 2000], [4, 16], num_cus=256, rows=128)
    assert p.groups_per_block == 2 and p.num_requests == 2
    for B, flags in ((1, binding.VA_PLAN_ROWS64 | binding.VA_PLAN_ROWS128),
                     (1, binding.VA_PLAN_ROWS128 | binding.VA_PLAN_SPLIT_TREE),
                     (2, binding.VA_PLAN_ROWS128 | binding.VA_PLAN_SPLIT_TREE), (1, 8)):
        pl = np.array([100] * B, np.int32)
        nt = np.array([4] * B, np.int32)
        assert lib.verify_attn_plan_ex(B, 8, pl.ctypes.data_as(ctypes.c_void_p),
                                       nt.ctypes.data_as(ctypes.c_void_p), 256, flags,
                                       ctypes.byref(b), None) == -2, (B, flags)


@pytest.mark.parametrize("gpb,B", [(0, 1), (3, 2), (2, 1), (2, 2)])
def test_run_refuses_a_tampered_block_size(gpb, B):
    """groups_per_block is 1, or 2 in the fused mode; any other value, or 2
    in a split-tree plan, is refused before a launch (no GPU)."""
    lib = va.load_library()
    plan = va.verify_attn_plan(8, [100] * B, [4] * B, num_cus=256, split_tree=gpb == 2)
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    bad.groups_per_block = gpb
    assert _run(lib, bad) == -5


@pytest.mark.parametrize("split_tree", [False, True])
def test_plans_fit_the_compute_units(split_tree):
    """Rounded-up split counts must not add up to more work items than CUs
    (the excess would run as a second round of blocks), unless every request
    is already down to one split per row group."""
    rng = np.random.default_rng(7)
    cases = [(16, [1024, 16384, 65536, 131072], [32] * 4, 256), (8, [65536], [16], 256),
             (64, [200000], [16], 256), (8, [4096], [16], 256), (16, [1024, 16384, 65536, 131072], [32] * 4, 80)]
    for _ in range(40):
        B = int(rng.integers(1, 9))
        cases.append((int(rng.integers(1, 65)), [int(x) for x in rng.integers(0, 300000, B)],
                      [int(x) for x in rng.integers(1, 65, B)], int(rng.choice([32, 100, 256, 304]))))
    for H, L, T, cus in cases:
        p = va.verify_attn_plan(H, L, T, num_cus=cus, split_tree=split_tree)
        groups = [(t * H + 63) // 64 for t in T]
        gpb = p.groups_per_block                       # blocks hold 1 or 2 row groups
        blocks = [-(-g // gpb) for g in groups]
        ns = list(p.nsplit[:len(L)])
        prefix_splits = [n - 1 for n in ns] if split_tree else ns
        budget = cus - (sum(groups) if split_tree else 0)
        prefix_items = sum(b * n for b, n in zip(blocks, prefix_splits))
        assert prefix_items <= max(budget, 1) or all(n == 1 for n in prefix_splits), (H, L, T, cus, ns)
        assert p.total_work == sum(g * n for g, n in zip(groups, ns))


@pytest.mark.parametrize("field,value", [("magic", 0), ("tree_begin0", 7), ("tree_size", 3),
                                         ("total_tree", 99)])
def test_build_tree_refuses_tampered_plans_before_launch(field, value):
    """The marshaling kernel indexes the caller's arrays through the plan's
    tree offsets; a plan whose offsets do not start at 0 and step by each
    request's tree size is refused (no launch, so no GPU)."""
    lib = va.load_library()
    plan = _plan(8, [100, 50], [4, 6])
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    if field == "magic":
        bad.magic = value
    elif field == "tree_begin0":
        bad.tree_begin[0] = value
    elif field == "tree_size":
        bad.tree_begin[1] = value   # request 0 would span 3 nodes, not 4
    else:
        bad.total_tree = value
    f = _fake
    assert lib.verify_attn_build_tree(ctypes.byref(bad), f(4096), f(4096), f(4096), f(4096),
                                      f(4096), 100, f(4096), f(4096), f(4096), f(4096), None) == -5
    assert lib.verify_attn_permute_rows(ctypes.byref(bad), f(4096), f(4096), f(8192), 4608,
                                        None) == -5
    assert lib.verify_attn_build_tree_rows(ctypes.byref(bad), f(4096), f(4096), f(4096), f(4096),
                                           f(4096), 100, f(4096), f(4096), f(4096), f(4096),
                                           f(4096), f(8192), 4608, None) == -5


def test_permute_rows_argument_errors_before_launch():
    """verify_attn_permute_rows checks its arguments on the host; every case
    here returns before a launch (so no GPU)."""
    lib = va.load_library()
    plan = _plan(8, [100, 50], [4, 6])
    f = _fake
    p = ctypes.byref(plan)
    assert lib.verify_attn_permute_rows(None, f(4096), f(4096), f(8192), 4608, None) == -1
    assert lib.verify_attn_permute_rows(p, None, f(4096), f(8192), 4608, None) == -1
    assert lib.verify_attn_permute_rows(p, f(4096), None, f(8192), 4608, None) == -1
    assert lib.verify_attn_permute_rows(p, f(4096), f(4096), None, 4608, None) == -1
    assert lib.verify_attn_permute_rows(p, f(4096), f(4096), f(8192), 4607, None) == -2   # not x8
    assert lib.verify_attn_permute_rows(p, f(4096), f(4096), f(8192), 0, None) == -2
    assert lib.verify_attn_permute_rows(p, f(4096), f(4104), f(8192), 4608, None) == -3   # src
    assert lib.verify_attn_permute_rows(p, f(4096), f(4096), f(8200), 4608, None) == -3   # dst


def test_build_tree_rows_argument_errors_before_launch():
    """verify_attn_build_tree_rows checks its arguments on the host; every case
    here returns before a launch (so no GPU)."""
    lib = va.load_library()
    plan = _plan(8, [100, 50], [4, 6])
    f = _fake
    p = ctypes.byref(plan)

    def call(*over):
        args = [p, f(4096), f(4096), f(4096), f(4096), f(4096), 100, f(4096), f(4096), f(4096),
                f(4096), f(4096), f(8192), 4608, None]
        for i, v in over:
            args[i] = v
        return lib.verify_attn_build_tree_rows(*args)

    for i in (0, 1, 2, 3, 4, 5, 7, 8, 9, 10, 11, 12):   # every pointer argument
        assert call((i, None)) == -1, i
    assert call((6, -1)) == -2                  # slot_table_len
    assert call((13, 4607)) == -2               # row_elems not a multiple of 8
    assert call((13, 0)) == -2
    assert call((11, f(4104))) == -3            # src not 16-byte aligned
    assert call((12, f(8200))) == -3            # dst


def test_128_row_block_map_covers_every_work_item_once():
    """The 128-row kernel's block order (XCD-interleaved, then request, split,
    row pair, as va_wide_kernel walks it) restated on the host over random
    plans: every 64-row work item of the plan is written by exactly one
    block, and no block addresses a split or row pair outside its request."""
    rng = np.random.default_rng(11)
    for _ in range(200):
        B = int(rng.integers(1, 65))
        H = int(rng.integers(1, 65))
        T = [int(x) for x in rng.integers(1, 65, B)]
        L = [int(x) for x in rng.integers(0, 300000, B)]
        p = va.verify_attn_plan(H, L, T, num_cus=int(rng.choice([32, 100, 256, 304])), rows=128)
        ns, G = list(p.nsplit[:B]), list(p.num_groups[:B])
        blocks = sum(n * ((g + 1) // 2) for n, g in zip(ns, G))
        per_xcd = (blocks + 7) >> 3
        written = []
        for blk in range(8 * per_xcd):
            it = (blk & 7) * per_xcd + (blk >> 3)
            if it >= blocks:
                continue
            r = 0
            while r + 1 < B and it >= ns[r] * ((G[r] + 1) >> 1):
                it -= ns[r] * ((G[r] + 1) >> 1)
                r += 1
            gw_count = (G[r] + 1) >> 1
            s, gw = divmod(it, gw_count)
            assert s < ns[r]
            written += [p.work_begin[r] + s * G[r] + vg for vg in (2 * gw, 2 * gw + 1) if vg < G[r]]
        assert sorted(written) == list(range(p.total_work))
