"""The allocation-free entry point verify_attn_forward_static against the
workspace entry points verify_attn_run + verify_attn_reduce.

Both run the same kernels in the same order, so the outputs must agree bit
for bit.  The GPU test calls the static entry several times in a row on one
device (the scratch keeps the previous call's contents), the later calls
with smaller inputs; the host-side checks need no GPU."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import speculative_tree_verify_mla_amd as va
from speculative_tree_verify_mla_amd import binding, inputs

VA_STATIC_SCRATCH_BYTES = 33818624


def _fake(addr):
    return ctypes.c_void_p(addr)


def _static(lib, plan, out=4096, lse=4096, q=4096, sm_scale=0.1):
    return lib.verify_attn_forward_static(ctypes.byref(plan), _fake(q), _fake(8192), 100, 576,
                                          _fake(64), 1000, _fake(64), _fake(64), _fake(64),
                                          sm_scale, _fake(out), _fake(lse), None)


def test_static_entry_refusals_before_any_launch(monkeypatch):
    lib = va.load_library()
    plan = va.verify_attn_plan(8, [100], [4], num_cus=256)
    assert plan.workspace_bytes <= VA_STATIC_SCRATCH_BYTES
    assert _static(lib, plan, out=0) == -1
    assert _static(lib, plan, lse=0) == -1
    assert _static(lib, plan, q=0) == -1
    assert _static(lib, plan, out=4100) == -3
    assert _static(lib, plan, sm_scale=0.0) == -2
    bad = binding.VaPlan()
    ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
    bad.magic = 0
    assert _static(lib, bad) == -5
    # 64 rows x 64 heads = 64 row groups; 9 splits each = 576 work items,
    # more than the scratch holds (with either block size)
    monkeypatch.setenv("VA_NSPLIT", "9")
    for rows in (64, 128):
        big = va.verify_attn_plan(64, [4096], [64], num_cus=256, rows=rows)
        assert big.total_work == 576 and big.workspace_bytes > VA_STATIC_SCRATCH_BYTES
        assert _static(lib, big) == -4
    # the largest plan the scratch holds: 512 work items
    monkeypatch.setenv("VA_NSPLIT", "8")
    edge = va.verify_attn_plan(64, [4096], [64], num_cus=256)
    assert edge.total_work == 512 and edge.workspace_bytes == VA_STATIC_SCRATCH_BYTES


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _bf16(a):
    return _t(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


@pytest.mark.gpu
def test_static_scratch_matches_run_and_reduce_on_calls_in_a_row():
    # the 64-head workload (128-row blocks, 512 work items: the scratch's
    # maximum), the 65k workload (256) and the 4k workload (64): each call
    # leaves the scratch holding its own partials for the next one
    for idx in (4, 3, 2):
        wl = inputs.make_config(idx)
        print(f"static entry: workload {wl.name}", flush=True)
        sys.stdout.flush()
        q, kv = _bf16(wl.q), _bf16(wl.kv_pool)
        tab, ind, pre, par = _t(wl.slot_table), _t(wl.slot_indptr), _t(wl.prefix_len), _t(wl.parent)
        plan = va.verify_attn_plan(wl.num_heads, wl.prefix_len, wl.num_tree)
        assert plan.workspace_bytes <= VA_STATIC_SCRATCH_BYTES
        rows = int(plan.total_tree) * wl.num_heads
        ws = va.workspace_for(plan, "cuda:0")
        out_ref = torch.empty((rows, 512), dtype=torch.bfloat16, device="cuda:0")
        lse_ref = torch.empty(rows, dtype=torch.float32, device="cuda:0")
        va.verify_attn_run(plan, q, kv, tab, ind, pre, par, wl.sm_scale, ws)
        va.verify_attn_reduce(plan, ws, out_ref, lse_ref)
        out = torch.full((rows, 512), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        lse = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda:0")
        va.verify_attn_forward_static(plan, q, kv, tab, ind, pre, par, wl.sm_scale, out, lse)
        torch.cuda.synchronize()
        assert va.verify_attn_read_status(plan, ws) == 0
        assert not torch.isnan(out_ref.float()).any() and not torch.isnan(lse_ref).any()
        assert torch.equal(out.view(torch.int16), out_ref.view(torch.int16)), wl.name
        assert torch.equal(lse.view(torch.int32), lse_ref.view(torch.int32)), wl.name
        del q, kv, ws
