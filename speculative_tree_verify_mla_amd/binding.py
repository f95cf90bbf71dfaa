"""Thin ctypes binding of libverify_attn.so (argument marshalling only).

Every step of the verify path runs in the HIP library; this module turns
torch tensors into device pointers and the current torch stream into a
hipStream_t.  The names mirror the C ABI declared in include/verify_attn.h.
If the library has not been built the import-time loader raises: there is
no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

PKG_DIR = Path(__file__).resolve().parent
LIB_PATH = PKG_DIR / "libverify_attn.so"

VA_D_QK = 576
VA_D_V = 512
VA_MAX_TREE = 64
VA_MAX_REQUESTS = 64
VA_MAX_SPLITS = 256
VA_PLAN_MAGIC = 0x56415054
VA_PLAN_VERSION = 3
VA_MODE_FUSED = 0
VA_MODE_SPLIT_TREE = 1
VA_PLAN_SPLIT_TREE = 1
VA_PLAN_ROWS64 = 2
VA_PLAN_ROWS128 = 4

VA_OK = 0
ERRORS = {
    -1: "VA_ERR_NULL", -2: "VA_ERR_SHAPE", -3: "VA_ERR_ALIGN", -4: "VA_ERR_WORKSPACE",
    -5: "VA_ERR_PLAN", -6: "VA_ERR_HIP", -7: "VA_ERR_TREE", -8: "VA_ERR_DEVICE_DATA",
}
STATUS_BITS = {1: "BAD_PREFIX", 2: "SHORT_TABLE", 4: "BAD_SLOT", 8: "BAD_PARENT"}

# Every symbol include/verify_attn.h declares.
EXPORTS = (
    "verify_attn_plan", "verify_attn_plan_ex", "verify_attn_run", "verify_attn_reduce",
    "verify_attn_forward_static", "verify_attn_read_status",
    "verify_attn_check_tree", "verify_attn_gather_rows", "verify_attn_stream_read",
    "verify_attn_error_string",
    "verify_attn_plan_struct_size", "verify_attn_compact_workspace_bytes", "verify_attn_compact",
    "verify_attn_build_tree", "verify_attn_permute_rows", "verify_attn_build_tree_rows",
)
TREE_BITS = {1: "BAD_PARENT", 2: "BAD_TABLE"}
COMPACT_BITS = {1: "BAD_SLOT", 2: "RUN_OCCUPIED"}


class VaPlan(ctypes.Structure):
    """Mirror of struct va_plan."""
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("num_requests", ctypes.c_int32), ("num_heads", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int32), ("tile_keys", ctypes.c_int32),
        ("total_work", ctypes.c_int32), ("total_tree", ctypes.c_int32),
        ("total_rows", ctypes.c_int32), ("num_cus", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("groups_per_block", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64), ("lse_offset", ctypes.c_int64),
        ("status_offset", ctypes.c_int64),
        ("num_tree", ctypes.c_int32 * VA_MAX_REQUESTS),
        ("max_prefix", ctypes.c_int32 * VA_MAX_REQUESTS),
        ("nsplit", ctypes.c_int32 * VA_MAX_REQUESTS),
        ("num_groups", ctypes.c_int32 * VA_MAX_REQUESTS),
        ("tree_begin", ctypes.c_int32 * (VA_MAX_REQUESTS + 1)),
        ("work_begin", ctypes.c_int32 * (VA_MAX_REQUESTS + 1)),
    ]

    def splits(self):
        return [int(self.nsplit[r]) for r in range(self.num_requests)]


class VerifyAttnError(RuntimeError):
    def __init__(self, where, code, msg=""):
        super().__init__(f"{where}: {ERRORS.get(code, code)} ({code}) {msg}".strip())
        self.code = code


_lib = None


def load_library(path: os.PathLike | None = None):
    """Load libverify_attn.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"HIP library {p} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(str(p))
    P = ctypes.c_void_p
    i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.verify_attn_plan.argtypes = [i32, i32, P, P, i32, ctypes.POINTER(VaPlan),
                                     ctypes.POINTER(sz)]
    lib.verify_attn_plan_ex.argtypes = [i32, i32, P, P, i32, ctypes.c_uint32,
                                        ctypes.POINTER(VaPlan), ctypes.POINTER(sz)]
    lib.verify_attn_run.argtypes = [ctypes.POINTER(VaPlan), P, P, i64, i32, P, i32, P, P, P, f32,
                                    P, sz, P]
    lib.verify_attn_reduce.argtypes = [ctypes.POINTER(VaPlan), P, P, P, P]
    lib.verify_attn_forward_static.argtypes = [ctypes.POINTER(VaPlan), P, P, i64, i32, P, i32, P,
                                               P, P, f32, P, P, P]
    lib.verify_attn_read_status.argtypes = [ctypes.POINTER(VaPlan), P, P,
                                            ctypes.POINTER(ctypes.c_uint32)]
    lib.verify_attn_check_tree.argtypes = [P, i32]
    lib.verify_attn_gather_rows.argtypes = [P, i64, i32, P, i32, P, P]
    lib.verify_attn_stream_read.argtypes = [P, i64, P, i32, P]
    lib.verify_attn_error_string.argtypes = [ctypes.c_int]
    lib.verify_attn_error_string.restype = ctypes.c_char_p
    lib.verify_attn_compact_workspace_bytes.argtypes = [i32, i32]
    lib.verify_attn_compact_workspace_bytes.restype = sz
    lib.verify_attn_compact.argtypes = [P, i64, i32, P, i32, i32, i32, P, sz, P, P]
    lib.verify_attn_compact.restype = ctypes.c_int
    lib.verify_attn_build_tree.argtypes = [ctypes.POINTER(VaPlan), P, P, P, P, P, i32, P, P, P, P, P]
    lib.verify_attn_build_tree.restype = ctypes.c_int
    lib.verify_attn_permute_rows.argtypes = [ctypes.POINTER(VaPlan), P, P, P, i64, P]
    lib.verify_attn_permute_rows.restype = ctypes.c_int
    lib.verify_attn_build_tree_rows.argtypes = [ctypes.POINTER(VaPlan), P, P, P, P, P, i32, P, P, P,
                                                P, P, P, i64, P]
    lib.verify_attn_build_tree_rows.restype = ctypes.c_int
    lib.verify_attn_plan_struct_size.argtypes = []
    lib.verify_attn_plan_struct_size.restype = sz
    for name in ("verify_attn_plan", "verify_attn_plan_ex", "verify_attn_run", "verify_attn_reduce",
                 "verify_attn_forward_static", "verify_attn_read_status", "verify_attn_check_tree", "verify_attn_gather_rows",
                 "verify_attn_stream_read"):
        getattr(lib, name).restype = ctypes.c_int
    if lib.verify_attn_plan_struct_size() != ctypes.sizeof(VaPlan):
        raise RuntimeError("va_plan layout mismatch between library and binding")
    if path is None:
        _lib = lib
    return lib


def _check(where, rc):
    if rc != VA_OK:
        msg = load_library().verify_attn_error_string(rc).decode()
        raise VerifyAttnError(where, rc, msg)


def _i32_host(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32).reshape(-1))


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dptr(t, dtypes, name):
    """Device pointer of a contiguous CUDA tensor with one of `dtypes`."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


# --------------------------------------------------------------------------- C ABI mirrors
def verify_attn_plan(num_heads, prefix_len, num_tree, num_cus=0, split_tree=False,
                     rows=None) -> VaPlan:
    """Host-only plan.  prefix_len / num_tree: per-request host sequences.
    split_tree=True plans the split-verify decomposition (VA_PLAN_SPLIT_TREE);
    rows=64 or 128 fixes the partial pass's block size (VA_PLAN_ROWS64 /
    VA_PLAN_ROWS128), rows=None leaves it to the planner.  Without flags this
    is verify_attn_plan, otherwise verify_attn_plan_ex."""
    pl = _i32_host(prefix_len)
    nt = _i32_host(num_tree)
    if pl.shape != nt.shape:
        raise ValueError("prefix_len and num_tree must have one entry per request")
    plan = VaPlan()
    ws = ctypes.c_size_t(0)
    args = (int(nt.shape[0]), int(num_heads), pl.ctypes.data_as(ctypes.c_void_p),
            nt.ctypes.data_as(ctypes.c_void_p), int(num_cus))
    flags = VA_PLAN_SPLIT_TREE if split_tree else 0
    if rows is not None:
        if rows not in (64, 128):
            raise ValueError("rows must be None, 64 or 128")
        flags |= VA_PLAN_ROWS64 if rows == 64 else VA_PLAN_ROWS128
    lib = load_library()
    if flags:
        rc = lib.verify_attn_plan_ex(*args, flags, ctypes.byref(plan), ctypes.byref(ws))
        _check("verify_attn_plan_ex", rc)
    else:
        rc = lib.verify_attn_plan(*args, ctypes.byref(plan), ctypes.byref(ws))
        _check("verify_attn_plan", rc)
    return plan


def _check_run_tensors(plan, q, kv_pool, slot_indptr, prefix_len, parent):
    B = int(plan.num_requests)
    if tuple(q.shape) != (int(plan.total_tree), int(plan.num_heads), VA_D_QK):
        raise ValueError(f"q must be [{plan.total_tree}, {plan.num_heads}, 576], got {tuple(q.shape)}")
    if kv_pool.dim() != 2 or kv_pool.shape[1] < VA_D_QK:
        raise ValueError("kv_pool must be [num_slots, >=576]")
    if kv_pool.stride(1) != 1:
        raise ValueError("kv_pool rows must be contiguous")
    if not kv_pool.is_cuda or kv_pool.dtype not in _bf16_types():
        raise TypeError("kv_pool must be a bf16 device tensor")
    if slot_indptr.numel() < B + 1 or prefix_len.numel() < B or parent.numel() < plan.total_tree:
        raise ValueError("slot_indptr / prefix_len / parent are shorter than the plan needs")


def verify_attn_run(plan, q, kv_pool, slot_table, slot_indptr, prefix_len, parent, sm_scale,
                    workspace, stream=None):
    """Enqueue the partial pass.  Tensors: q/kv_pool bf16 (or 16-bit ints),
    tables int32, workspace uint8 of at least plan.workspace_bytes."""
    import torch
    b16 = _bf16_types()
    i32 = (torch.int32,)
    _check_run_tensors(plan, q, kv_pool, slot_indptr, prefix_len, parent)
    kv_ptr = ctypes.c_void_p(kv_pool.data_ptr())
    rc = load_library().verify_attn_run(
        ctypes.byref(plan), _dptr(q, b16, "q"), kv_ptr, int(kv_pool.shape[0]),
        int(kv_pool.stride(0)), _dptr(slot_table, i32, "slot_table"), int(slot_table.numel()),
        _dptr(slot_indptr, i32, "slot_indptr"), _dptr(prefix_len, i32, "prefix_len"),
        _dptr(parent, i32, "parent"), float(sm_scale),
        _dptr(workspace, (torch.uint8, torch.int8, torch.float32, torch.int32), "workspace"),
        int(workspace.numel() * workspace.element_size()), _stream_handle(stream))
    _check("verify_attn_run", rc)


def verify_attn_reduce(plan, workspace, out, lse, stream=None):
    import torch
    rows = int(plan.total_tree) * int(plan.num_heads)
    if out.numel() != rows * VA_D_V or lse.numel() != rows:
        raise ValueError(f"out must hold {rows}x512 and lse {rows} elements")
    rc = load_library().verify_attn_reduce(
        ctypes.byref(plan),
        _dptr(workspace, (torch.uint8, torch.int8, torch.float32, torch.int32), "workspace"),
        _dptr(out, _bf16_types(), "out"), _dptr(lse, (torch.float32,), "lse"),
        _stream_handle(stream))
    _check("verify_attn_reduce", rc)


def verify_attn_forward_static(plan, q, kv_pool, slot_table, slot_indptr, prefix_len, parent,
                               sm_scale, out, lse, stream=None):
    """Partial pass and merge in one call, with the partials in the library's
    per-device scratch (no workspace, nothing allocated).  Arguments as
    verify_attn_run and verify_attn_reduce."""
    import torch
    b16 = _bf16_types()
    i32 = (torch.int32,)
    _check_run_tensors(plan, q, kv_pool, slot_indptr, prefix_len, parent)
    rows = int(plan.total_tree) * int(plan.num_heads)
    if out.numel() != rows * VA_D_V or lse.numel() != rows:
        raise ValueError(f"out must hold {rows}x512 and lse {rows} elements")
    rc = load_library().verify_attn_forward_static(
        ctypes.byref(plan), _dptr(q, b16, "q"), ctypes.c_void_p(kv_pool.data_ptr()),
        int(kv_pool.shape[0]), int(kv_pool.stride(0)), _dptr(slot_table, i32, "slot_table"),
        int(slot_table.numel()), _dptr(slot_indptr, i32, "slot_indptr"),
        _dptr(prefix_len, i32, "prefix_len"), _dptr(parent, i32, "parent"), float(sm_scale),
        _dptr(out, b16, "out"), _dptr(lse, (torch.float32,), "lse"), _stream_handle(stream))
    _check("verify_attn_forward_static", rc)


def verify_attn_read_status(plan, workspace, stream=None) -> int:
    import torch
    st = ctypes.c_uint32(0)
    rc = load_library().verify_attn_read_status(
        ctypes.byref(plan),
        _dptr(workspace, (torch.uint8, torch.int8, torch.float32, torch.int32), "workspace"),
        _stream_handle(stream), ctypes.byref(st))
    _check("verify_attn_read_status", rc)
    return int(st.value)


def verify_attn_check_tree(parent) -> int:
    p = _i32_host(parent)
    return int(load_library().verify_attn_check_tree(p.ctypes.data_as(ctypes.c_void_p),
                                                     int(p.shape[0])))


def verify_attn_gather_rows(kv_pool, slot_table, n, dst, stream=None):
    import torch
    if slot_table.numel() < n or dst.numel() < n * VA_D_QK:
        raise ValueError("slot_table / dst are shorter than n rows")
    rc = load_library().verify_attn_gather_rows(
        _dptr(kv_pool, _bf16_types(), "kv_pool"), int(kv_pool.shape[0]), int(kv_pool.stride(0)),
        _dptr(slot_table, (torch.int32,), "slot_table"), int(n),
        _dptr(dst, _bf16_types(), "dst"), _stream_handle(stream))
    _check("verify_attn_gather_rows", rc)


def verify_attn_stream_read(buf, sink, stream=None):
    """Read every byte of the device tensor `buf` once (the read-ceiling
    helper); the XOR of all words of the int32 device tensor `sink`
    (initialised by the caller; 4096 words keep blocks from sharing one)
    becomes the XOR of buf's 32-bit words."""
    import torch
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink.numel() < 1 or sink.dtype != torch.int32 or not sink.is_cuda:
        raise ValueError("sink must be a device int32 tensor")
    nbytes = buf.numel() * buf.element_size()
    rc = load_library().verify_attn_stream_read(ctypes.c_void_p(buf.data_ptr()), int(nbytes),
                                                ctypes.c_void_p(sink.data_ptr()), int(sink.numel()),
                                                _stream_handle(stream))
    _check("verify_attn_stream_read", rc)


def verify_attn_error_string(code) -> str:
    return load_library().verify_attn_error_string(int(code)).decode()


def verify_attn_compact(kv_pool, slot_table, dst_begin, budget, workspace=None, copied=None,
                        stream=None):
    """Enqueue the compaction of one request's slot table (rewritten in place)
    into the run [dst_begin, dst_begin + n) of kv_pool, copying at most
    `budget` rows.  Returns the device int32 tensor [1] of rows copied (or
    minus the VA_COMPACT_* bits of a failed precondition)."""
    import torch
    if kv_pool.dim() != 2 or kv_pool.shape[1] < VA_D_QK or kv_pool.stride(1) != 1:
        raise ValueError("kv_pool must be [num_slots, >=576] with unit column stride")
    if not kv_pool.is_cuda or kv_pool.dtype not in _bf16_types():
        raise TypeError("kv_pool must be a bf16 (or 16-bit integer) device tensor")
    if slot_table.dim() != 1:
        raise ValueError("slot_table must be one request's [n] table")
    n = int(slot_table.numel())
    lib = load_library()
    if workspace is None:
        workspace = torch.empty(int(lib.verify_attn_compact_workspace_bytes(n, int(budget))),
                                dtype=torch.uint8, device=kv_pool.device)
    if copied is None:
        copied = torch.empty(1, dtype=torch.int32, device=kv_pool.device)
    rc = lib.verify_attn_compact(
        ctypes.c_void_p(kv_pool.data_ptr()),
        int(kv_pool.shape[0]), int(kv_pool.stride(0)),
        _dptr(slot_table, (torch.int32,), "slot_table"), n, int(dst_begin), int(budget),
        _dptr(workspace, (torch.uint8,), "workspace"), int(workspace.numel()),
        _dptr(copied, (torch.int32,), "copied"), _stream_handle(stream))
    _check("verify_attn_compact", rc)
    return copied


def verify_attn_build_tree(plan, raw_parent, raw_slot, prefix_len, slot_indptr, slot_table,
                           stream=None):
    """Enqueue the device marshaling of raw draft trees (any node order) into
    verify order.  Writes the draft entries of slot_table in place; returns
    device tensors (perm int32, parent int32, anc int64 bit masks, status
    uint32 per request -- stored as int32)."""
    import torch
    dev = raw_parent.device
    n = int(plan.total_tree)
    if raw_parent.numel() != n or raw_slot.numel() != n:
        raise ValueError("raw_parent and raw_slot need sum(T_r) entries")
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    parent = torch.empty(n, dtype=torch.int32, device=dev)
    anc = torch.empty(n, dtype=torch.int64, device=dev)
    status = torch.empty(int(plan.num_requests), dtype=torch.int32, device=dev)
    i32 = (torch.int32,)
    rc = load_library().verify_attn_build_tree(
        ctypes.byref(plan), _dptr(raw_parent, i32, "raw_parent"), _dptr(raw_slot, i32, "raw_slot"),
        _dptr(prefix_len, i32, "prefix_len"), _dptr(slot_indptr, i32, "slot_indptr"),
        _dptr(slot_table, i32, "slot_table"), int(slot_table.numel()),
        _dptr(perm, i32, "perm"), _dptr(parent, i32, "parent"),
        _dptr(anc, (torch.int64,), "anc"), _dptr(status, i32, "status"), _stream_handle(stream))
    _check("verify_attn_build_tree", rc)
    return perm, parent, anc, status


def verify_attn_permute_rows(plan, perm, src, dst=None, stream=None):
    """Enqueue the gather of per-node rows from raw node order into verify
    order (dst[t0 + i] = src[t0 + perm[t0 + i]] per request).  src: [sum T_r,
    ...] bf16 (for q: [sum T_r, H, 576]); dst: same shape (allocated if None).
    Returns dst."""
    import torch
    n = int(plan.total_tree)
    if src.shape[0] != n or perm.numel() != n:
        raise ValueError("src and perm need sum(T_r) rows")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.shape != src.shape:
        raise ValueError("dst must have the shape of src")
    b16 = _bf16_types()
    rc = load_library().verify_attn_permute_rows(
        ctypes.byref(plan), _dptr(perm, (torch.int32,), "perm"), _dptr(src, b16, "src"),
        _dptr(dst, b16, "dst"), int(src.numel() // n), _stream_handle(stream))
    _check("verify_attn_permute_rows", rc)
    return dst


def verify_attn_build_tree_rows(plan, raw_parent, raw_slot, prefix_len, slot_indptr, slot_table,
                                src, dst=None, stream=None):
    """verify_attn_build_tree and verify_attn_permute_rows in one launch:
    returns (perm, parent, anc, status, dst) as those two calls would."""
    import torch
    dev = raw_parent.device
    n = int(plan.total_tree)
    if raw_parent.numel() != n or raw_slot.numel() != n:
        raise ValueError("raw_parent and raw_slot need sum(T_r) entries")
    if src.shape[0] != n:
        raise ValueError("src needs sum(T_r) rows")
    if dst is None:
        dst = torch.empty_like(src)
    if dst.shape != src.shape:
        raise ValueError("dst must have the shape of src")
    perm = torch.empty(n, dtype=torch.int32, device=dev)
    parent = torch.empty(n, dtype=torch.int32, device=dev)
    anc = torch.empty(n, dtype=torch.int64, device=dev)
    status = torch.empty(int(plan.num_requests), dtype=torch.int32, device=dev)
    i32 = (torch.int32,)
    b16 = _bf16_types()
    rc = load_library().verify_attn_build_tree_rows(
        ctypes.byref(plan), _dptr(raw_parent, i32, "raw_parent"), _dptr(raw_slot, i32, "raw_slot"),
        _dptr(prefix_len, i32, "prefix_len"), _dptr(slot_indptr, i32, "slot_indptr"),
        _dptr(slot_table, i32, "slot_table"), int(slot_table.numel()),
        _dptr(perm, i32, "perm"), _dptr(parent, i32, "parent"),
        _dptr(anc, (torch.int64,), "anc"), _dptr(status, i32, "status"),
        _dptr(src, b16, "src"), _dptr(dst, b16, "dst"), int(src.numel() // n),
        _stream_handle(stream))
    _check("verify_attn_build_tree_rows", rc)
    return perm, parent, anc, status, dst


# --------------------------------------------------------------------------- convenience
def workspace_for(plan, device="cuda"):
    import torch
    return torch.empty(int(plan.workspace_bytes), dtype=torch.uint8, device=device)


def verify_attn(q, kv_pool, slot_table, slot_indptr, prefix_len, parent, sm_scale, *,
                num_tree, prefix_len_host, plan=None, workspace=None, out=None, lse=None,
                stream=None, split_tree=False):
    """plan (if not given) + run + reduce.  Returns (out [sumT,H,512] bf16, lse [sumT,H] fp32).

    num_tree / prefix_len_host: host sequences per request (prefix_len_host is
    the planned bound; prefix_len is the device tensor the kernel reads)."""
    import torch
    H = int(q.shape[1])
    if plan is None:
        plan = verify_attn_plan(H, prefix_len_host, num_tree, split_tree=split_tree)
    if workspace is None:
        workspace = workspace_for(plan, q.device)
    total_tree = int(plan.total_tree)
    if out is None:
        out = torch.empty((total_tree, H, VA_D_V), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((total_tree, H), dtype=torch.float32, device=q.device)
    verify_attn_run(plan, q, kv_pool, slot_table, slot_indptr, prefix_len, parent, sm_scale,
                    workspace, stream)
    verify_attn_reduce(plan, workspace, out, lse, stream)
    return out, lse
