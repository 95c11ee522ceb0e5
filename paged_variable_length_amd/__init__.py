"""Paged, variable-length attention for MI355X (gfx950): Python binding of libpagedattn.so.

The functions here carry the names of the C ABI (include/pagedattn.h) and only marshal
arguments: torch tensors are used for device memory and streams, every step of the path runs
in the library's HIP kernels or its host C++. Nothing here computes attention, and nothing
falls back to a CPU path: a missing library raises.

    pack_seqlens             per-sequence lengths -> cu_seqlens (host)
    build_task_table         Dynamic Decomposer: load-sorted task table (host)
    workspace_bytes          bytes of the split-partial workspace
    reshape_and_cache        write new K/V rows into their pages (device)
    paged_attn_decode        decode attention, one query token per sequence (device)
    paged_attn_varlen_prefill  packed causal attention, any mix of decode and prefill (device)
    paged_attn_varlen_prefill_noalloc  the same with partial rows in the library's own scratch
    validate_block_table     debug check of a host block table
    StepPlan                 convenience: a built table copied to the device with its workspace
    build_gemm_table         SmoothGEMM's Linear decomposition: load-sorted tile tasks (host)
    gemm_workspace_bytes     bytes of SmoothGEMM's partial tiles
    smooth_gemm              C = A W^T for arbitrary M, N, K from a task table (device)
    GemmPlan                 convenience: a built SmoothGEMM table on the device
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _abi
from ._abi import (PA_BF16, PA_FP32, PA_TASK_DECODE, PA_TASK_PREFILL,  # noqa: F401
                   PA_TASK_VERIFY, PA_TASK_SHARED, PagedAttnError, PaCombine, PaGemmParams,
                   PaGemmReduce, PaGemmTask, PaParams, PaTask, check, lib)

__all__ = ["pack_seqlens", "build_task_table", "workspace_bytes", "reshape_and_cache",
           "paged_attn_decode", "paged_attn_varlen_prefill", "paged_attn_varlen_prefill_noalloc",
           "validate_block_table",
           "reshape_and_cache_fp8", "paged_attn_decode_fp8", "paged_attn_verify_fp8",
           "paged_attn_varlen_prefill_fp8",
           "TaskTable", "StepPlan", "make_params", "PagedAttnError", "PA_BF16", "PA_FP32",
           "build_gemm_table", "gemm_workspace_bytes", "smooth_gemm", "GemmTable", "GemmPlan"]

_I32P = ctypes.POINTER(ctypes.c_int32)


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_I32P)


def pack_seqlens(lengths) -> np.ndarray:
    """Host lengths [n] -> cu_seqlens int32 [n+1] (library call)."""
    ln = _i32(lengths)
    cu = np.zeros(ln.shape[0] + 1, dtype=np.int32)
    check(lib().pa_pack_seqlens(_ptr(ln), ln.shape[0], _ptr(cu)), "pa_pack_seqlens")
    return cu


def make_params(num_q_heads, num_kv_heads, head_dim, block_size, dec_split=512, pf_q_tile=128,
                pf_kv_split=0, num_workers=256, decode_weight=1, verify_rows=0,
                shared_min=0) -> PaParams:
    return PaParams(num_q_heads, num_kv_heads, head_dim, block_size, dec_split, pf_q_tile,
                    pf_kv_split, num_workers, decode_weight, verify_rows, shared_min, 0)


@dataclass
class TaskTable:
    tasks: np.ndarray        # int32 [n, 8]
    combines: np.ndarray     # int32 [m, 8]
    num_partials: int
    balance_snake: float
    balance_modulo: float
    kinds: int               # PA_KIND_BIT mask of the task kinds present


def build_task_table(params: PaParams, cu_seqlens_q, context_lens, tasks_out=None,
                     combines_out=None, with_balance=True, block_table=None) -> TaskTable:
    """Host task table (library call).

    Without output buffers the table is sized with a first call (PA_ERR_CAPACITY) and filled
    by a second. With ``tasks_out`` / ``combines_out`` (int32 [cap, 8] numpy arrays, e.g. views
    of pinned host memory) it is one call that writes into them; the returned TaskTable then
    holds views of the filled rows. A host ``block_table`` ([N, max_blocks]) selects
    build_task_table_shared, which groups decode sequences that share leading blocks when
    ``params.shared_min`` > 0.
    """
    L = lib()
    cu = _i32(cu_seqlens_q)
    ctx = _i32(context_lens)
    n = ctx.shape[0]
    if block_table is None:
        fn, name, head = L.build_task_table, "build_task_table", []
    else:
        bt = _i32(block_table)
        if bt.ndim != 2 or bt.shape[0] != n:
            raise ValueError("block_table must be [num_seqs, max_blocks]")
        fn, name, head = L.build_task_table_shared, "build_task_table_shared", \
            [_ptr(bt), bt.shape[1]]
    nt, nc, npart = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    kinds = ctypes.c_uint32(0)
    bal = (ctypes.c_double * 2)() if with_balance else None
    if tasks_out is None:
        rc = fn(ctypes.byref(params), _ptr(cu), _ptr(ctx), n, *head, None, 0, ctypes.byref(nt),
                None, 0, ctypes.byref(nc), ctypes.byref(npart), None, None)
        if rc not in (_abi.PA_OK, _abi.PA_ERR_CAPACITY):
            check(rc, name)
        tasks_out = np.zeros((nt.value, 8), dtype=np.int32)
        combines_out = np.zeros((nc.value, 8), dtype=np.int32)
    for a in (tasks_out, combines_out):
        if a.dtype != np.int32 or a.ndim != 2 or a.shape[1] != 8 or not a.flags.c_contiguous:
            raise ValueError("table buffers must be contiguous int32 [cap, 8]")
    rc = fn(ctypes.byref(params), _ptr(cu), _ptr(ctx), n, *head,
            tasks_out.ctypes.data_as(ctypes.POINTER(PaTask)), tasks_out.shape[0],
            ctypes.byref(nt), combines_out.ctypes.data_as(ctypes.POINTER(PaCombine)),
            combines_out.shape[0], ctypes.byref(nc), ctypes.byref(npart), bal,
            ctypes.byref(kinds))
    check(rc, name)
    return TaskTable(tasks_out[:nt.value], combines_out[:nc.value], npart.value,
                     bal[0] if bal is not None else float("nan"),
                     bal[1] if bal is not None else float("nan"), kinds.value)


def workspace_bytes(num_partials: int, head_dim: int) -> int:
    return int(lib().pa_workspace_bytes(int(num_partials), int(head_dim)))


def validate_block_table(block_table, context_lens, num_blocks, block_size):
    bt = _i32(block_table)
    ctx = _i32(context_lens)
    check(lib().pa_validate_block_table(_ptr(bt), bt.shape[1] if bt.ndim == 2 else 0, _ptr(ctx),
                                        ctx.shape[0], int(num_blocks), int(block_size)),
          "pa_validate_block_table")


# ------------------------------------------------------------------ device-side marshalling
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype == torch.float32:
        return PA_FP32
    raise PagedAttnError(_abi.PA_ERR_DTYPE, "binding", f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None, ndim=None):
    """Check a tensor is a contiguous GPU tensor (a kernel given a host pointer would fault)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def reshape_and_cache(k_new, v_new, k_pages, v_pages, block_table, cu_seqlens_q, context_lens,
                      stream=None):
    """Write packed new K/V rows [T, Hkv, D] into pages [NB, Hkv, bs, D] (library kernel)."""
    torch = _torch()
    T, hkv, d = k_new.shape
    nb, hkv2, bs, d2 = k_pages.shape
    if (hkv, d) != (hkv2, d2) or v_new.shape != k_new.shape or v_pages.shape != k_pages.shape:
        raise ValueError("k/v shapes disagree")
    if not (k_new.dtype == v_new.dtype == k_pages.dtype == v_pages.dtype):
        raise ValueError("k/v dtypes disagree")
    n = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != n or cu_seqlens_q.shape[0] != n + 1:
        raise ValueError("block_table / cu_seqlens_q / context_lens sizes disagree")
    args = [_dev(k_new, "k_new", ndim=3), _dev(v_new, "v_new", ndim=3),
            _dev(k_pages, "k_pages", ndim=4), _dev(v_pages, "v_pages", ndim=4),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1],
            _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
            _dev(context_lens, "context_lens", torch.int32), n, T, nb, hkv, d, bs,
            _dtype_code(k_new), _stream(stream)]
    check(lib().reshape_and_cache(*args), "reshape_and_cache")


def reshape_and_cache_fp8(k_new, v_new, k_pages, v_pages, scales, block_table,
                          cu_seqlens_q, context_lens, stream=None):
    """Write packed bf16 rows [T, Hkv, D] into fp8 pages (uint8 [NB, Hkv, bs, D]) with float32
    page scales [NB, Hkv, 2] (K then V per page), rescaling every page the step writes into
    (library kernel)."""
    torch = _torch()
    T, hkv, d = k_new.shape
    nb, hkv2, bs, d2 = k_pages.shape
    if (hkv, d) != (hkv2, d2) or v_new.shape != k_new.shape or v_pages.shape != k_pages.shape:
        raise ValueError("k/v shapes disagree")
    if tuple(scales.shape) != (nb, hkv, 2):
        raise ValueError("page scales must be [num_blocks, Hkv, 2]")
    n = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != n or cu_seqlens_q.shape[0] != n + 1:
        raise ValueError("block_table / cu_seqlens_q / context_lens sizes disagree")
    args = [_dev(k_new, "k_new", torch.bfloat16, 3), _dev(v_new, "v_new", torch.bfloat16, 3),
            _dev(k_pages, "k_pages", torch.uint8, 4), _dev(v_pages, "v_pages", torch.uint8, 4),
            _dev(scales, "scales", torch.float32),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1],
            _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
            _dev(context_lens, "context_lens", torch.int32), n, T, nb, hkv, d, bs,
            _stream(stream)]
    check(lib().reshape_and_cache_fp8(*args), "reshape_and_cache_fp8")


def _attn_common(q, k_pages, v_pages, block_table, context_lens, out):
    torch = _torch()
    if k_pages.shape != v_pages.shape or k_pages.dim() != 4:
        raise ValueError("k_pages and v_pages must both be [NB, Hkv, bs, D]")
    if q.dim() != 3 or out.shape != q.shape or q.dtype != out.dtype:
        raise ValueError("q and out must both be [T, Hq, D] of one dtype")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise ValueError("q and pages must share a dtype")
    if q.shape[2] != k_pages.shape[3]:
        raise ValueError("head_dim of q and pages differ")
    n = context_lens.shape[0]
    if block_table.dim() != 2 or block_table.shape[0] != n:
        raise ValueError("block_table must be [num_seqs, max_blocks]")
    return [_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1]]


def _table_args(tasks_dev, task_kinds, combines_dev, num_partials, workspace):
    torch = _torch()
    _dev(tasks_dev, "tasks_dev", torch.int32, 2)
    if combines_dev.shape[0] > 0:
        _dev(combines_dev, "combines_dev", torch.int32, 2)
    ws = None
    wsb = 0
    if workspace is not None and workspace.numel() > 0:
        ws = _dev(workspace, "workspace")
        wsb = workspace.numel() * workspace.element_size()
    return [ctypes.c_void_p(tasks_dev.data_ptr()), tasks_dev.shape[0], int(task_kinds),
            ctypes.c_void_p(combines_dev.data_ptr() if combines_dev.numel() else 0),
            combines_dev.shape[0], int(num_partials), ws, wsb]


def paged_attn_decode(q, k_pages, v_pages, block_table, context_lens, scale, tasks_dev,
                      task_kinds, combines_dev, num_partials, workspace, out, stream=None):
    """Decode attention (library kernels). q/out [N, Hq, D]; tasks from a table built with
    cu_seqlens = 0..N, copied to the device as int32 [n, 8]; task_kinds is the table's kind
    mask (TaskTable.kinds)."""
    torch = _torch()
    head = _attn_common(q, k_pages, v_pages, block_table, context_lens, out)
    n, hq, d = q.shape
    if context_lens.shape[0] != n:
        raise ValueError("decode takes one query row per sequence")
    args = head + [_dev(context_lens, "context_lens", torch.int32), n, hq, k_pages.shape[1], d,
                   k_pages.shape[2], float(scale), _dtype_code(q)] + \
        _table_args(tasks_dev, task_kinds, combines_dev, num_partials, workspace) + \
        [_dev(out, "out"), _stream(stream)]
    check(lib().paged_attn_decode(*args), "paged_attn_decode")


def paged_attn_decode_fp8(q, k_pages, v_pages, scales, block_table, context_lens,
                          scale, tasks_dev, task_kinds, combines_dev, num_partials, workspace,
                          out, stream=None):
    """Decode attention over fp8 pages with page scales (library kernels). q/out bf16
    [N, Hq, D]; pages uint8 [NB, Hkv, bs, D]; scales float32 [NB, Hkv, 2]."""
    torch = _torch()
    if k_pages.shape != v_pages.shape or k_pages.dim() != 4:
        raise ValueError("k_pages and v_pages must both be [NB, Hkv, bs, D]")
    if q.dim() != 3 or out.shape != q.shape or q.shape[2] != k_pages.shape[3]:
        raise ValueError("q and out must both be [N, Hq, D] with the pages' head_dim")
    nb, hkv = k_pages.shape[:2]
    if tuple(scales.shape) != (nb, hkv, 2):
        raise ValueError("page scales must be [num_blocks, Hkv, 2]")
    n, hq, d = q.shape
    if context_lens.shape[0] != n or block_table.dim() != 2 or block_table.shape[0] != n:
        raise ValueError("decode takes one query row per sequence")
    args = [_dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", torch.uint8),
            _dev(v_pages, "v_pages", torch.uint8), _dev(scales, "scales", torch.float32),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1],
            _dev(context_lens, "context_lens", torch.int32), n, hq, hkv, d, k_pages.shape[2],
            float(scale)] + \
        _table_args(tasks_dev, task_kinds, combines_dev, num_partials, workspace) + \
        [_dev(out, "out", torch.bfloat16), _stream(stream)]
    check(lib().paged_attn_decode_fp8(*args), "paged_attn_decode_fp8")


def _fp8_packed_args(q, k_pages, v_pages, scales, block_table, cu_seqlens_q, context_lens,
                     scale, tasks_dev, task_kinds, combines_dev, num_partials, workspace, out,
                     stream):
    """Argument list of the fp8 entries over packed rows (verify and the unified launch)."""
    torch = _torch()
    if k_pages.shape != v_pages.shape or k_pages.dim() != 4:
        raise ValueError("k_pages and v_pages must both be [NB, Hkv, bs, D]")
    if q.dim() != 3 or out.shape != q.shape or q.shape[2] != k_pages.shape[3]:
        raise ValueError("q and out must both be [T, Hq, D] with the pages' head_dim")
    nb, hkv = k_pages.shape[:2]
    if tuple(scales.shape) != (nb, hkv, 2):
        raise ValueError("page scales must be [num_blocks, Hkv, 2]")
    t, hq, d = q.shape
    n = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != n + 1 or block_table.dim() != 2 or block_table.shape[0] != n:
        raise ValueError("block_table / cu_seqlens_q / context_lens sizes disagree")
    args = [_dev(q, "q", torch.bfloat16), _dev(k_pages, "k_pages", torch.uint8),
            _dev(v_pages, "v_pages", torch.uint8), _dev(scales, "scales", torch.float32),
            _dev(block_table, "block_table", torch.int32), block_table.shape[1],
            _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
            _dev(context_lens, "context_lens", torch.int32), n, t, hq, hkv, d, k_pages.shape[2],
            float(scale)] + \
        _table_args(tasks_dev, task_kinds, combines_dev, num_partials, workspace) + \
        [_dev(out, "out", torch.bfloat16), _stream(stream)]
    return args


def paged_attn_verify_fp8(q, k_pages, v_pages, scales, block_table, cu_seqlens_q,
                          context_lens, scale, tasks_dev, task_kinds, combines_dev, num_partials,
                          workspace, out, stream=None):
    """Decode rows and speculative drafts over fp8 pages with page scales (library kernels).
    q/out bf16 [T, Hq, D] packed by cu_seqlens_q; pages uint8 [NB, Hkv, bs, D]; scales
    float32 [NB, Hkv, 2]. Runs the table's decode and verify tasks only."""
    args = _fp8_packed_args(q, k_pages, v_pages, scales, block_table, cu_seqlens_q,
                            context_lens, scale, tasks_dev, task_kinds, combines_dev,
                            num_partials, workspace, out, stream)
    check(lib().paged_attn_verify_fp8(*args), "paged_attn_verify_fp8")


def paged_attn_varlen_prefill_fp8(q, k_pages, v_pages, scales, block_table, cu_seqlens_q,
                                  context_lens, scale, tasks_dev, task_kinds, combines_dev,
                                  num_partials, workspace, out, stream=None):
    """The unified launch over fp8 pages (library kernels): decode, prefill, verify and
    shared-prefix tasks in one grid. q/out bf16 [T, Hq, D] packed by cu_seqlens_q; pages uint8
    [NB, Hkv, bs, D]; scales float32 [NB, Hkv, 2]."""
    args = _fp8_packed_args(q, k_pages, v_pages, scales, block_table, cu_seqlens_q,
                            context_lens, scale, tasks_dev, task_kinds, combines_dev,
                            num_partials, workspace, out, stream)
    check(lib().paged_attn_varlen_prefill_fp8(*args), "paged_attn_varlen_prefill_fp8")


def paged_attn_varlen_prefill(q, k_pages, v_pages, block_table, cu_seqlens_q, context_lens,
                              scale, tasks_dev, task_kinds, combines_dev, num_partials, workspace,
                              out, stream=None):
    """Packed causal attention over paged prefixes, decode rows and prefill chunks mixed
    (library kernels). q/out [T, Hq, D]."""
    torch = _torch()
    head = _attn_common(q, k_pages, v_pages, block_table, context_lens, out)
    T, hq, d = q.shape
    n = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != n + 1:
        raise ValueError("cu_seqlens_q must be [num_seqs + 1]")
    args = head + [_dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                   _dev(context_lens, "context_lens", torch.int32), n, T, hq, k_pages.shape[1],
                   d, k_pages.shape[2], float(scale), _dtype_code(q)] + \
        _table_args(tasks_dev, task_kinds, combines_dev, num_partials, workspace) + \
        [_dev(out, "out"), _stream(stream)]
    check(lib().paged_attn_varlen_prefill(*args), "paged_attn_varlen_prefill")


def paged_attn_varlen_prefill_noalloc(q, k_pages, v_pages, block_table, cu_seqlens_q,
                                      context_lens, scale, tasks_dev, task_kinds, combines_dev,
                                      num_partials, out, stream=None):
    """paged_attn_varlen_prefill with its partial rows in the library's own device scratch
    (no workspace argument; nothing is allocated). Calls that overlap on one GPU share that
    scratch and must be ordered by the caller."""
    torch = _torch()
    head = _attn_common(q, k_pages, v_pages, block_table, context_lens, out)
    T, hq, d = q.shape
    n = context_lens.shape[0]
    if cu_seqlens_q.shape[0] != n + 1:
        raise ValueError("cu_seqlens_q must be [num_seqs + 1]")
    tbl = _table_args(tasks_dev, task_kinds, combines_dev, num_partials, None)[:-2]
    args = head + [_dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
                   _dev(context_lens, "context_lens", torch.int32), n, T, hq, k_pages.shape[1],
                   d, k_pages.shape[2], float(scale), _dtype_code(q)] + tbl + \
        [_dev(out, "out"), _stream(stream)]
    check(lib().paged_attn_varlen_prefill_noalloc(*args), "paged_attn_varlen_prefill_noalloc")


class StepPlan:
    """A task table built on the host for one batch, copied to the device, with its workspace.

    Holds device int32 copies of cu_seqlens, context_lens, the block table and the table, so a
    caller can launch the step repeatedly. All memory comes from torch's allocator.
    """

    def __init__(self, q_lens, context_lens, block_table, num_q_heads, num_kv_heads, head_dim,
                 block_size, device="cuda", **tiling):
        torch = _torch()
        self.cu_host = pack_seqlens(q_lens)
        self.ctx_host = _i32(context_lens)
        self.params = make_params(num_q_heads, num_kv_heads, head_dim, block_size, **tiling)
        self.table = build_task_table(self.params, self.cu_host, self.ctx_host,
                                      block_table=block_table if self.params.shared_min else None)
        self.head_dim = head_dim
        self.device = device
        self.cu = torch.from_numpy(self.cu_host).to(device)
        self.ctx = torch.from_numpy(self.ctx_host).to(device)
        self.block_table = torch.from_numpy(_i32(block_table)).to(device)
        self.tasks = torch.from_numpy(self.table.tasks).to(device)
        self.combines = torch.from_numpy(self.table.combines).to(device)
        nbytes = workspace_bytes(self.table.num_partials, head_dim)
        self.workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)
        self.decode_only = bool(np.all(np.diff(self.cu_host) == 1))

    @property
    def num_partials(self):
        return self.table.num_partials

    def write_cache(self, k_new, v_new, k_pages, v_pages, stream=None):
        reshape_and_cache(k_new, v_new, k_pages, v_pages, self.block_table, self.cu, self.ctx,
                          stream)

    def _check_decode_table(self, who):
        if not self.decode_only or self.params.verify_rows:
            raise ValueError(f"{who} runs decode tasks only: every q_len must be 1 and "
                             "verify_rows 0 (use varlen for other batches)")

    def decode(self, q, k_pages, v_pages, scale, out, stream=None):
        self._check_decode_table("decode")
        paged_attn_decode(q, k_pages, v_pages, self.block_table, self.ctx, scale, self.tasks,
                          self.table.kinds, self.combines, self.num_partials, self.workspace, out,
                          stream)

    def write_cache_fp8(self, k_new, v_new, k_pages, v_pages, scales, stream=None):
        reshape_and_cache_fp8(k_new, v_new, k_pages, v_pages, scales,
                              self.block_table, self.cu, self.ctx, stream)

    def decode_fp8(self, q, k_pages, v_pages, scales, scale, out, stream=None):
        self._check_decode_table("decode_fp8")
        paged_attn_decode_fp8(q, k_pages, v_pages, scales, self.block_table,
                              self.ctx, scale, self.tasks, self.table.kinds, self.combines,
                              self.num_partials, self.workspace, out, stream)

    def verify_fp8(self, q, k_pages, v_pages, scales, scale, out, stream=None):
        kinds = set(np.unique(self.table.tasks[:, 0]).tolist()) if len(self.table.tasks) else set()
        if not kinds <= {PA_TASK_DECODE, PA_TASK_VERIFY}:
            raise ValueError("verify_fp8 runs decode and verify tasks only: build the table with "
                             "verify_rows covering every draft and shared_min 0")
        paged_attn_verify_fp8(q, k_pages, v_pages, scales, self.block_table, self.cu,
                              self.ctx, scale, self.tasks, self.table.kinds, self.combines,
                              self.num_partials, self.workspace, out, stream)

    def varlen(self, q, k_pages, v_pages, scale, out, stream=None):
        paged_attn_varlen_prefill(q, k_pages, v_pages, self.block_table, self.cu, self.ctx,
                                  scale, self.tasks, self.table.kinds, self.combines,
                                  self.num_partials, self.workspace, out, stream)

    def varlen_fp8(self, q, k_pages, v_pages, scales, scale, out, stream=None):
        paged_attn_varlen_prefill_fp8(q, k_pages, v_pages, scales, self.block_table, self.cu,
                                      self.ctx, scale, self.tasks, self.table.kinds,
                                      self.combines, self.num_partials, self.workspace, out,
                                      stream)


# ------------------------------------------------------------------ SmoothGEMM
@dataclass
class GemmTable:
    tasks: np.ndarray        # int32 [n, 8]: m0, rows, n0, cols, k0, k1, slot, 0
    reduces: np.ndarray      # int32 [m, 8]: m0, rows, n0, cols, first_slot, n_slots, 0, 0
    num_slots: int
    balance_snake: float
    balance_modulo: float


def build_gemm_table(M, N, K, tile=256, k_split=0, num_workers=256,
                     tail_split=False) -> GemmTable:
    """Host Linear decomposition for C = A W^T (library call; sized by a first call). With
    ``tail_split`` the blocks of the last, partial round of ``num_workers`` are cut into K
    pieces."""
    L = lib()
    prm = PaGemmParams(int(tile), int(k_split), int(num_workers), int(bool(tail_split)))
    nt, nr, ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    rc = L.build_gemm_table(ctypes.byref(prm), int(M), int(N), int(K), None, 0, ctypes.byref(nt),
                            None, 0, ctypes.byref(nr), ctypes.byref(ns), None)
    if rc not in (_abi.PA_OK, _abi.PA_ERR_CAPACITY):
        check(rc, "build_gemm_table")
    tasks = np.zeros((nt.value, 8), dtype=np.int32)
    reds = np.zeros((nr.value, 8), dtype=np.int32)
    bal = (ctypes.c_double * 2)()
    rc = L.build_gemm_table(ctypes.byref(prm), int(M), int(N), int(K),
                            tasks.ctypes.data_as(ctypes.POINTER(PaGemmTask)), tasks.shape[0],
                            ctypes.byref(nt), reds.ctypes.data_as(ctypes.POINTER(PaGemmReduce)),
                            reds.shape[0], ctypes.byref(nr), ctypes.byref(ns), bal)
    check(rc, "build_gemm_table")
    return GemmTable(tasks, reds, ns.value, bal[0], bal[1])


def gemm_workspace_bytes(num_slots: int, tile: int) -> int:
    return int(lib().pa_gemm_workspace_bytes(int(num_slots), int(tile)))


def smooth_gemm(a, w, c, tile, tasks_dev, reduces_dev, num_slots, workspace, stream=None):
    """C [M, N] = A [M, K] W [N, K]^T in bf16 with fp32 accumulation (library kernels), from a
    table built by build_gemm_table for the same M, N, K and tile, copied to the device."""
    torch = _torch()
    if a.dim() != 2 or w.dim() != 2 or c.dim() != 2:
        raise ValueError("a, w, c must be 2-D")
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or tuple(c.shape) != (M, N):
        raise ValueError(f"shapes disagree: a {tuple(a.shape)}, w {tuple(w.shape)}, "
                         f"c {tuple(c.shape)}")
    args = [_dev(a, "a", torch.bfloat16), _dev(w, "w", torch.bfloat16),
            _dev(c, "c", torch.bfloat16), M, N, K, int(tile),
            _dev(tasks_dev, "tasks_dev", torch.int32, 2) if tasks_dev.numel() else None,
            tasks_dev.shape[0]]
    if reduces_dev.shape[0] > 0:
        args += [_dev(reduces_dev, "reduces_dev", torch.int32, 2), reduces_dev.shape[0]]
    else:
        args += [None, 0]
    ws, wsb = None, 0
    if workspace is not None and workspace.numel() > 0:
        ws = _dev(workspace, "workspace")
        wsb = workspace.numel() * workspace.element_size()
    args += [int(num_slots), ws, wsb, _stream(stream)]
    check(lib().smooth_gemm(*args), "smooth_gemm")


class GemmPlan:
    """A SmoothGEMM table for one (M, N, K) built on the host and copied to the device, with
    its workspace (torch allocations)."""

    def __init__(self, M, N, K, tile=256, k_split=0, num_workers=256, device="cuda",
                 tail_split=False):
        torch = _torch()
        self.M, self.N, self.K, self.tile = int(M), int(N), int(K), int(tile)
        self.table = build_gemm_table(M, N, K, tile, k_split, num_workers, tail_split)
        self.tasks = torch.from_numpy(self.table.tasks).to(device)
        self.reduces = torch.from_numpy(self.table.reduces).to(device)
        nbytes = gemm_workspace_bytes(self.table.num_slots, tile)
        self.workspace = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)

    def run(self, a, w, c, stream=None):
        if (a.shape[0], w.shape[0], a.shape[1]) != (self.M, self.N, self.K):
            raise ValueError("operands do not match the plan's M, N, K")
        smooth_gemm(a, w, c, self.tile, self.tasks, self.reduces, self.table.num_slots,
                    self.workspace, stream)
