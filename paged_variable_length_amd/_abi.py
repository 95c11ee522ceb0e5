"""ctypes view of libpagedattn.so (the C ABI declared in include/pagedattn.h).

Argument marshalling only: every computation happens in the library. Loading fails loudly when
the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedattn.so")

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_SHAPE = -2
PA_ERR_BLOCK_SIZE = -3
PA_ERR_DTYPE = -4
PA_ERR_CAPACITY = -5
PA_ERR_INPUT = -6
PA_ERR_HIP = -7
PA_BF16 = 0
PA_FP32 = 1
PA_TASK_DECODE = 0
PA_TASK_PREFILL = 1
PA_TASK_VERIFY = 2
PA_TASK_SHARED = 3
NOALLOC_SCRATCH_BYTES = 64 << 20   # PA_NOALLOC_SCRATCH_BYTES
ALL_KINDS = 0xF          # PA_KIND_BIT of every task kind
ABI_VERSION = 10

ERROR_NAMES = {
    PA_ERR_NULL: "PA_ERR_NULL", PA_ERR_SHAPE: "PA_ERR_SHAPE",
    PA_ERR_BLOCK_SIZE: "PA_ERR_BLOCK_SIZE", PA_ERR_DTYPE: "PA_ERR_DTYPE",
    PA_ERR_CAPACITY: "PA_ERR_CAPACITY", PA_ERR_INPUT: "PA_ERR_INPUT", PA_ERR_HIP: "PA_ERR_HIP",
}

# every symbol include/pagedattn.h declares
EXPORTS = ("pa_abi_version", "pa_last_error", "pa_pack_seqlens", "build_task_table",
           "pa_workspace_bytes", "reshape_and_cache", "paged_attn_decode",
           "paged_attn_varlen_prefill", "pa_validate_block_table", "reshape_and_cache_fp8",
           "paged_attn_decode_fp8", "paged_attn_verify_fp8", "paged_attn_varlen_prefill_fp8",
           "paged_attn_varlen_prefill_noalloc",
           "build_task_table_shared", "build_gemm_table", "pa_gemm_workspace_bytes",
           "smooth_gemm")


class PaTask(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("kind", "seq", "head", "q_row0", "q_rows", "kv0", "kv1", "partial")]


class PaCombine(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("seq", "q_row0", "q_rows", "head", "heads", "first_slot", "n_slots", "reserved")]


class PaGemmTask(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("m0", "rows", "n0", "cols", "k0", "k1", "slot", "reserved")]


class PaGemmReduce(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("m0", "rows", "n0", "cols", "first_slot", "n_slots", "reserved0", "reserved1")]


class PaGemmParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("tile", "k_split", "num_workers", "tail_split")]


class PaParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("num_q_heads", "num_kv_heads", "head_dim", "block_size", "dec_split",
                 "pf_q_tile", "pf_kv_split", "num_workers", "decode_weight", "verify_rows",
                 "shared_min", "reserved")]


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m paged_variable_length_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    i32, u32, p = ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    L.pa_abi_version.restype = ctypes.c_int
    L.pa_abi_version.argtypes = []
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    L.pa_pack_seqlens.restype = ctypes.c_int
    L.pa_pack_seqlens.argtypes = [pi32, i32, pi32]
    L.build_task_table.restype = ctypes.c_int
    pu32 = ctypes.POINTER(ctypes.c_uint32)
    L.build_task_table.argtypes = [ctypes.POINTER(PaParams), pi32, pi32, i32,
                                   ctypes.POINTER(PaTask), i32, pi32,
                                   ctypes.POINTER(PaCombine), i32, pi32, pi32,
                                   ctypes.POINTER(ctypes.c_double), pu32]
    L.build_task_table_shared.restype = ctypes.c_int
    L.build_task_table_shared.argtypes = [ctypes.POINTER(PaParams), pi32, pi32, i32, pi32, i32,
                                          ctypes.POINTER(PaTask), i32, pi32,
                                          ctypes.POINTER(PaCombine), i32, pi32, pi32,
                                          ctypes.POINTER(ctypes.c_double), pu32]
    L.pa_workspace_bytes.restype = ctypes.c_size_t
    L.pa_workspace_bytes.argtypes = [i32, i32]
    L.reshape_and_cache.restype = ctypes.c_int
    L.reshape_and_cache.argtypes = [p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32, i32,
                                    i32, p]
    L.paged_attn_decode.restype = ctypes.c_int
    L.paged_attn_decode.argtypes = [p, p, p, p, i32, p, i32, i32, i32, i32, i32,
                                    ctypes.c_float, i32, p, i32, u32, p, i32, i32, p,
                                    ctypes.c_size_t, p, p]
    L.paged_attn_varlen_prefill.restype = ctypes.c_int
    L.paged_attn_varlen_prefill.argtypes = [p, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                                            i32, ctypes.c_float, i32, p, i32, u32, p, i32, i32,
                                            p, ctypes.c_size_t, p, p]
    L.paged_attn_varlen_prefill_noalloc.restype = ctypes.c_int
    L.paged_attn_varlen_prefill_noalloc.argtypes = [p, p, p, p, i32, p, p, i32, i32, i32, i32,
                                                    i32, i32, ctypes.c_float, i32, p, i32, u32, p,
                                                    i32, i32, p, p]
    L.reshape_and_cache_fp8.restype = ctypes.c_int
    L.reshape_and_cache_fp8.argtypes = [p, p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                                        i32, p]
    L.paged_attn_decode_fp8.restype = ctypes.c_int
    L.paged_attn_decode_fp8.argtypes = [p, p, p, p, p, i32, p, i32, i32, i32, i32, i32,
                                        ctypes.c_float, p, i32, u32, p, i32, i32, p,
                                        ctypes.c_size_t, p, p]
    L.paged_attn_verify_fp8.restype = ctypes.c_int
    L.paged_attn_verify_fp8.argtypes = [p, p, p, p, p, i32, p, p, i32, i32, i32, i32, i32,
                                        i32, ctypes.c_float, p, i32, u32, p, i32, i32, p,
                                        ctypes.c_size_t, p, p]
    # same argument list as the verify entry
    L.paged_attn_varlen_prefill_fp8.restype = ctypes.c_int
    L.paged_attn_varlen_prefill_fp8.argtypes = list(L.paged_attn_verify_fp8.argtypes)
    L.pa_validate_block_table.restype = ctypes.c_int
    L.pa_validate_block_table.argtypes = [pi32, i32, pi32, i32, i32, i32]
    L.build_gemm_table.restype = ctypes.c_int
    L.build_gemm_table.argtypes = [ctypes.POINTER(PaGemmParams), i32, i32, i32,
                                   ctypes.POINTER(PaGemmTask), i32, pi32,
                                   ctypes.POINTER(PaGemmReduce), i32, pi32, pi32,
                                   ctypes.POINTER(ctypes.c_double)]
    L.pa_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.pa_gemm_workspace_bytes.argtypes = [i32, i32]
    L.smooth_gemm.restype = ctypes.c_int
    L.smooth_gemm.argtypes = [p, p, p, i32, i32, i32, i32, p, i32, p, i32, i32, p,
                              ctypes.c_size_t, p]
    if L.pa_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libpagedattn ABI {L.pa_abi_version()} != binding {ABI_VERSION}")
    _lib = L
    return L


def check(rc: int, where: str):
    if rc != PA_OK:
        raise PagedAttnError(rc, where, lib().pa_last_error().decode(errors="replace"))
