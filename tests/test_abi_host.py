"""Host-side checks of libpagedattn.so (no GPU needed): the library loads and exports every
symbol the header declares, and its host functions -- packing, the task table, workspace
sizing, block-table validation, argument checks -- agree with the oracle or the header.
The task table must match the oracle's bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import paged_variable_length_amd as pa
from bench import TILING as BENCH_TILING
from paged_variable_length_amd import _abi
from oracle import task_table as ot
from tests.helpers import aliased_batch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "pagedattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\(", text, flags=re.M))


def test_library_exports_every_declared_symbol():
    L = _abi.lib()
    declared = header_functions()
    assert declared == set(_abi.EXPORTS), declared ^ set(_abi.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    assert L.pa_abi_version() == _abi.ABI_VERSION


def test_pack_seqlens_worked_example_and_errors():
    assert pa.pack_seqlens([128, 64, 256]).tolist() == [0, 128, 192, 448]
    assert pa.pack_seqlens([]).tolist() == [0]
    with pytest.raises(pa.PagedAttnError) as e:
        pa.pack_seqlens([3, 0])
    assert e.value.code == _abi.PA_ERR_INPUT
    with pytest.raises(pa.PagedAttnError):
        pa.pack_seqlens([2**30, 2**30, 2**30])


def compare_tables(q_lens, ctx, **kw):
    hq, hkv, d, bs = kw.pop("hq"), kw.pop("hkv"), kw.pop("d", 128), kw.pop("bs")
    cu = pa.pack_seqlens(q_lens)
    got = pa.build_task_table(pa.make_params(hq, hkv, d, bs, **kw), cu, ctx)
    ref_t, ref_c, ref_np, _, ref_bal = ot.build_task_table(ot.Params(hq, hkv, d, bs, **kw), cu, ctx)
    assert np.array_equal(got.tasks, ref_t)
    assert np.array_equal(got.combines, ref_c)
    assert got.num_partials == ref_np
    assert got.balance_snake == ref_bal["snake"]
    assert got.balance_modulo == ref_bal["modulo"]
    assert got.kinds == kind_mask(ref_t)
    return got


def kind_mask(tasks):
    """PA_KIND_BIT mask of the kinds among task records (column 0)."""
    m = 0
    for k in set(np.asarray(tasks)[:, 0].tolist()):
        m |= 1 << int(k)
    return m


@pytest.mark.parametrize("name", ["tiny_decode_fp32", "decode_mha_bf16", "decode_gqa_bf16_bs16",
                                  "decode_gqa_bf16_bs64", "prefill_varlen_bf16", "mixed_bf16"])
def test_task_table_bit_exact_on_workloads(name):
    w = synth.make_workload(name)
    tiling = dict(dec_split=512, pf_q_tile=128, pf_kv_split=0 if name != "mixed_bf16" else 8192)
    compare_tables(w.q_lens, w.ctx_lens, hq=w.num_q_heads, hkv=w.num_kv_heads, d=w.head_dim,
                   bs=w.block_size, num_workers=512, **tiling)


@pytest.mark.parametrize("name", sorted(BENCH_TILING))
def test_task_table_bit_exact_in_bench_tilings(name):
    """Every workload bench.py times, in the tiling it times (its TILING, with the 512
    resident workgroups it reports balance for): the C++ table equals the oracle's bit for bit,
    shared-prefix groups included."""
    w = synth.make_workload(name.split(":")[0])
    tiling = dict(BENCH_TILING[name], num_workers=512)
    args = dict(hq=w.num_q_heads, hkv=w.num_kv_heads, d=w.head_dim, bs=w.block_size, **tiling)
    if tiling.get("shared_min"):
        got = compare_shared(w.q_lens, w.ctx_lens, w.block_table, **args)
    else:
        got = compare_tables(w.q_lens, w.ctx_lens, **args)
    assert len(got.tasks) > 0


@pytest.mark.parametrize("seed", range(8))
def test_task_table_bit_exact_random(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 12))
    q = [1 if rng.random() < 0.4 else
         int(rng.integers(2, 9)) if rng.random() < 0.5 else int(rng.integers(2, 300))
         for _ in range(n)]
    ctx = [qq + int(rng.integers(0, 700)) for qq in q]
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 4, 8]))
    compare_tables(q, ctx, hq=hq, hkv=hkv, bs=int(rng.choice([16, 32, 64, 128, 256])),
                   dec_split=64 * int(rng.integers(1, 6)), pf_q_tile=int(rng.integers(1, 129)),
                   pf_kv_split=64 * int(rng.integers(0, 5)), num_workers=int(rng.integers(1, 40)),
                   decode_weight=int(rng.integers(1, 4)),
                   verify_rows=int(rng.choice([0, 2, 4, 8, 16])))


def test_task_table_many_distinct_loads():
    # prefill tiles over long prefixes give loads spread over ~2^22, so the sort takes several
    # digit passes; ties between heads must keep emission order
    q = [200, 1, 130, 1, 77]
    ctx = [40000, 9000, 25000, 3, 4000]
    compare_tables(q, ctx, hq=4, hkv=2, bs=64, dec_split=192, pf_q_tile=64, pf_kv_split=0,
                   num_workers=7, decode_weight=3)


def test_task_table_loads_wider_than_32_bits():
    # a 128-row tile behind a 2^25-key prefix has a load above 2^32, next to a one-key decode
    q = [128, 1, 1]
    ctx = [2**25 + 128, 1, 70]
    compare_tables(q, ctx, hq=2, hkv=1, bs=16, dec_split=64, pf_q_tile=128, pf_kv_split=0,
                   num_workers=3)


def test_task_table_errors_match_oracle():
    cases = [
        (dict(hq=2, hkv=1, bs=12), [1], [5], _abi.PA_ERR_BLOCK_SIZE),
        (dict(hq=2, hkv=1, bs=48), [1], [5], _abi.PA_ERR_BLOCK_SIZE),
        (dict(hq=3, hkv=2, bs=16), [1], [5], _abi.PA_ERR_SHAPE),
        (dict(hq=2, hkv=1, bs=16, dec_split=100), [1], [5], _abi.PA_ERR_SHAPE),
        (dict(hq=2, hkv=1, bs=16, pf_q_tile=0), [1], [5], _abi.PA_ERR_SHAPE),
        (dict(hq=2, hkv=1, bs=16, pf_kv_split=32), [1], [5], _abi.PA_ERR_SHAPE),
        (dict(hq=2, hkv=1, bs=16), [4], [3], _abi.PA_ERR_INPUT),
        (dict(hq=2, hkv=1, bs=16, verify_rows=1), [1], [5], _abi.PA_ERR_SHAPE),
        (dict(hq=2, hkv=1, bs=16, verify_rows=17), [1], [5], _abi.PA_ERR_SHAPE),
    ]
    for kw, q, ctx, code in cases:
        hq, hkv, bs = kw.pop("hq"), kw.pop("hkv"), kw.pop("bs")
        cu = np.concatenate([[0], np.cumsum(q)]).astype(np.int32)
        with pytest.raises(pa.PagedAttnError) as e:
            pa.build_task_table(pa.make_params(hq, hkv, 64, bs, **kw), cu, ctx)
        assert e.value.code == code
        with pytest.raises(ot.TaskTableError) as e2:
            ot.build_task_table(ot.Params(hq, hkv, 64, bs, **kw), cu, ctx)
        assert e2.value.code == code
    # the library's tasks hold at most 128 rows (four waves of 32): its builder refuses taller
    # tiles, which the oracle's decomposition itself would accept
    with pytest.raises(pa.PagedAttnError) as e:
        pa.build_task_table(pa.make_params(2, 1, 64, 16, pf_q_tile=129), np.array([0, 1], np.int32),
                            [5])
    assert e.value.code == _abi.PA_ERR_SHAPE
    tasks, *_ = ot.build_task_table(ot.Params(2, 1, 64, 16, pf_q_tile=300), [0, 300], [300])
    assert len(tasks) == 2 and tasks[0][4] == 300      # one tile of 300 rows per head
    # non-increasing offsets are caught by the table builder itself
    with pytest.raises(pa.PagedAttnError) as e:
        pa.build_task_table(pa.make_params(2, 1, 64, 16), np.array([0, 2, 2], np.int32), [5, 5])
    assert e.value.code == _abi.PA_ERR_INPUT


def test_reserved_params_must_be_zero():
    p = pa.make_params(2, 1, 64, 16)
    p.reserved = 3
    with pytest.raises(pa.PagedAttnError) as e:
        pa.build_task_table(p, np.array([0, 1], np.int32), np.array([5], np.int32))
    assert e.value.code == _abi.PA_ERR_SHAPE


def test_task_table_capacity_sizing():
    L = _abi.lib()
    p = pa.make_params(2, 1, 64, 16, dec_split=64)
    cu = np.array([0, 1], np.int32)
    ctx = np.array([200], np.int32)
    nt, nc, npart = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    P = ctypes.POINTER(ctypes.c_int32)
    rc = L.build_task_table(ctypes.byref(p), cu.ctypes.data_as(P), ctx.ctypes.data_as(P), 1,
                            None, 0, ctypes.byref(nt), None, 0, ctypes.byref(nc),
                            ctypes.byref(npart), None, None)
    assert rc == _abi.PA_ERR_CAPACITY
    assert (nt.value, nc.value, npart.value) == (4, 1, 8)


def test_empty_batch_table():
    t = pa.build_task_table(pa.make_params(2, 1, 64, 16), np.array([0], np.int32),
                            np.zeros(0, np.int32))
    assert t.tasks.shape == (0, 8) and t.combines.shape == (0, 8) and t.num_partials == 0


def test_workspace_bytes():
    assert pa.workspace_bytes(0, 128) == 0
    # 3 rows * 128 floats = 1536 B (already 256-aligned) + 3 * 8 B -> 1560 -> 1792
    assert pa.workspace_bytes(3, 128) == 1792
    assert pa.workspace_bytes(1, 64) % 256 == 0 and pa.workspace_bytes(1, 64) >= 256 + 8


def test_validate_block_table():
    w = synth.custom_workload([1, 1], [20, 40], 2, 1, 64, 16, seed=1)
    pa.validate_block_table(w.block_table, w.ctx_lens, w.num_blocks, 16)
    bad = w.block_table.copy()
    bad[1, 1] = w.num_blocks            # out of range
    with pytest.raises(pa.PagedAttnError) as e:
        pa.validate_block_table(bad, w.ctx_lens, w.num_blocks, 16)
    assert e.value.code == _abi.PA_ERR_INPUT
    dup = w.block_table.copy()
    dup[1, 0] = dup[0, 0]               # one physical block claimed twice
    with pytest.raises(pa.PagedAttnError):
        pa.validate_block_table(dup, w.ctx_lens, w.num_blocks, 16)
    # an entry past a sequence's need is never checked (it is never read)
    tail = w.block_table.copy()
    tail[0, 2] = 10**6                 # seq 0 (ctx 20) needs 2 of the 3 columns
    pa.validate_block_table(tail, w.ctx_lens, w.num_blocks, 16)


def test_launcher_scalar_errors_need_no_gpu():
    """Scalar argument checks run before any HIP call, so bad shapes are reported on the host."""
    L = _abi.lib()
    nul = None
    # block size 12
    rc = L.reshape_and_cache(nul, nul, nul, nul, nul, 1, nul, nul, 1, 1, 1, 1, 64, 12, 0, nul)
    assert rc == _abi.PA_ERR_BLOCK_SIZE
    # head_dim 96
    rc = L.reshape_and_cache(nul, nul, nul, nul, nul, 1, nul, nul, 1, 1, 1, 1, 96, 16, 0, nul)
    assert rc == _abi.PA_ERR_SHAPE
    # zero tokens: no-op, no pointer needed
    rc = L.reshape_and_cache(nul, nul, nul, nul, nul, 1, nul, nul, 1, 0, 1, 1, 64, 16, 0, nul)
    assert rc == _abi.PA_OK
    args = lambda hq, hkv, d, bs, dt, ncomb=0, ws=None, wsb=0: [  # noqa: E731
        nul, nul, nul, nul, 1, nul, 1, hq, hkv, d, bs, 0.1, dt, nul, 1, 1, nul, ncomb, 8, ws,
        wsb, nul, nul]
    assert L.paged_attn_decode(*args(3, 2, 64, 16, 0)) == _abi.PA_ERR_SHAPE
    assert L.paged_attn_decode(*args(34, 1, 64, 16, 0)) == _abi.PA_ERR_SHAPE     # G > 16
    assert L.paged_attn_decode(*args(2, 1, 64, 16, 7)) == _abi.PA_ERR_DTYPE
    assert L.paged_attn_decode(*args(2, 1, 64, 16, 0, 1, None, 0)) == _abi.PA_ERR_NULL
    assert L.paged_attn_decode(*args(2, 1, 64, 16, 0, 1, ctypes.c_void_p(16), 8)) == \
        _abi.PA_ERR_CAPACITY
    # a workspace is needed whenever the table has partial rows, combines or not
    assert L.paged_attn_decode(*args(2, 1, 64, 16, 0)) == _abi.PA_ERR_NULL
    assert b"workspace" in L.pa_last_error()
    ws = ctypes.c_void_p(256)
    assert L.paged_attn_decode(*args(2, 1, 64, 16, 0, 0, ws, 1 << 20)) == _abi.PA_ERR_NULL  # q
    assert b"NULL pointer" in L.pa_last_error()
    # every device pointer but context_lens given: still refused before any launch
    p = ctypes.c_void_p(256)
    full = [p, p, p, p, 1, None, 1, 2, 1, 64, 16, 0.1, 0, p, 1, 1, p, 1, 8, p, 1 << 20, p, None]
    assert L.paged_attn_decode(*full) == _abi.PA_ERR_NULL
    fp8 = full[:3] + [p] + full[3:12] + full[13:]     # one scales array after the pages
    assert L.paged_attn_decode_fp8(*fp8) == _abi.PA_ERR_NULL
    # one workgroup per task: 2^23 tasks exceed one launch
    big = list(full)
    big[5], big[14] = p, 1 << 23
    assert L.paged_attn_decode(*big) == _abi.PA_ERR_SHAPE
    assert b"at most 8388607" in L.pa_last_error()
    rc = L.reshape_and_cache(p, p, p, p, p, 1, p, p, 1, 1 << 23, 1, 1, 64, 16, 0, None)
    assert rc == _abi.PA_ERR_SHAPE
    # the fp8 verify entry: packed rows need cu_seqlens, at least one token per sequence
    ver = [p, p, p, p, p, 1, None, p, 2, 4, 8, 2, 128, 16, 0.1, p, 3, 1, p, 1, 4, p, 1 << 20,
           p, None]
    assert L.paged_attn_verify_fp8(*ver) == _abi.PA_ERR_NULL
    ver[6] = p
    ver[9] = 1                                            # 1 token for 2 sequences
    assert L.paged_attn_verify_fp8(*ver) == _abi.PA_ERR_SHAPE
    ver[9], ver[16] = 4, 0                                # an empty table: a no-op
    assert L.paged_attn_verify_fp8(*ver) == _abi.PA_OK
    # the fp8 unified launch takes the verify entry's argument list and its checks, plus the
    # scales array: every other pointer given, scales NULL
    uni = [p, p, p, None, p, 1, p, p, 2, 4, 8, 2, 128, 16, 0.1, p, 3, 0xF, p, 1, 4, p, 1 << 20,
           p, None]
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_ERR_NULL
    uni[3], uni[9] = p, 1                                 # 1 token for 2 sequences
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_ERR_SHAPE
    uni[9], uni[12] = 4, 96                               # head_dim 96
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_ERR_SHAPE
    uni[12], uni[13] = 128, 24                            # block size 24
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_ERR_BLOCK_SIZE
    uni[13], uni[21] = 16, None                           # partial rows without a workspace
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_ERR_NULL
    assert b"workspace" in L.pa_last_error()
    uni[21], uni[16] = p, 0                               # an empty table: a no-op
    assert L.paged_attn_varlen_prefill_fp8(*uni) == _abi.PA_OK
    v = [nul, nul, nul, nul, 1, nul, nul, 1, 1, 2, 1, 64, 16, 0.1, 1, nul, 1, 1, nul, 0, 0, nul,
         0, nul, nul]
    assert L.paged_attn_varlen_prefill(*v) == _abi.PA_ERR_DTYPE                  # fp32 prefill


def test_attention_entries_refuse_task_kinds_they_do_not_run():
    """Each attention entry takes the table's kind mask and refuses, before any HIP call, a
    table holding a kind its kernel would skip (those rows of `out` would stay unwritten). An
    accepted mask gets past that check and stops at the NULL pointer left in each call, so no
    kernel is launched here."""
    L = _abi.lib()
    p = ctypes.c_void_p(256)
    DEC, PRE, VER, SHA = (1 << _abi.PA_TASK_DECODE, 1 << _abi.PA_TASK_PREFILL,
                          1 << _abi.PA_TASK_VERIFY, 1 << _abi.PA_TASK_SHARED)

    def decode(kinds):      # context_lens NULL
        return L.paged_attn_decode(p, p, p, p, 1, None, 1, 2, 1, 64, 16, 0.1, 0, p, 1, kinds, p,
                                   1, 8, p, 1 << 20, p, None)

    def decode_fp8(kinds):  # context_lens NULL
        return L.paged_attn_decode_fp8(p, p, p, p, p, 1, None, 1, 2, 1, 64, 16, 0.1, p, 1,
                                       kinds, p, 1, 8, p, 1 << 20, p, None)

    def verify_fp8(kinds):  # cu_seqlens NULL
        return L.paged_attn_verify_fp8(p, p, p, p, p, 1, None, p, 2, 4, 8, 2, 128, 16, 0.1, p,
                                       3, kinds, p, 1, 4, p, 1 << 20, p, None)

    def varlen(kinds):      # context_lens NULL
        return L.paged_attn_varlen_prefill(p, p, p, p, 1, p, None, 1, 2, 2, 1, 64, 16, 0.1, 0, p,
                                           1, kinds, p, 1, 8, p, 1 << 20, p, None)

    def varlen_fp8(kinds):  # context_lens NULL
        return L.paged_attn_varlen_prefill_fp8(p, p, p, p, p, 1, p, None, 1, 2, 2, 1, 64, 16, 0.1,
                                               p, 1, kinds, p, 1, 8, p, 1 << 20, p, None)

    cases = [(decode, DEC | SHA), (decode_fp8, DEC | SHA), (verify_fp8, DEC | VER),
             (varlen, DEC | PRE | VER | SHA), (varlen_fp8, DEC | PRE | VER | SHA)]
    for fn, allowed in cases:
        for kinds in range(1, 16):
            rc = fn(kinds)
            if kinds & ~allowed:
                assert rc == _abi.PA_ERR_INPUT, (fn.__name__, kinds)
                assert b"task kinds" in L.pa_last_error()
            else:
                assert rc == _abi.PA_ERR_NULL, (fn.__name__, kinds)
        assert fn(0) == _abi.PA_ERR_INPUT                     # no mask for a non-empty table
        assert fn(1 << 7) == _abi.PA_ERR_INPUT                # not a kind
    # a real table: a prefill chunk among decode rows cannot go through the decode entry
    t = pa.build_task_table(pa.make_params(8, 2, 64, 16), pa.pack_seqlens([1, 40, 1]),
                            np.array([70, 100, 5], np.int32))
    assert t.kinds == DEC | PRE
    assert decode(t.kinds) == _abi.PA_ERR_INPUT
    assert varlen(t.kinds) == _abi.PA_ERR_NULL
    # verify rows need the verify entry (or the unified one), not the fp8 decode entry
    t = pa.build_task_table(pa.make_params(8, 2, 64, 16, verify_rows=4),
                            pa.pack_seqlens([1, 3]), np.array([70, 100], np.int32))
    assert t.kinds == DEC | VER
    assert decode_fp8(t.kinds) == _abi.PA_ERR_INPUT
    assert verify_fp8(t.kinds) == _abi.PA_ERR_NULL


def test_noalloc_entry_checks_need_no_gpu():
    """The allocation-free unified entry refuses, before any HIP call, a table whose partial
    rows exceed its fixed scratch, and shares the unified entry's other checks."""
    L = _abi.lib()
    p = ctypes.c_void_p(256)
    fn = L.paged_attn_varlen_prefill_noalloc
    # 200000 partial rows at D = 128 need ~104 MB > 64 MiB of scratch
    big = 200000
    assert pa.workspace_bytes(big, 128) > _abi.NOALLOC_SCRATCH_BYTES
    rc = fn(p, p, p, p, 1, p, p, 1, 2, 8, 2, 128, 16, 0.1, 0, p, 1, 1, p, 1, big, p, None)
    assert rc == _abi.PA_ERR_CAPACITY
    assert b"paged_attn_varlen_prefill with a workspace" in L.pa_last_error()
    # at the limit the size check passes and the NULL context_lens is what stops the call
    fit = (_abi.NOALLOC_SCRATCH_BYTES - 256) // (4 * 130)
    assert pa.workspace_bytes(fit, 128) <= _abi.NOALLOC_SCRATCH_BYTES
    rc = fn(p, p, p, p, 1, p, None, 1, 2, 8, 2, 128, 16, 0.1, 0, p, 1, 1, p, 1, fit, p, None)
    assert rc == _abi.PA_ERR_NULL
    # the unified entry's own checks: dtype, kinds, token count; an empty table is a no-op
    assert fn(p, p, p, p, 1, p, p, 1, 2, 8, 2, 128, 16, 0.1, 1, p, 1, 1, p, 1, 8, p,
              None) == _abi.PA_ERR_DTYPE
    assert fn(p, p, p, p, 1, p, p, 1, 2, 8, 2, 128, 16, 0.1, 0, p, 1, 0, p, 1, 8, p,
              None) == _abi.PA_ERR_INPUT
    assert fn(p, p, p, p, 1, p, p, 3, 2, 8, 2, 128, 16, 0.1, 0, p, 1, 1, p, 1, 8, p,
              None) == _abi.PA_ERR_SHAPE
    assert fn(None, None, None, None, 1, None, None, 1, 1, 8, 2, 128, 16, 0.1, 0, None, 0, 0,
              None, 0, 0, None, None) == _abi.PA_OK


def test_binding_refuses_host_tensors():
    import torch
    k = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    pages = torch.zeros(4, 1, 16, 64, dtype=torch.bfloat16)
    i = torch.zeros(2, 1, dtype=torch.int32)
    with pytest.raises(ValueError):
        pa.reshape_and_cache(k, k, pages, pages, i, torch.zeros(3, dtype=torch.int32),
                             torch.zeros(2, dtype=torch.int32))


def test_step_plan_decode_refuses_non_decode_tables():
    """The decode entry points run decode tasks only: a plan with a multi-row sequence or with
    verify rows must go through varlen instead (checked before any device call)."""
    import torch
    table = np.array([[0, 1], [2, 3]], dtype=np.int32)
    q = torch.zeros(1)
    for q_lens, extra in (([2, 1], {}), ([1, 1], {"verify_rows": 2})):
        plan = pa.StepPlan(q_lens, [20, 17], table, 8, 2, 128, 16, device="cpu", **extra)
        with pytest.raises(ValueError, match="decode tasks only"):
            plan.decode(q, q, q, 0.1, q)
        with pytest.raises(ValueError, match="decode tasks only"):
            plan.decode_fp8(q, q, q, q, q, 0.1, q)


# ---- shared-prefix tables (build_task_table_shared) against the oracle ----

def compare_shared(q_lens, ctx, bt, **kw):
    hq, hkv, d, bs = kw.pop("hq"), kw.pop("hkv"), kw.pop("d", 128), kw.pop("bs")
    cu = pa.pack_seqlens(q_lens)
    got = pa.build_task_table(pa.make_params(hq, hkv, d, bs, **kw), cu, ctx, block_table=bt)
    ref_t, ref_c, ref_np, _, ref_bal = ot.build_task_table(ot.Params(hq, hkv, d, bs, **kw), cu,
                                                           ctx, bt)
    assert np.array_equal(got.tasks, ref_t)
    assert np.array_equal(got.combines, ref_c)
    assert got.num_partials == ref_np
    assert got.balance_snake == ref_bal["snake"]
    assert got.balance_modulo == ref_bal["modulo"]
    assert got.kinds == kind_mask(ref_t)
    return got


@pytest.mark.parametrize("seed", range(10))
def test_shared_table_bit_exact_random(seed):
    rng = np.random.default_rng(300 + seed)
    bs = int(rng.choice([16, 32, 64]))
    q, ctx, bt = aliased_batch(rng, bs, int(rng.integers(1, 9)))
    hkv = int(rng.choice([1, 2, 4]))
    got = compare_shared(q, ctx, bt, hq=hkv * int(rng.choice([1, 2, 4, 8, 16])), hkv=hkv, bs=bs,
                         dec_split=64 * int(rng.integers(1, 4)), pf_q_tile=int(rng.integers(1, 9)),
                         num_workers=int(rng.integers(1, 40)), decode_weight=int(rng.integers(1, 3)),
                         verify_rows=int(rng.choice([0, 4])),
                         shared_min=64 * int(rng.integers(0, 4)))
    assert got.tasks.shape[0] > 0


def test_shared_table_bit_exact_on_workload():
    w = synth.make_workload("decode_shared_mha_bf16")
    got = compare_shared(w.q_lens, w.ctx_lens, w.block_table, hq=32, hkv=32, bs=16,
                         dec_split=1024, num_workers=512, shared_min=64)
    kinds = set(got.tasks[:, 0].tolist())
    assert kinds == {_abi.PA_TASK_DECODE, _abi.PA_TASK_SHARED}
    # one shared pass per (group, kv head, piece): 8 groups of 16 members, one column set each
    shared = got.tasks[got.tasks[:, 0] == _abi.PA_TASK_SHARED]
    assert set(shared[:, 4].tolist()) == {16}
    # the shared length is the prefix rounded down to a multiple of 64
    assert len(shared) == 32 * sum(-(-(p // 64 * 64) // 1024) for p in w.extra["prefix_lens"])


def test_shared_table_errors():
    bt = np.array([[0, 1, 2, 3, 4, 5, 6, -1], [0, 1, 2, 3, 4, 7, 8, -1]], dtype=np.int32)
    cu = np.array([0, 1, 2], np.int32)
    ctx = np.array([100, 90], np.int32)
    with pytest.raises(pa.PagedAttnError) as e:           # sharing needs the table
        pa.build_task_table(pa.make_params(2, 1, 64, 16, shared_min=64), cu, ctx)
    assert e.value.code == _abi.PA_ERR_INPUT
    with pytest.raises(pa.PagedAttnError) as e:           # not a multiple of 64
        pa.build_task_table(pa.make_params(2, 1, 64, 16, shared_min=32), cu, ctx, block_table=bt)
    assert e.value.code == _abi.PA_ERR_SHAPE
    with pytest.raises(pa.PagedAttnError) as e:           # a shared block receives a new row
        pa.build_task_table(pa.make_params(2, 1, 64, 16, shared_min=64), cu,
                            np.array([40, 48], np.int32), block_table=bt[:, :3].copy() * 0 +
                            np.array([0, 1, 2], np.int32))
    assert e.value.code == _abi.PA_ERR_INPUT
    with pytest.raises(pa.PagedAttnError) as e:           # table narrower than a context needs
        pa.build_task_table(pa.make_params(2, 1, 64, 16, shared_min=64), cu,
                            np.array([100, 200], np.int32), block_table=bt)
    assert e.value.code == _abi.PA_ERR_SHAPE
    L = pa.lib()
    nt, nc, npart = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    p = pa.make_params(2, 1, 64, 16, shared_min=64)
    rc = L.build_task_table_shared(ctypes.byref(p), cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   ctx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), 2, None, 8,
                                   None, 0, ctypes.byref(nt), None, 0, ctypes.byref(nc),
                                   ctypes.byref(npart), None, None)
    assert rc == _abi.PA_ERR_NULL
    # shared_min 0: the plain table, block table or not
    plain = pa.build_task_table(pa.make_params(2, 1, 64, 16), cu, ctx)
    off = pa.build_task_table(pa.make_params(2, 1, 64, 16), cu, ctx, block_table=bt)
    assert np.array_equal(plain.tasks, off.tasks) and np.array_equal(plain.combines, off.combines)
