"""Oracle for the Dynamic Decomposer's task table -- test infrastructure only.

XY-Serve page, section 2.2 ("Token 级调度与任务分解", "任务重排机制") and section 4.4
("实现动态分解器"): split each sequence's attention into fixed-size tasks that record their actual
shape and a compute load, sort the tasks by load from large to small, and report the balance
ratio min/max of per-core load sums when the sorted tasks are dealt to the cores.

Readings taken where the pages leave the step open:
  * decode sequences (one query row) are split along the keys into pieces of ``dec_split``; one
    task covers all query heads of one kv head (grouped-query heads share the KV pages);
  * short multi-row sequences (a draft being verified; the XY-Serve page's Meta-Attention serves
    prefill, decode and verify alike) are split the same way when ``verify_rows`` allows it
    (2 <= q_len <= verify_rows and G * q_len <= 16): one task covers all their rows and the G
    query heads of one kv head, with the causal mask inside the task;
  * prefill rows are tiled by ``pf_q_tile`` per query head, and each tile's visible key range
    (causal, bottom-right aligned) is split into pieces of ``pf_kv_split`` (0 = no split);
  * tiles with no visible key are never emitted; every emitted split holds at least one key
    for the tile's last row;
  * a task's load is the number of unmasked (query row, key) pairs times the heads it covers,
    an integer (the pages use q*kv in section 2.2 and q*kv*heads in section 4.4); decode loads
    may be multiplied by an integer ``decode_weight`` so bandwidth-bound and compute-bound tasks
    can be weighed against each other;
  * the sort is stable and descending (the pages' sorted(..., reverse=True) keeps ties in
    emission order: sequence, head, query tile, key split);
  * a group of tasks that share output rows and have more than one split gets partial-result
    rows numbered in emission order, plus one combine record; single-split tasks write the
    output directly (partial = -1);
  * the page's own code deals sorted tasks with i % num_cores while its prose says
    "symmetric round robin"; both balance ratios are reported.

Records (8 int32 each):
  task    = (kind, seq, head, q_row0, q_rows, kv0, kv1, partial)
            kind 0 = decode split, head = kv head (covers query heads head*G .. head*G+G-1)
            kind 1 = prefill tile, head = query head
            kind 2 = verify split, head = kv head, q_rows = the sequence's rows, q_row0 = 0
  combine = (seq, q_row0, q_rows, head, heads, first_slot, n_slots, 0)
            partial row of split k, query row i, head j = first_slot + k*q_rows*heads + i*heads + j
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ERR_SHAPE = -2
ERR_BLOCK_SIZE = -3
ERR_INPUT = -6


class TaskTableError(ValueError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


@dataclass
class Params:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dec_split: int = 512
    pf_q_tile: int = 128
    pf_kv_split: int = 0
    num_workers: int = 256
    decode_weight: int = 1
    verify_rows: int = 0


def _check(p: Params, cu, ctx):
    if p.num_q_heads < 1 or p.num_kv_heads < 1 or p.num_q_heads % p.num_kv_heads:
        raise TaskTableError(ERR_SHAPE, "query heads must be a positive multiple of kv heads")
    bs = p.block_size
    if bs < 16 or bs > 256 or (bs & (bs - 1)):
        # cann-recipes-infer page, section 5.3: page size must be a power of two >= 16
        raise TaskTableError(ERR_BLOCK_SIZE, "block size must be a power of two in [16, 256]")
    if p.dec_split < 64 or p.dec_split % 64:
        raise TaskTableError(ERR_SHAPE, "dec_split must be a positive multiple of 64")
    if not 1 <= p.pf_q_tile <= 128:
        raise TaskTableError(ERR_SHAPE, "pf_q_tile must lie in [1, 128]")
    if p.pf_kv_split < 0 or p.pf_kv_split % 64:
        raise TaskTableError(ERR_SHAPE, "pf_kv_split must be 0 or a positive multiple of 64")
    if p.num_workers < 1 or p.decode_weight < 1:
        raise TaskTableError(ERR_SHAPE, "num_workers and decode_weight must be >= 1")
    if p.verify_rows != 0 and not 2 <= p.verify_rows <= 16:
        raise TaskTableError(ERR_SHAPE, "verify_rows must be 0 or lie in [2, 16]")
    # cann-recipes-infer page, section 4.4: offsets start at 0 and increase strictly
    if len(cu) != len(ctx) + 1 or cu[0] != 0:
        raise TaskTableError(ERR_INPUT, "cu_seqlens must have N+1 entries starting at 0")
    for s in range(len(ctx)):
        if cu[s + 1] <= cu[s]:
            raise TaskTableError(ERR_INPUT, "cu_seqlens must increase strictly")
        if ctx[s] < cu[s + 1] - cu[s]:
            raise TaskTableError(ERR_INPUT, "context shorter than the new query rows")


def _ceil_div(a, b):
    return -(-a // b)


def build_task_table(p: Params, cu_seqlens_q, context_lens):
    """Return (tasks int32 [n, 8], combines int32 [m, 8], num_partials, loads int64 [n],
    balance dict {"snake", "modulo"})."""
    cu = [int(x) for x in cu_seqlens_q]
    ctx = [int(x) for x in context_lens]
    _check(p, cu, ctx)
    G = p.num_q_heads // p.num_kv_heads
    emitted = []          # (load, task) in emission order
    combines = []
    num_partials = 0
    for s in range(len(ctx)):
        ql = cu[s + 1] - cu[s]
        prefix = ctx[s] - ql
        verify = 2 <= ql <= p.verify_rows and G * ql <= 16
        if ql == 1 or verify:
            kind = 2 if verify else 0
            nsplit = _ceil_div(ctx[s], p.dec_split)
            for g in range(p.num_kv_heads):
                first = -1
                if nsplit > 1:
                    first = num_partials
                    num_partials += nsplit * ql * G
                    combines.append((s, 0, ql, g * G, G, first, nsplit, 0))
                for k in range(nsplit):
                    kv0 = k * p.dec_split
                    kv1 = min(ctx[s], kv0 + p.dec_split)
                    part = first + k * ql * G if nsplit > 1 else -1
                    pairs = 0
                    for i in range(ql):
                        pairs += max(0, min(kv1, prefix + i + 1) - kv0)
                    load = pairs * G * p.decode_weight
                    emitted.append((load, (kind, s, g, 0, ql, kv0, kv1, part)))
        else:
            for h in range(p.num_q_heads):
                for r0 in range(0, ql, p.pf_q_tile):
                    rows = min(p.pf_q_tile, ql - r0)
                    lim = prefix + r0 + rows          # keys visible to the tile's last row
                    split = p.pf_kv_split if p.pf_kv_split > 0 else lim
                    nsplit = _ceil_div(lim, split)
                    first = -1
                    if nsplit > 1:
                        first = num_partials
                        num_partials += nsplit * rows
                        combines.append((s, r0, rows, h, 1, first, nsplit, 0))
                    for k in range(nsplit):
                        kv0 = k * split
                        kv1 = min(lim, kv0 + split)
                        load = 0
                        for i in range(r0, r0 + rows):
                            load += max(0, min(kv1, prefix + i + 1) - kv0)
                        part = first + k * rows if nsplit > 1 else -1
                        emitted.append((load, (1, s, h, r0, rows, kv0, kv1, part)))
    # stable sort, load descending (ties keep emission order)
    order = sorted(range(len(emitted)), key=lambda i: -emitted[i][0])
    tasks = np.array([emitted[i][1] for i in order], dtype=np.int32).reshape(-1, 8)
    loads = np.array([emitted[i][0] for i in order], dtype=np.int64)
    comb = np.array(combines, dtype=np.int32).reshape(-1, 8)
    W = p.num_workers
    snake = [0] * W
    modulo = [0] * W
    for i, ld in enumerate(loads):
        rnd, pos = divmod(i, W)
        snake[pos if rnd % 2 == 0 else W - 1 - pos] += int(ld)
        modulo[i % W] += int(ld)

    def ratio(v):
        return 1.0 if max(v) == 0 else min(v) / max(v)

    return tasks, comb, num_partials, loads, {"snake": ratio(snake), "modulo": ratio(modulo)}
