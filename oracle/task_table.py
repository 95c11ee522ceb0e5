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

Shared prefixes (XY-Serve page, "自动前缀缓存": requests that repeat a prompt prefix reuse its
cached keys and values; ATB page, "KV缓存复用": a later turn reuses the blocks of the earlier
ones). When the block table makes several sequences point at the same physical blocks, the
attention over those keys can read them once for all of them. Readings:
  * sharing is looked for between neighbouring decode sequences (q_len 1) in batch order, and
    only when ``shared_min`` > 0 and a task's 16 columns hold at least two sequences
    (G <= 8); the host has a copy of the block table;
  * two neighbours share the leading logical blocks whose physical ids are equal (among the
    blocks both need); a block that receives either one's new row this step must not be
    shared (an input error); their shared keys are those blocks' keys, rounded down to a
    multiple of 64;
  * a group is a maximal run of neighbours that share at least ``shared_min`` keys pairwise;
    the group's shared length L is the smallest pairwise value (equal ids are transitive);
  * a group is cut into ceil(n / (16 // G)) column sets of consecutive members with sizes as
    equal as possible (the first n % sets one larger);
  * per kv head and column set: [0, L) in pieces of ``dec_split`` as shared tasks whose
    columns are (member, query head) pairs, and each member's own keys [L, ctx) in pieces of
    ``dec_split`` as decode tasks; every member's row merges all its pieces, so each member
    gets partial rows and one combine record even with a single piece;
  * partial rows of a column set: member i owns W = (S + max U) * G rows from base + i*W
    (S shared pieces, U_i own pieces), piece k's rows at + k*G; a shared task's partial field
    is base + k*G and its q_row0 field holds the member stride W; rows past S + U_i of a
    member with fewer own pieces stay unused;
  * a shared task's load is keys x members x G (pairs x heads, as for every task).

Records (8 int32 each):
  task    = (kind, seq, head, q_row0, q_rows, kv0, kv1, partial)
            kind 0 = decode split, head = kv head (covers query heads head*G .. head*G+G-1)
            kind 1 = prefill tile, head = query head
            kind 2 = verify split, head = kv head, q_rows = the sequence's rows, q_row0 = 0
            kind 3 = shared-prefix split, seq = first member, q_rows = members (consecutive
                     decode sequences), q_row0 = member stride W of its partial rows
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
    shared_min: int = 0


def _check(p: Params, cu, ctx):
    if p.num_q_heads < 1 or p.num_kv_heads < 1 or p.num_q_heads % p.num_kv_heads:
        raise TaskTableError(ERR_SHAPE, "query heads must be a positive multiple of kv heads")
    bs = p.block_size
    if bs < 16 or bs > 256 or (bs & (bs - 1)):
        # cann-recipes-infer page, section 5.3: page size must be a power of two >= 16
        raise TaskTableError(ERR_BLOCK_SIZE, "block size must be a power of two in [16, 256]")
    if p.dec_split < 64 or p.dec_split % 64:
        raise TaskTableError(ERR_SHAPE, "dec_split must be a positive multiple of 64")
    # any positive tile height decomposes the rows; how many rows one kernel task can hold is
    # the library's limit, checked by its own table builder
    if p.pf_q_tile < 1:
        raise TaskTableError(ERR_SHAPE, "pf_q_tile must be positive")
    if p.pf_kv_split < 0 or p.pf_kv_split % 64:
        raise TaskTableError(ERR_SHAPE, "pf_kv_split must be 0 or a positive multiple of 64")
    if p.num_workers < 1 or p.decode_weight < 1:
        raise TaskTableError(ERR_SHAPE, "num_workers and decode_weight must be >= 1")
    if p.verify_rows != 0 and not 2 <= p.verify_rows <= 16:
        raise TaskTableError(ERR_SHAPE, "verify_rows must be 0 or lie in [2, 16]")
    if p.shared_min < 0 or p.shared_min % 64:
        raise TaskTableError(ERR_SHAPE, "shared_min must be 0 or a positive multiple of 64")
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


def shared_keys_with_previous(p: Params, cu, ctx, block_table):
    """pair[s] for s >= 1: keys that decode sequences s-1 and s both read from the same physical
    blocks, rounded down to a multiple of 64 (0 when either is not a decode row)."""
    bs = p.block_size
    pair = [0] * len(ctx)
    for s in range(1, len(ctx)):
        if cu[s + 1] - cu[s] != 1 or cu[s] - cu[s - 1] != 1:
            continue
        need = min(_ceil_div(ctx[s - 1], bs), _ceil_div(ctx[s], bs))
        common = 0
        while common < need and int(block_table[s - 1][common]) == int(block_table[s][common]):
            common += 1
        # logical block (ctx-1)//bs receives the sequence's new row in this step
        if common > min((ctx[s - 1] - 1) // bs, (ctx[s] - 1) // bs):
            raise TaskTableError(ERR_INPUT, f"sequences {s - 1} and {s} share a block that "
                                 "receives a new row")
        pair[s] = common * bs // 64 * 64
    return pair


def build_task_table(p: Params, cu_seqlens_q, context_lens, block_table=None):
    """Return (tasks int32 [n, 8], combines int32 [m, 8], num_partials, loads int64 [n],
    balance dict {"snake", "modulo"}). ``block_table`` (host, [N, max_blocks]) is needed only
    when ``p.shared_min`` > 0."""
    cu = [int(x) for x in cu_seqlens_q]
    ctx = [int(x) for x in context_lens]
    _check(p, cu, ctx)
    G = p.num_q_heads // p.num_kv_heads
    emitted = []          # (load, task) in emission order
    combines = []
    num_partials = 0
    columns = 16 // G     # sequences per shared task
    pair = [0] * len(ctx)
    if p.shared_min > 0:
        if block_table is None:
            raise TaskTableError(ERR_INPUT, "shared_min > 0 needs the block table")
        for s in range(len(ctx)):
            if _ceil_div(ctx[s], p.block_size) > len(block_table[s]):
                raise TaskTableError(ERR_SHAPE, "block table narrower than a context needs")
        pair = shared_keys_with_previous(p, cu, ctx, block_table)
    ds, w = p.dec_split, p.decode_weight
    s = 0
    while s < len(ctx):
        end = s
        if p.shared_min > 0 and columns >= 2:
            while end + 1 < len(ctx) and pair[end + 1] >= p.shared_min:
                end += 1
        if end > s:
            # a shared-prefix group: members s .. end
            L = min(pair[s + 1:end + 1])
            n = end - s + 1
            nsets = _ceil_div(n, columns)
            sizes = [n // nsets + (1 if i < n % nsets else 0) for i in range(nsets)]
            S = _ceil_div(L, ds)
            for g in range(p.num_kv_heads):
                m0 = s
                for size in sizes:
                    members = list(range(m0, m0 + size))
                    U = [_ceil_div(ctx[m] - L, ds) for m in members]
                    W = (S + max(U)) * G
                    base = num_partials
                    num_partials += size * W
                    for i, m in enumerate(members):
                        combines.append((m, 0, 1, g * G, G, base + i * W, S + U[i], 0))
                    for k in range(S):
                        kv0 = k * ds
                        kv1 = min(L, kv0 + ds)
                        emitted.append(((kv1 - kv0) * size * G * w,
                                        (3, m0, g, W, size, kv0, kv1, base + k * G)))
                    for i, m in enumerate(members):
                        for j in range(U[i]):
                            kv0 = L + j * ds
                            kv1 = min(ctx[m], kv0 + ds)
                            emitted.append(((kv1 - kv0) * G * w,
                                            (0, m, g, 0, 1, kv0, kv1,
                                             base + i * W + (S + j) * G)))
                    m0 += size
            s = end + 1
            continue
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
        s += 1
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
