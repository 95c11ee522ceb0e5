"""fp64 oracle for attention over a block-paged KV cache on packed variable-length sequences.

Test infrastructure only (see the package docstring).

Notation follows the pages:
  * packed queries q [T, Hq, D]; sequence s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1
    (cann-recipes-infer Paged KV / Packed Sequence page, section 2.3, "Packed Sequence");
  * pages [num_blocks, Hkv, block_size, D] and a per-sequence block table mapping logical block
    j to a physical block (same page, sections 2.2 and 3.1);
  * attention is GEMM -> softmax -> GEMM over the sequence's own keys (XY-Serve page, section 2.2,
    "Meta-Attention"), causal (cann-recipes-infer page, section 3.3, is_causal=True).

Readings where the pages are silent:
  * context_lens[s] counts the keys visible after this step's cache writes, so the cached prefix
    is P_s = context_lens[s] - q_len_s;
  * causal alignment is bottom-right: query row i of a chunk sits at absolute position P_s + i
    and sees keys 0 .. P_s + i (for a one-token decode that is every key);
  * grouped-query heads: query head h reads kv head h // (Hq // Hkv);
  * softmax is the plain max-subtracted exponential over the visible keys, no dropout.
"""
from __future__ import annotations

import numpy as np


def pack_lengths(lengths) -> np.ndarray:
    """Cumulative offsets of packed sequences: [0, l0, l0+l1, ...].

    cann-recipes-infer page, section 2.3: three sequences of lengths [128, 64, 256] pack into one
    buffer of 448 rows with offsets [0, 128, 192, 448]. Offsets must start at 0 and increase
    strictly (same page, section 4.4, second check), so every length must be >= 1.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.ndim != 1 or np.any(lengths < 1):
        raise ValueError("every packed sequence needs at least one row")
    cu = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    running = 0
    for s, n in enumerate(lengths):
        running += int(n)
        cu[s + 1] = running
    return cu


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks a context of ``num_tokens`` keys occupies: ceil(num_tokens / block_size).

    cann-recipes-infer page, section 2.2: 327 tokens in 16-token pages take 21 pages.
    """
    return -(-int(num_tokens) // int(block_size))


def gather_kv(k_pages, v_pages, block_table_row, ctx: int, block_size: int):
    """Logical K and V of one sequence, read through its block table.

    Key j lives in physical block block_table_row[j // block_size] at slot j % block_size
    (cann-recipes-infer page, section 2.2, "page table"). Only the first ceil(ctx / block_size)
    table entries are read; entries after them and slots past ctx are never touched.
    Returns fp64 arrays K, V of shape [ctx, Hkv, D].
    """
    hkv, d = k_pages.shape[1], k_pages.shape[3]
    K = np.empty((ctx, hkv, d), dtype=np.float64)
    V = np.empty((ctx, hkv, d), dtype=np.float64)
    for j in range(blocks_needed(ctx, block_size)):
        b = int(block_table_row[j])
        lo = j * block_size
        n = min(block_size, ctx - lo)
        # page layout [Hkv, block_size, D] -> rows [n, Hkv, D]
        K[lo:lo + n] = np.transpose(np.asarray(k_pages[b, :, :n, :], dtype=np.float64), (1, 0, 2))
        V[lo:lo + n] = np.transpose(np.asarray(v_pages[b, :, :n, :], dtype=np.float64), (1, 0, 2))
    return K, V


def attend_rows(q_rows, K, V, first_pos: int, scale: float):
    """Softmax attention of consecutive query rows of one head over one sequence's keys.

    q_rows [R, D] are the queries at absolute positions first_pos .. first_pos + R - 1; row r
    sees keys 0 .. first_pos + r. K, V are [ctx, D] for that head's kv head.
    z = scale * q . k_j ; w = exp(z - max z) ; out = sum_j w_j v_j / sum_j w_j.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    out = np.empty_like(q_rows)
    for r in range(q_rows.shape[0]):
        visible = first_pos + r + 1
        z = scale * (K[:visible] @ q_rows[r])
        w = np.exp(z - z.max())
        out[r] = (w @ V[:visible]) / w.sum()
    return out


def paged_attention(q, k_pages, v_pages, block_table, q_lens, context_lens, scale,
                    seqs=None, rows=None):
    """Packed, paged, causal, grouped-query attention in fp64.

    q            [T, Hq, D] packed queries (any float dtype; converted to fp64)
    k_pages      [NB, Hkv, bs, D]
    v_pages      [NB, Hkv, bs, D]
    block_table  [N, max_blocks] int
    q_lens       [N] new query rows per sequence
    context_lens [N] keys visible to the last row of each sequence
    scale        softmax scale (the configs pass 1/sqrt(D))
    seqs         optional subset of sequences to compute (others are left NaN)
    rows         optional {seq: list of row indices within the sequence} to compute

    Returns out [T, Hq, D] fp64 (rows not computed are NaN).
    """
    q = np.asarray(q)
    T, hq, d = q.shape
    hkv, bs = k_pages.shape[1], k_pages.shape[2]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    group = hq // hkv
    cu = pack_lengths(q_lens)
    if cu[-1] != T:
        raise ValueError("q rows do not match the sum of q_lens")
    out = np.full((T, hq, d), np.nan, dtype=np.float64)
    todo = range(len(q_lens)) if seqs is None else seqs
    for s in todo:
        ql, ctx = int(q_lens[s]), int(context_lens[s])
        prefix = ctx - ql
        if prefix < 0:
            raise ValueError("context shorter than the new query rows")
        K, V = gather_kv(k_pages, v_pages, block_table[s], ctx, bs)
        sel = list(range(ql)) if rows is None or s not in rows else list(rows[s])
        for h in range(hq):
            g = h // group
            for r in sel:
                t = int(cu[s]) + r
                out[t, h] = attend_rows(np.asarray(q[t, h], dtype=np.float64)[None, :],
                                        K[:, g, :], V[:, g, :], prefix + r, scale)[0]
    return out


def paged_attention_fast(q, k_pages, v_pages, block_table, q_lens, context_lens, scale,
                         seqs=None, row_chunk=256):
    """The same definition as ``paged_attention``, vectorised per (sequence, head) with a
    masked score matrix instead of a per-row loop. Used where the per-row loop is too slow;
    the CPU tests check that the two agree.
    """
    q = np.asarray(q)
    T, hq, d = q.shape
    hkv, bs = k_pages.shape[1], k_pages.shape[2]
    group = hq // hkv
    cu = pack_lengths(q_lens)
    out = np.full((T, hq, d), np.nan, dtype=np.float64)
    todo = range(len(q_lens)) if seqs is None else seqs
    for s in todo:
        ql, ctx = int(q_lens[s]), int(context_lens[s])
        prefix = ctx - ql
        K, V = gather_kv(k_pages, v_pages, block_table[s], ctx, bs)
        for h in range(hq):
            g = h // group
            for r0 in range(0, ql, row_chunk):
                r1 = min(ql, r0 + row_chunk)
                Q = np.asarray(q[cu[s] + r0:cu[s] + r1, h], dtype=np.float64)
                z = scale * (Q @ K[:, g, :].T)                       # [R, ctx]
                pos = prefix + np.arange(r0, r1)[:, None]
                z = np.where(np.arange(ctx)[None, :] <= pos, z, -np.inf)
                w = np.exp(z - z.max(axis=1, keepdims=True))
                out[cu[s] + r0:cu[s] + r1, h] = (w @ V[:, g, :]) / w.sum(axis=1, keepdims=True)
    return out
