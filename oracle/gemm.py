"""Oracle for SmoothGEMM, the dynamic-shape matrix product with virtual padding -- test
infrastructure only.

XY-Serve page, section 2.2 ("SmoothGEMM"): a product of arbitrary M, N, K computed in fixed
blocks, where a block at the matrix edge loads and stores only the valid part of its region
(no padded copies in memory; the invalid part is skipped by masking); section 4.4
(``decompose_linear``): the output is cut into M x N blocks, the reduction dimension into K
blocks, each task records its actual shape and a load of actual_m * actual_n * actual_k, and the
tasks are sorted by load, largest first, like the attention tasks.

Readings taken where the page leaves the step open:
  * the product is C = A W^T with A [M, K] and W [N, K] (a Linear layer's weight layout, both
    operands contiguous along K), bf16 inputs, fp32 accumulation, C rounded to bf16;
  * output blocks are square tiles of ``tile`` rows and columns (128 or 256); the K axis is cut
    into pieces of ``k_split`` (0 = all of K, else a positive multiple of 64);
  * the page chains the K blocks of one output block by a dependency; here they are
    independent tasks that write fp32 partial tiles, merged afterwards by one reduce record per
    output block (the sum is the same; only the summation order differs);
  * emission order m block, n block, k block (the page's loops); a stable sort by load,
    descending; tasks of an output block with one K piece write C directly (slot -1);
  * partial slots are numbered in emission order, one full tile each;
  * tail pieces (``tail_split`` = 1, with ``k_split`` = 0): the page sizes blocks so that the
    sorted tasks keep every worker busy. With T output blocks and W workers, the blocks that
    fill the last, partial round (the last r = T mod W of the load-sorted whole blocks; all of
    them when T < W) are cut into p = min(W // r, ceil(K / 64)) K pieces when p >= 2, each piece
    ceil(K / p) rounded up to a multiple of 64 (the last one takes the rest), so the last round
    holds up to W shorter tasks instead of r whole ones.

Records (8 int32 each):
  task   = (m0, rows, n0, cols, k0, k1, slot, 0)
  reduce = (m0, rows, n0, cols, first_slot, n_slots, 0, 0)
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

ERR_SHAPE = -2


class GemmTableError(ValueError):
    def __init__(self, code, msg):
        super().__init__(msg)
        self.code = code


@dataclass
class GemmParams:
    tile: int = 256
    k_split: int = 0
    num_workers: int = 256
    tail_split: int = 0


def matmul(a, w):
    """C = A W^T in float64 (the definition the kernels approximate)."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def _ceil_div(a, b):
    return -(-a // b)


def decompose_linear(p: GemmParams, M: int, N: int, K: int):
    """Return (tasks int32 [n, 8], reduces int32 [m, 8], num_slots, loads int64 [n],
    balance dict {"snake", "modulo"})."""
    if p.tile not in (128, 256):
        raise GemmTableError(ERR_SHAPE, "tile must be 128 or 256")
    if p.k_split < 0 or p.k_split % 64:
        raise GemmTableError(ERR_SHAPE, "k_split must be 0 or a positive multiple of 64")
    if p.num_workers < 1:
        raise GemmTableError(ERR_SHAPE, "num_workers must be >= 1")
    if p.tail_split not in (0, 1) or (p.tail_split and p.k_split):
        raise GemmTableError(ERR_SHAPE, "tail_split must be 0, or 1 with k_split 0")
    if M < 0 or N < 0 or K < 0:
        raise GemmTableError(ERR_SHAPE, "negative size")
    if K == 0 and M > 0 and N > 0:
        raise GemmTableError(ERR_SHAPE, "K must be >= 1 for a non-empty product")
    # output blocks in emission order, and the K piece length of each
    blocks = [(m0, min(p.tile, M - m0), n0, min(p.tile, N - n0))
              for m0 in range(0, M, p.tile) for n0 in range(0, N, p.tile)]
    split = [p.k_split if p.k_split > 0 else max(K, 1)] * len(blocks)
    if p.tail_split and blocks and K > 0:
        T, W = len(blocks), p.num_workers
        r = T % W
        pieces = min(W // r, _ceil_div(K, 64)) if r else 1
        if pieces >= 2:
            kp = _ceil_div(_ceil_div(K, pieces), 64) * 64
            whole = sorted(range(T), key=lambda i: -(blocks[i][1] * blocks[i][3]))
            for i in whole[T - r:]:
                split[i] = kp
    emitted, reduces = [], []
    slots = 0
    for b, (m0, rows, n0, cols) in enumerate(blocks):
        nk = _ceil_div(K, split[b]) if K > 0 else 0
        first = -1
        if nk > 1:
            first = slots
            slots += nk
            reduces.append((m0, rows, n0, cols, first, nk, 0, 0))
        for j in range(nk):
            k0 = j * split[b]
            k1 = min(K, k0 + split[b])
            slot = first + j if nk > 1 else -1
            emitted.append((rows * cols * (k1 - k0), (m0, rows, n0, cols, k0, k1, slot, 0)))
    order = sorted(range(len(emitted)), key=lambda i: -emitted[i][0])
    tasks = np.array([emitted[i][1] for i in order], dtype=np.int32).reshape(-1, 8)
    loads = np.array([emitted[i][0] for i in order], dtype=np.int64)
    red = np.array(reduces, dtype=np.int32).reshape(-1, 8)
    W = p.num_workers
    snake, modulo = [0] * W, [0] * W
    for i, ld in enumerate(loads):
        rnd, pos = divmod(i, W)
        snake[pos if rnd % 2 == 0 else W - 1 - pos] += int(ld)
        modulo[i % W] += int(ld)

    def ratio(v):
        return 1.0 if max(v) == 0 else min(v) / max(v)

    return tasks, red, slots, loads, {"snake": ratio(snake), "modulo": ratio(modulo)}
