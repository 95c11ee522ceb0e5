"""Seeded synthetic inputs for paged, variable-length attention.

This module only *draws* inputs: per-sequence query and context lengths, a shuffled pool of
physical blocks dealt into per-sequence block tables, and tensor values. It holds none of the
attention arithmetic (no packing into offsets, no gather, no softmax, no task decomposition), so
both the CPU oracle and the GPU path can consume what it returns without sharing any of the
method's code.

Workload shapes follow the pages' statement of the problem:
  * paged KV pool of fixed-size blocks with an int32 block table, -1 for unused entries
    (cann-recipes-infer Paged KV / Packed Sequence page, sections 2.2 and 3.1);
  * one query token per sequence for decode (MindIE page, "Continuous Batching");
  * 512-token prefill chunks over a cached prefix (MindIE page, "Prefill Chunking");
  * packed variable-length prompts (cann-recipes-infer page, section 2.3).
The pages' own datasets (ShareGPT-V3, an internal RAG trace) are not available; the length
distributions below stand in for them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_workload", "deal_block_table", "make_values",
           "make_fp8_pages", "custom_workload", "shared_prefix_workload", "GEMM_SHAPES",
           "gemm_shape", "make_gemm_operands"]


@dataclass
class Workload:
    """Shapes and integer inputs of one synthetic batch (no tensor values)."""
    name: str
    seed: int
    q_lens: np.ndarray          # int64 [N]  new query tokens per sequence
    ctx_lens: np.ndarray        # int64 [N]  keys visible after this step's cache writes
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                  # "bf16" or "fp32"
    block_table: np.ndarray     # int32 [N, max_blocks_per_seq], -1 = unused entry
    num_blocks: int             # physical blocks in the pool
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])


def deal_block_table(ctx_lens: np.ndarray, block_size: int, rng: np.random.Generator,
                     pool_blocks: int | None = None, min_width: int = 1):
    """Deal a seeded permutation of a block pool to each sequence's logical blocks, in order.

    Sequence s needs ceil(ctx_s / block_size) blocks. The pool holds ``pool_blocks`` physical
    blocks (default: exactly the total need). Entries past a sequence's need stay -1.
    Returns (block_table int32 [N, width], pool size).
    """
    need = [(int(c) + block_size - 1) // block_size for c in ctx_lens]
    total = int(sum(need))
    nb = total if pool_blocks is None else int(pool_blocks)
    if nb < total:
        raise ValueError("pool smaller than the blocks the contexts need")
    perm = rng.permutation(nb)
    width = max(max(need) if need else 1, min_width)
    table = np.full((len(need), width), -1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        table[s, :n] = perm[pos:pos + n]
        pos += n
    return table, nb


def _lengths(name: str, rng: np.random.Generator):
    """Per-config length draws. Returns (q_lens, ctx_lens, Hq, Hkv, D, bs, dtype, pool)."""
    if name == "tiny_decode_fp32":
        ctx = np.array([5, 17, 33, 64], dtype=np.int64)
        return np.ones(4, np.int64), ctx, 2, 2, 64, 16, "fp32", 16
    if name == "decode_mha_bf16":
        ctx = rng.integers(128, 4097, size=64).astype(np.int64)
        return np.ones(64, np.int64), ctx, 32, 32, 128, 16, "bf16", None
    if name in ("decode_gqa_bf16_bs16", "decode_gqa_bf16_bs64"):
        u = rng.uniform(math.log(64.0), math.log(32768.0), size=256)
        ctx = np.clip(np.floor(np.exp(u)), 64, 32768).astype(np.int64)
        bs = 16 if name.endswith("bs16") else 64
        return np.ones(256, np.int64), ctx, 32, 8, 128, bs, "bf16", None
    if name in ("prefill_varlen_bf16", "prefill_varlen_fp8"):
        # (the fp8 variant has the same lengths, over fp8 pages with per-page scales)
        comp = rng.choice(3, size=16, p=[0.6, 0.25, 0.15])
        lo = np.array([10, 1000, 10000])
        hi = np.array([50, 5000, 20000])
        lens = np.array([rng.integers(lo[c], hi[c] + 1) for c in comp], dtype=np.int64)
        return lens.copy(), lens.copy(), 32, 8, 128, 16, "bf16", None
    if name in ("mixed_bf16", "mixed_fp8"):
        # (the fp8 variant has the same lengths, over fp8 pages with per-page scales)
        dec_ctx = rng.integers(256, 32769, size=200).astype(np.int64)
        prefix = rng.integers(0, 131073, size=4).astype(np.int64)
        q = np.concatenate([np.ones(200, np.int64), np.full(4, 512, np.int64)])
        ctx = np.concatenate([dec_ctx, prefix + 512])
        return q, ctx, 64, 8, 128, 128, "bf16", None
    if name == "decode_mha_fp8":
        # the MHA decode batch (same lengths) over fp8 pages with per-page scales
        ctx = rng.integers(128, 4097, size=64).astype(np.int64)
        return np.ones(64, np.int64), ctx, 32, 32, 128, 16, "bf16", None
    if name in ("verify_gqa_bf16", "verify_gqa_fp8"):
        # the GQA decode batch with a 4-row draft per sequence (3 drafted tokens plus the last
        # accepted one) verified in one step; contexts include the draft rows (the fp8 variant
        # has the same lengths, over fp8 pages with per-page scales)
        u = rng.uniform(math.log(64.0), math.log(32768.0), size=256)
        ctx = np.clip(np.floor(np.exp(u)), 64, 32768).astype(np.int64)
        return np.full(256, 4, np.int64), ctx, 32, 8, 128, 16, "bf16", None
    raise KeyError(name)


# name -> seed; the GQA block-size pair shares a seed so both runs see identical lengths.
WORKLOADS = {
    "tiny_decode_fp32": 1,
    "decode_mha_bf16": 2,
    "decode_gqa_bf16_bs16": 3,
    "decode_gqa_bf16_bs64": 3,
    "prefill_varlen_bf16": 4,
    "prefill_varlen_fp8": 4,
    "mixed_bf16": 5,
    "mixed_fp8": 5,
    "verify_gqa_bf16": 6,
    "verify_gqa_fp8": 6,
    "decode_mha_fp8": 2,
    "decode_shared_mha_bf16": 7,
}


def make_workload(name: str, seed: int | None = None) -> Workload:
    """Build the integer side of a named synthetic workload (lengths + block table)."""
    seed = WORKLOADS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "decode_shared_mha_bf16":
        # agent-style serving: 8 prompts, each repeated by 16 requests that now decode; a prompt
        # of U[1024, 8192] keys (whole blocks) is cached once, and every request has
        # U[16, 512] keys of its own after it
        prefix = rng.integers(64, 513, size=8) * 16
        own = rng.integers(16, 513, size=(8, 16))
        return shared_prefix_workload(prefix, own, 32, 32, 128, 16, seed=seed, name=name,
                                      rng=rng)
    q, ctx, hq, hkv, d, bs, dt, pool = _lengths(name, rng)
    table, nb = deal_block_table(ctx, bs, rng, pool_blocks=pool)
    return Workload(name, seed, q, ctx, hq, hkv, d, bs, dt, table, nb)


def custom_workload(q_lens, ctx_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                    dtype="bf16", seed=0, spare_blocks=0, name="custom", min_width=1):
    """A workload with caller-chosen lengths; the block pool is shuffled with ``seed``."""
    rng = np.random.default_rng(seed)
    q = np.asarray(q_lens, dtype=np.int64)
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    need = int(sum((int(c) + block_size - 1) // block_size for c in ctx))
    table, nb = deal_block_table(ctx, block_size, rng, pool_blocks=need + spare_blocks,
                                 min_width=min_width)
    return Workload(name, seed, q, ctx, num_q_heads, num_kv_heads, head_dim, block_size,
                    dtype, table, nb)


def shared_prefix_workload(prefix_lens, own_lens, num_q_heads, num_kv_heads, head_dim,
                           block_size, dtype="bf16", seed=0, name="shared", rng=None,
                           spare_blocks=0):
    """Decode sequences in groups that share a cached prefix.

    Group g's first prefix_lens[g] keys (a multiple of block_size) sit in blocks that every
    member's table lists first; member m of group g then has own_lens[g][m] >= 1 keys of its
    own in private blocks (the last of them is the row this step writes). Groups are laid out
    one after another in batch order, members consecutively. Physical ids come from a seeded
    permutation of the pool.
    """
    rng = np.random.default_rng(seed) if rng is None else rng
    bs = block_size
    prefix = [int(x) for x in prefix_lens]
    own = [[int(x) for x in row] for row in own_lens]
    if any(x % bs for x in prefix) or any(x < 1 for row in own for x in row):
        raise ValueError("prefixes must be whole blocks and every member needs an own key")
    need = sum(x // bs for x in prefix) + sum((x + bs - 1) // bs for row in own for x in row)
    nb = need + spare_blocks
    perm = rng.permutation(nb)
    rows, ctx = [], []
    pos = 0
    for g, P in enumerate(prefix):
        shared = perm[pos:pos + P // bs].tolist()
        pos += P // bs
        for x in own[g]:
            k = (x + bs - 1) // bs
            rows.append(shared + perm[pos:pos + k].tolist())
            pos += k
            ctx.append(P + x)
    width = max(len(r) for r in rows)
    table = np.full((len(rows), width), -1, dtype=np.int32)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    q = np.ones(len(rows), dtype=np.int64)
    return Workload(name, seed, q, np.asarray(ctx, dtype=np.int64), num_q_heads, num_kv_heads,
                    head_dim, block_size, dtype, table, nb,
                    extra={"prefix_lens": prefix, "own_lens": own})


def make_values(w: Workload, device="cpu", seed: int | None = None, nan_sentinels=True):
    """Draw tensor values for a workload with a seeded torch generator.

    Returns a dict of torch tensors on ``device``:
      q      [T, Hq, D]           new queries, packed in sequence order
      k_new  [T, Hkv, D]          new keys for the same packed tokens
      v_new  [T, Hkv, D]
      k_pages, v_pages [NB, Hkv, bs, D]  the pool, holding the cached prefix of every sequence
    Values are N(0,1) drawn in fp32, then rounded to bf16 (round to nearest even) for bf16
    workloads. With ``nan_sentinels`` every slot that holds no cached key -- unused blocks, the
    tail of each sequence's last block, and the slots this step's new tokens will be written
    to -- is NaN, so a kernel that reads any of them, or skips a write, cannot go unnoticed.
    """
    import torch
    seed = w.seed if seed is None else seed
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    T, hq, hkv, d, bs, nb = w.num_tokens, w.num_q_heads, w.num_kv_heads, w.head_dim, \
        w.block_size, w.num_blocks

    def draw(*shape):
        return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(dt)

    q = draw(T, hq, d)
    k_new = draw(T, hkv, d)
    v_new = draw(T, hkv, d)
    k_pages = draw(nb, hkv, bs, d)
    v_pages = draw(nb, hkv, bs, d)
    if nan_sentinels:
        valid, _ = _cached_slots(w)
        mask = torch.from_numpy(~valid).to(device)
        # [NB, bs] mask over the [NB, bs] leading dims of the (block, slot, head, dim) view
        k_pages.transpose(1, 2)[mask] = float("nan")
        v_pages.transpose(1, 2)[mask] = float("nan")
    return dict(q=q, k_new=k_new, v_new=v_new, k_pages=k_pages, v_pages=v_pages)


def make_fp8_pages(w: Workload, device="cpu", seed: int | None = None, nan_sentinels=True):
    """Draw an fp8 page pool for a workload with a seeded torch generator on ``device``: uint8
    codes [NB, Hkv, bs, D] and float32 page scales [NB, Hkv, 2] (the K page's scale, then the
    V page's).

    Codes are uniform over the finite OCP E4M3FN codes (magnitude 0x00..0x7E, then a random
    sign bit), so every magnitude of the format occurs; scales are 2^-e with e uniform in
    {6, 7, 8} per page. Nothing here encodes values: the codes are drawn directly. With
    ``nan_sentinels`` every slot that holds no cached key (as in make_values) holds the NaN
    code 0x7F, and the scales of blocks no sequence owns are NaN.
    """
    import torch
    seed = (w.seed if seed is None else seed) + 7919
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    hkv, d, bs, nb = w.num_kv_heads, w.head_dim, w.block_size, w.num_blocks

    def codes():
        mag = torch.randint(0, 0x7F, (nb, hkv, bs, d), generator=g, device=device,
                            dtype=torch.uint8)
        sign = torch.randint(0, 2, (nb, hkv, bs, d), generator=g, device=device,
                             dtype=torch.uint8)
        return mag | (sign << 7)

    k_codes, v_codes = codes(), codes()
    e = torch.randint(6, 9, (nb, hkv, 2), generator=g, device=device, dtype=torch.int32)
    scales = torch.exp2(-e.to(torch.float32))
    if nan_sentinels:
        valid, owned = _cached_slots(w)
        mask = torch.from_numpy(~valid).to(device)
        k_codes.transpose(1, 2)[mask] = 0x7F
        v_codes.transpose(1, 2)[mask] = 0x7F
        scales[torch.from_numpy(~owned).to(device)] = float("nan")
    return dict(k_codes=k_codes, v_codes=v_codes, scales=scales)


def _cached_slots(w: Workload):
    """valid [NB, bs]: slots that hold a key cached before this step; owned [NB]: blocks some
    sequence's table lists."""
    bs = w.block_size
    valid = np.zeros((w.num_blocks, bs), dtype=bool)
    owned = np.zeros(w.num_blocks, dtype=bool)
    for s in range(w.num_seqs):
        prefix = int(w.ctx_lens[s] - w.q_lens[s])      # slots already cached
        nblk = (int(w.ctx_lens[s]) + bs - 1) // bs
        for j in range(nblk):
            b = int(w.block_table[s, j])
            owned[b] = True
            lo, hi = j * bs, min((j + 1) * bs, prefix)
            if hi > lo:
                valid[b, : hi - lo] = True
    return valid, owned


# ---------------------------------------------------------------- Linear (SmoothGEMM) inputs
# (M, N, K) of C = A W^T. The first three are the shapes of the XY-Serve page's Linear kernel
# table (section 3.1); the others are Linear layers of this step's own batches: the query
# projection over the packed prefill batch (M = its token count, which the seed decides; a
# 32-head x 128 model of hidden size 4096) and the output projection over the mixed step
# (M = 200 decode rows + 4 x 512 chunk rows; 64 heads x 128, hidden size 8192).
GEMM_SHAPES = {
    "linear_1024x1024x1024": (1024, 1024, 1024),
    "linear_512x2048x1024": (512, 2048, 1024),
    "linear_2048x512x2048": (2048, 512, 2048),
    "linear_prefill_qproj": ("prefill_varlen_bf16", 4096, 4096),
    "linear_mixed_oproj": ("mixed_bf16", 8192, 8192),
}


def gemm_shape(name: str):
    """(M, N, K) of a named Linear shape; M of a batch-derived shape is its packed token
    count."""
    m, n, k = GEMM_SHAPES[name]
    if isinstance(m, str):
        w = make_workload(m)
        m = int(w.q_lens.sum())
    return int(m), int(n), int(k)


def make_gemm_operands(M: int, N: int, K: int, device="cpu", seed: int = 0):
    """A [M, K] and W [N, K]: N(0,1) drawn in fp32 with a seeded torch generator, rounded to
    bf16."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    a = torch.randn(M, K, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    return a, w
