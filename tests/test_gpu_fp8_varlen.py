"""GPU parity of the unified launch over fp8 pages (paged_attn_varlen_prefill_fp8): decode rows,
prefill chunks, verify drafts and shared prefixes in one grid. The cache write runs on the GPU
(its codes and scales are checked bit for bit elsewhere); the reference is the fp64 attention
oracle on the fp8 oracle's own cache write of host copies of the pages, dequantized. Run on an
MI355X with the library built in-tree."""
import math

import numpy as np
import pytest
import torch

import synth
import paged_variable_length_amd as pa
from bench import TILING as BENCH_TILING
from oracle import attention as oa
from oracle import fp8 as of
from tests.helpers import aliased_workload, check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def fp8_host_subset(w, vals, pages, seqs):
    """Host copies of what the oracle needs for `seqs`, taken before the GPU writes: their
    blocks' codes and scales (each physical block once, renumbered 0..), their table rows in
    that numbering, and their rows of q / k_new / v_new."""
    bs = w.block_size
    cu = oa.pack_lengths(w.q_lens)
    new_id, blocks, table_rows = {}, [], []
    for s in seqs:
        row = []
        for b in w.block_table[s, :oa.blocks_needed(int(w.ctx_lens[s]), bs)].tolist():
            if b not in new_id:
                new_id[b] = len(blocks)
                blocks.append(b)
            row.append(new_id[b])
        table_rows.append(row)
    table = np.full((len(seqs), max(len(r) for r in table_rows)), -1, dtype=np.int64)
    for i, r in enumerate(table_rows):
        table[i, :len(r)] = r
    idx = torch.tensor(blocks, dtype=torch.long, device=pages["k_codes"].device)
    sc = pages["scales"].index_select(0, idx).cpu().numpy().astype(np.float64)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    ridx = torch.tensor(rows, dtype=torch.long, device=vals["q"].device)
    return dict(q=to_np(vals["q"].index_select(0, ridx)),
                k_new=to_np(vals["k_new"].index_select(0, ridx)),
                v_new=to_np(vals["v_new"].index_select(0, ridx)),
                k_codes=pages["k_codes"].index_select(0, idx).cpu().numpy(),
                v_codes=pages["v_codes"].index_select(0, idx).cpu().numpy(),
                k_scales=sc[..., 0], v_scales=sc[..., 1], table=table, rows=rows,
                q_lens=w.q_lens[list(seqs)], ctx=w.ctx_lens[list(seqs)])


def fp8_oracle(h, scale, sample_rows=None):
    """The fp8 oracle's cache write on the subset, then fp64 attention on its dequantized
    pages (all rows, or the sampled rows per sequence)."""
    kc, vc, ks, vs = of.reshape_and_cache_fp8(h["k_new"], h["v_new"], h["k_codes"], h["v_codes"],
                                              h["k_scales"], h["v_scales"], h["table"],
                                              h["q_lens"], h["ctx"])
    kp, vp = of.dequantize_pages(kc, ks), of.dequantize_pages(vc, vs)
    if sample_rows is None:
        return oa.paged_attention_fast(h["q"], kp, vp, h["table"], h["q_lens"], h["ctx"], scale)
    return oa.paged_attention(h["q"], kp, vp, h["table"], h["q_lens"], h["ctx"], scale,
                              rows=sample_rows)


def fp8_case(w, seqs=None, sample_rows=None, values_on=DEV, q_mult=1.0, **tiling):
    """Cache write and unified launch over fp8 pages on the GPU; the sampled sequences' rows
    against the oracle. q is drawn on `values_on` and multiplied by q_mult (a power of two, so
    exact in bf16). Returns (max-abs, mean-abs), out, plan."""
    _announce(f"{w.name} fp8 unified N={w.num_seqs} T={w.num_tokens} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} D={w.head_dim} bs={w.block_size} q x {q_mult} {tiling}")
    vals = synth.make_values(w, device=values_on)
    del vals["k_pages"], vals["v_pages"]
    vals = {k: v.to(DEV) for k, v in vals.items()}
    vals["q"] = (vals["q"].float() * q_mult).to(vals["q"].dtype)
    pages = synth.make_fp8_pages(w, device=values_on)
    pages = {k: v.to(DEV) for k, v in pages.items()}
    seqs = list(range(w.num_seqs)) if seqs is None else seqs
    h = fp8_host_subset(w, vals, pages, seqs)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device=DEV, **tiling)
    plan.write_cache_fp8(vals["k_new"], vals["v_new"], pages["k_codes"], pages["v_codes"],
                         pages["scales"])
    out = torch.full_like(vals["q"], float("nan"))
    scale = 1.0 / math.sqrt(w.head_dim)
    plan.varlen_fp8(vals["q"], pages["k_codes"], pages["v_codes"], pages["scales"], scale, out)
    torch.cuda.synchronize()
    ref = fp8_oracle(h, scale, sample_rows)
    return check_close(to_np(out)[h["rows"]], ref, "bf16", w.name), out, plan


def _kinds(plan):
    return {int(k) for k in plan.table.tasks[:, 0]}


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("tiling", [dict(pf_q_tile=128, pf_kv_split=0),
                                    dict(pf_q_tile=64, pf_kv_split=128),
                                    dict(pf_q_tile=37, pf_kv_split=64)])
def test_varlen_fp8_ragged(d, tiling):
    """Chunks of 1 .. 300 rows over prefixes of 0 .. 300 keys: partial key tiles, causal
    diagonals inside a tile, key splits merged by the combine, decode rows beside them."""
    q = [1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 300]
    ctx = [c + p for c, p in zip(q, [0, 5, 0, 64, 100, 0, 17, 0, 300, 1, 0])]
    w = synth.custom_workload(q, ctx, 8, 2, d, 16, seed=d + tiling["pf_q_tile"], spare_blocks=2)
    _, _, plan = fp8_case(w, values_on="cpu", dec_split=64, **tiling)
    assert pa.PA_TASK_PREFILL in _kinds(plan)


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_varlen_fp8_decode_and_chunks(bs):
    """Decode rows and long chunks over long prefixes at every block size the wave's 16-key
    piece can sit in (a piece never crosses a block), with key splits on both kinds."""
    q = [1, 512, 1, 1, 77, 1, 200]
    ctx = [900, 512 + 700, 5, 64, 77 + 1000, 1, 200]
    w = synth.custom_workload(q, ctx, 16, 2, 128, bs, seed=bs, spare_blocks=2)
    fp8_case(w, values_on="cpu", dec_split=256, pf_q_tile=128, pf_kv_split=512)


def _append_sequences(w, q_extra, ctx_extra, rng):
    """w with more sequences after its own, each in fresh blocks (a shuffled range of ids
    after w's pool)."""
    bs = w.block_size
    need = [-(-int(c) // bs) for c in ctx_extra]
    ids = w.num_blocks + rng.permutation(sum(need))
    width = max(w.block_table.shape[1], max(need))
    table = np.full((w.num_seqs + len(need), width), -1, dtype=np.int32)
    table[:w.num_seqs, :w.block_table.shape[1]] = w.block_table
    pos = 0
    for i, n in enumerate(need):
        table[w.num_seqs + i, :n] = ids[pos:pos + n]
        pos += n
    return synth.Workload(w.name, w.seed, np.concatenate([w.q_lens, q_extra]).astype(np.int64),
                          np.concatenate([w.ctx_lens, ctx_extra]).astype(np.int64),
                          w.num_q_heads, w.num_kv_heads, w.head_dim, bs, w.dtype, table,
                          w.num_blocks + pos)


@pytest.mark.parametrize("seed,G", [(1, 1), (2, 2), (3, 4), (4, 8)])
def test_varlen_fp8_every_kind_in_one_launch(seed, G):
    """Decode rows, verify drafts, prefill chunks and shared-prefix groups in one table and one
    launch over fp8 pages: groups of decode sequences that alias leading blocks, short drafts
    between them, and two chunks (one over a cached prefix) after them."""
    rng = np.random.default_rng(60 + seed)
    w = _append_sequences(aliased_workload(rng, 16, 8, 2 * G, 2, 128, seed=seed),
                          [150, 40], [150 + 333, 40], rng)
    _, _, plan = fp8_case(w, values_on="cpu", dec_split=64, pf_q_tile=64, verify_rows=4,
                          shared_min=64)
    assert _kinds(plan) == {pa.PA_TASK_DECODE, pa.PA_TASK_PREFILL, pa.PA_TASK_VERIFY,
                            pa.PA_TASK_SHARED}


def test_varlen_fp8_scores_far_above_the_first_tile():
    """Queries scaled by 32 (exact in bf16) make later key tiles hold scores far above a wave's
    first tile, so the prefill loop moves its reference maximum over fp8 pages too."""
    q = [64, 200, 300, 129]
    ctx = [64 + 500, 200, 300 + 77, 129 + 1000]
    w = synth.custom_workload(q, ctx, 8, 2, 128, 16, seed=32, spare_blocks=2)
    fp8_case(w, values_on="cpu", q_mult=32.0, dec_split=64, pf_q_tile=128, pf_kv_split=0)


def test_mixed_fp8_full_size_sampled():
    """The mixed unified step at full size over fp8 pages (200 decode rows + 4 x 512-row chunks
    over prefixes up to 131072 keys) in the launch configuration bench.py times; sampled decode
    sequences (shortest and longest context included), and rows of all four chunks with the
    first and last row of every 128-row tile of the chunk with the longest prefix."""
    w = synth.make_workload("mixed_fp8")
    tiling = BENCH_TILING["mixed_fp8"]
    rng = np.random.default_rng(8)
    chunks = sorted(range(200, 204), key=lambda s: int(w.ctx_lens[s]))
    order = np.argsort(w.ctx_lens[:200])
    dec = sorted(set(rng.choice(200, 10, replace=False).tolist() +
                     [int(order[0]), int(order[-1])]))
    rows = {i: [0] for i in range(len(dec))}
    for i, s in enumerate(chunks):
        ql = int(w.q_lens[s])
        if s == chunks[-1]:
            rows[len(dec) + i] = sorted({r for r0 in range(0, ql, 128)
                                         for r in (r0, min(ql, r0 + 128) - 1)})
        else:
            rows[len(dec) + i] = [0, ql // 2 - 1, ql - 1]
    (_, _), out, plan = fp8_case(w, seqs=dec + chunks, sample_rows=rows, **tiling)
    assert _kinds(plan) == {pa.PA_TASK_DECODE, pa.PA_TASK_PREFILL}
    assert torch.isfinite(out).all()


def test_prefill_fp8_full_size_sampled():
    """The packed varlen prefill batch at full size over fp8 pages (every page of it written by
    this step's cache write) in the launch configuration bench.py times; the first, the last and
    random rows of every sequence against the oracle."""
    w = synth.make_workload("prefill_varlen_fp8")
    rng = np.random.default_rng(9)
    rows = {}
    for s in range(w.num_seqs):
        ql = int(w.q_lens[s])
        rows[s] = sorted(set([0, ql - 1] + rng.integers(0, ql, size=min(ql, 6)).tolist()))
    (_, _), out, plan = fp8_case(w, sample_rows=rows, **BENCH_TILING["prefill_varlen_fp8"])
    assert _kinds(plan) == {pa.PA_TASK_PREFILL}
    assert torch.isfinite(out).all()
