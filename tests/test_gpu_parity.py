"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on the same seeded
inputs. Run on an MI355X with the library built in-tree.

Bars: reshape_and_cache bit-exact; attention within max-abs 2e-2 / mean-abs 2e-3 (bf16) or
1e-4 / 1e-5 (fp32) of the oracle. Pages hold NaN in every slot no sequence owns, in the tails of
last blocks and in the slots this step writes, so a stray read or a skipped write shows up.
"""
import math

import numpy as np
import pytest
import torch

import synth
import paged_variable_length_amd as pa
from bench import TILING as BENCH_TILING
from oracle import attention as oa
from oracle import cache as oc
from tests.helpers import check_close, to_np, to_np_raw

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def host_subset(w, vals_dev, seqs):
    """Host fp64 copies of what the oracle needs for `seqs`, taken before the GPU path runs:
    their blocks (renumbered 0..) and their rows of q/k_new/v_new."""
    bs = w.block_size
    cu = oa.pack_lengths(w.q_lens)
    blocks, table_rows = [], []
    for s in seqs:
        nblk = oa.blocks_needed(int(w.ctx_lens[s]), bs)
        ids = w.block_table[s, :nblk].astype(np.int64)
        table_rows.append(np.arange(len(blocks), len(blocks) + nblk))
        blocks.extend(ids.tolist())
    idx = torch.tensor(blocks, dtype=torch.long, device=vals_dev["k_pages"].device)
    kp = to_np(vals_dev["k_pages"].index_select(0, idx))
    vp = to_np(vals_dev["v_pages"].index_select(0, idx))
    width = max(len(r) for r in table_rows)
    table = np.full((len(seqs), width), -1, dtype=np.int64)
    for i, r in enumerate(table_rows):
        table[i, :len(r)] = r
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    ridx = torch.tensor(rows, dtype=torch.long, device=vals_dev["q"].device)
    return dict(q=to_np(vals_dev["q"].index_select(0, ridx)),
                k_new=to_np(vals_dev["k_new"].index_select(0, ridx)),
                v_new=to_np(vals_dev["v_new"].index_select(0, ridx)),
                k_pages=kp, v_pages=vp, table=table, rows=rows,
                q_lens=w.q_lens[list(seqs)], ctx=w.ctx_lens[list(seqs)])


def oracle_subset(h, scale, sample_rows=None):
    kp, vp = oc.reshape_and_cache(h["k_new"], h["v_new"], h["k_pages"], h["v_pages"], h["table"],
                                  h["q_lens"], h["ctx"])
    if sample_rows is None:
        return oa.paged_attention_fast(h["q"], kp, vp, h["table"], h["q_lens"], h["ctx"], scale)
    return oa.paged_attention(h["q"], kp, vp, h["table"], h["q_lens"], h["ctx"], scale,
                              rows=sample_rows)


def run_gpu(w, vals, entry, **tiling):
    """Cache write + attention through the library; returns (out, plan)."""
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device=DEV, **tiling)
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    out = torch.full_like(vals["q"], float("nan"))
    scale = 1.0 / math.sqrt(w.head_dim)
    if entry == "decode":
        plan.decode(vals["q"], vals["k_pages"], vals["v_pages"], scale, out)
    else:
        plan.varlen(vals["q"], vals["k_pages"], vals["v_pages"], scale, out)
    torch.cuda.synchronize()
    return out, plan


def small_case(w, entry, seqs=None, **tiling):
    _announce(f"{w.name} entry={entry} N={w.num_seqs} T={w.num_tokens} Hq={w.num_q_heads} "
              f"Hkv={w.num_kv_heads} D={w.head_dim} bs={w.block_size} {tiling}")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    seqs = list(range(w.num_seqs)) if seqs is None else seqs
    h = host_subset(w, vals, seqs)
    out, plan = run_gpu(w, vals, entry, **tiling)
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim))
    got = to_np(out)[h["rows"]]
    return check_close(got, ref, w.dtype, w.name), out, vals, plan


# ------------------------------------------------------------------------ reshape_and_cache
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64), ("fp32", 128)])
def test_reshape_and_cache_bit_exact(dtype, d):
    w = synth.custom_workload([1, 5, 17, 40, 1], [1, 21, 17, 300, 77], 4, 2, d, 16, dtype=dtype,
                              seed=31, spare_blocks=3)
    _announce(f"reshape_and_cache {dtype} D={d}")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    before_k = to_np_raw(vals["k_pages"]).copy()
    before_v = to_np_raw(vals["v_pages"]).copy()
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, 4, 2, d, 16, device=DEV)
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    torch.cuda.synchronize()
    ek, ev = oc.reshape_and_cache(to_np_raw(vals["k_new"]), to_np_raw(vals["v_new"]), before_k,
                                  before_v, w.block_table, w.q_lens, w.ctx_lens)
    gk, gv = to_np_raw(vals["k_pages"]), to_np_raw(vals["v_pages"])
    assert np.array_equal(gk.view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), ev.view(np.uint8))


@pytest.mark.parametrize("name", ["prefill_varlen_bf16", "mixed_bf16"])
def test_reshape_and_cache_full_size(name):
    """Full-size cache writes: every written slot holds its token's K/V bit for bit, and since
    each target slot held a NaN sentinel and every new value is finite, the pool loses exactly
    T*Hkv*D NaNs per tensor -- no other slot was written."""
    w = synth.make_workload(name)
    _announce(f"reshape_and_cache full {name} T={w.num_tokens}")
    vals = synth.make_values(w, device=DEV)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device=DEV)
    blk, slot = [], []
    for s in range(w.num_seqs):
        P = int(w.ctx_lens[s] - w.q_lens[s])
        pos = P + np.arange(int(w.q_lens[s]))
        blk.append(w.block_table[s, pos // w.block_size]); slot.append(pos % w.block_size)
    blk = torch.from_numpy(np.concatenate(blk).astype(np.int64)).to(DEV)
    slot = torch.from_numpy(np.concatenate(slot).astype(np.int64)).to(DEV)
    nan_k0 = int(torch.isnan(vals["k_pages"]).sum()); nan_v0 = int(torch.isnan(vals["v_pages"]).sum())
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    torch.cuda.synchronize()
    got_k = vals["k_pages"].transpose(1, 2)[blk, slot]     # [T, Hkv, D]
    got_v = vals["v_pages"].transpose(1, 2)[blk, slot]
    assert torch.equal(got_k.view(torch.int16), vals["k_new"].view(torch.int16))
    assert torch.equal(got_v.view(torch.int16), vals["v_new"].view(torch.int16))
    n_written = w.num_tokens * w.num_kv_heads * w.head_dim
    assert int(torch.isnan(vals["k_pages"]).sum()) == nan_k0 - n_written
    assert int(torch.isnan(vals["v_pages"]).sum()) == nan_v0 - n_written


# ------------------------------------------------------------------------ decode
def test_tiny_decode_fp32_full():
    """The tiny fp32 workload (contexts 5, 17, 33, 64; 16-block pool), every output row."""
    w = synth.make_workload("tiny_decode_fp32")
    (mx, mean), *_ = small_case(w, "decode", dec_split=64)
    assert mx < 1e-5


@pytest.mark.parametrize("d,hq,hkv,bs", [(128, 4, 1, 16), (128, 8, 8, 32), (64, 16, 1, 64),
                                         (128, 32, 8, 128), (64, 6, 2, 256), (128, 16, 16, 16)])
def test_decode_bf16_ragged(d, hq, hkv, bs):
    ctx = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 200, 511, 512, 513, 1400]
    w = synth.custom_workload([1] * len(ctx), ctx, hq, hkv, d, bs, seed=d + hq + bs, spare_blocks=5)
    small_case(w, "decode", dec_split=128)
    small_case(w, "decode", dec_split=1024)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_fp32_ragged(d):
    ctx = [1, 3, 16, 17, 40, 100, 333]
    w = synth.custom_workload([1] * len(ctx), ctx, 8, 2, d, 16, dtype="fp32", seed=d)
    (mx, _), *_ = small_case(w, "decode", dec_split=64)


def test_single_key_returns_value_exactly_on_gpu():
    """A context of one key gives that key's value, exactly (its weight is 1 after rounding)."""
    w = synth.custom_workload([1, 1, 1], [1, 1, 1], 8, 2, 128, 16, seed=7)
    _, out, vals, plan = small_case(w, "decode", dec_split=64)
    expect = vals["v_new"].repeat_interleave(4, dim=1)
    assert torch.equal(out.view(torch.int16), expect.view(torch.int16))


@pytest.mark.parametrize("name", ["decode_mha_bf16", "decode_gqa_bf16_bs16", "decode_gqa_bf16_bs64"])
def test_decode_full_size(name):
    """Full-size decode workloads in the launch configuration bench.py times (its TILING: the
    MHA batch unsplit, one task per sequence and head writing `out` directly; key splits of 8192
    merged by the combine for the GQA batches); the oracle checks a seeded sample of sequences
    that always holds the shortest and the longest."""
    w = synth.make_workload(name)
    _announce(f"decode full {name} N={w.num_seqs}")
    rng = np.random.default_rng(0)
    n_sample = 24 if name == "decode_mha_bf16" else 40
    order = np.argsort(w.ctx_lens)
    seqs = sorted(set([int(order[0]), int(order[-1])] +
                      rng.choice(w.num_seqs, n_sample, replace=False).tolist()))[:n_sample + 2]
    vals = synth.make_values(w, device=DEV)
    h = host_subset(w, vals, seqs)
    out, _ = run_gpu(w, vals, "decode", **BENCH_TILING[name])
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim))
    check_close(to_np(out)[h["rows"]], ref, "bf16", name)
    assert torch.isfinite(out).all()


# ------------------------------------------------------------------------ prefill / mixed
@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("tiling", [dict(pf_q_tile=128, pf_kv_split=0),
                                    dict(pf_q_tile=64, pf_kv_split=128),
                                    dict(pf_q_tile=37, pf_kv_split=64)])
def test_prefill_ragged(d, tiling):
    q = [1, 2, 31, 32, 33, 64, 65, 127, 128, 129, 300]
    ctx = [c + p for c, p in zip(q, [0, 5, 0, 64, 100, 0, 17, 0, 300, 1, 0])]
    w = synth.custom_workload(q, ctx, 8, 2, d, 16, seed=d + tiling["pf_q_tile"], spare_blocks=2)
    small_case(w, "varlen", dec_split=64, **tiling)


@pytest.mark.parametrize("q_mult", [8.0, 32.0])
def test_prefill_scores_far_above_the_first_tile(q_mult):
    """Queries scaled by a power of two (exact in bf16) spread the scores so widely that later
    key tiles often hold scores far above everything in a wave's first tile: the prefill tile
    loop then has to move its reference maximum (weights above 2^16 otherwise), which N(0,1)
    inputs never make it do."""
    q = [64, 200, 300, 129]
    ctx = [64 + 500, 200, 300 + 77, 129 + 1000]
    w = synth.custom_workload(q, ctx, 8, 2, 128, 16, seed=int(q_mult), spare_blocks=2)
    _announce(f"prefill q x {q_mult} N={w.num_seqs} T={w.num_tokens}")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    vals["q"] = (vals["q"].float() * q_mult).to(vals["q"].dtype)
    h = host_subset(w, vals, list(range(w.num_seqs)))
    out, _ = run_gpu(w, vals, "varlen", dec_split=64, pf_q_tile=128, pf_kv_split=0)
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim))
    check_close(to_np(out)[h["rows"]], ref, "bf16", f"q x {q_mult}")


@pytest.mark.parametrize("bs", [16, 64, 256])
def test_mixed_decode_and_chunks(bs):
    q = [1, 512, 1, 1, 77, 1, 200]
    ctx = [900, 512 + 700, 5, 64, 77 + 1000, 1, 200]
    w = synth.custom_workload(q, ctx, 16, 2, 128, bs, seed=bs)
    small_case(w, "varlen", dec_split=256, pf_q_tile=128, pf_kv_split=512)


def test_prefill_full_size_sampled():
    """The packed varlen prefill workload at full size in the launch configuration bench.py
    times; sampled rows of every sequence (first, last, and random rows), all heads, checked one
    by one against the oracle."""
    w = synth.make_workload("prefill_varlen_bf16")
    _announce(f"prefill full T={w.num_tokens} lens={w.q_lens.tolist()}")
    vals = synth.make_values(w, device=DEV)
    seqs = list(range(w.num_seqs))
    h = host_subset(w, vals, seqs)
    out, _ = run_gpu(w, vals, "varlen", **BENCH_TILING["prefill_varlen_bf16"])
    rng = np.random.default_rng(1)
    rows = {}
    for i, s in enumerate(seqs):
        ql = int(w.q_lens[s])
        rows[i] = sorted(set([0, ql - 1] + rng.integers(0, ql, size=min(ql, 6)).tolist()))
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim), sample_rows=rows)
    check_close(to_np(out)[h["rows"]], ref, "bf16", "prefill full")
    assert torch.isfinite(out).all()


def test_mixed_full_size_sampled():
    """The mixed unified step at full size (200 decode rows + 4 x 512-row chunks over prefixes
    up to 131072 keys) in one launch, in the launch configuration bench.py times (decode splits
    of 4096 keys, each 128-row chunk tile over its whole prefix with no key split, so it writes
    `out` directly). Sampled decode sequences (shortest and longest context included), rows of
    all four chunks, and in the chunk with the longest prefix the first and last row of every
    128-row tile, all heads, against the oracle."""
    w = synth.make_workload("mixed_bf16")
    tiling = BENCH_TILING["mixed_bf16"]
    _announce(f"mixed full T={w.num_tokens} NB={w.num_blocks} {tiling}")
    vals = synth.make_values(w, device=DEV)
    rng = np.random.default_rng(2)
    chunks = sorted(range(200, 204), key=lambda s: int(w.ctx_lens[s]))
    order = np.argsort(w.ctx_lens[:200])
    dec = sorted(set(rng.choice(200, 10, replace=False).tolist() +
                     [int(order[0]), int(order[-1])]))
    seqs = dec + chunks
    h = host_subset(w, vals, seqs)
    out, plan = run_gpu(w, vals, "varlen", **tiling)
    pf = plan.table.tasks[plan.table.tasks[:, 0] == pa.PA_TASK_PREFILL]
    assert np.all(pf[:, 7] == -1), "the benched mixed tiling runs prefill tiles unsplit"
    rows = {i: [0] for i in range(len(dec))}
    for i, s in enumerate(chunks):
        ql = int(w.q_lens[s])
        if s == chunks[-1]:
            rows[len(dec) + i] = sorted({r for r0 in range(0, ql, 128)
                                         for r in (r0, min(ql, r0 + 128) - 1)})
        else:
            rows[len(dec) + i] = [0, ql // 2 - 1, ql - 1]
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim), sample_rows=rows)
    check_close(to_np(out)[h["rows"]], ref, "bf16", "mixed full")
    assert torch.isfinite(out).all()


# ------------------------------------------------------------------------ verify (draft rows)
@pytest.mark.parametrize("hq,hkv,bs", [(4, 1, 16), (8, 2, 64), (16, 8, 16), (8, 8, 128)])
@pytest.mark.parametrize("dec_split", [64, 512])
def test_verify_ragged(hq, hkv, bs, dec_split):
    """Short multi-row sequences as verify tasks (all rows and the G heads of a kv head in one
    task, causal inside the draft), with key splits and block tails; G*q_len <= 16 throughout
    so every multi-row sequence is a verify task."""
    G = hq // hkv
    rmax = 16 // G
    q = [min(r, rmax) for r in (2, 3, 4, 2, 8, 5, 16, 1, 2)]
    ctx = [qq + p for qq, p in zip(q, [0, 1, 14, 61, 100, 300, 700, 513, 1030])]
    w = synth.custom_workload(q, ctx, hq, hkv, 128, bs, seed=hq + bs + dec_split, spare_blocks=3)
    plan_tasks = pa.build_task_table(
        pa.make_params(hq, hkv, 128, bs, dec_split=dec_split, verify_rows=16),
        pa.pack_seqlens(q), w.ctx_lens).tasks
    assert {int(k) for k in plan_tasks[:, 0]} <= {0, 2} and 2 in set(plan_tasks[:, 0].tolist())
    small_case(w, "varlen", dec_split=dec_split, verify_rows=16)


def test_verify_with_decode_and_prefill_in_one_launch():
    """Decode rows, verify drafts and prefill chunks in one table and one launch."""
    q = [1, 4, 300, 1, 3, 2, 64]
    ctx = [900, 4 + 1000, 300 + 50, 7, 3, 2 + 4095, 64 + 64]
    w = synth.custom_workload(q, ctx, 32, 8, 128, 16, seed=77, spare_blocks=4)
    small_case(w, "varlen", dec_split=256, pf_q_tile=128, pf_kv_split=128, verify_rows=4)


def test_verify_full_size_sampled():
    """The 256-sequence GQA batch with 4-row drafts as verify tasks in the benchmark's launch
    configuration; every row of a seeded sample of sequences (shortest and longest included)."""
    w = synth.make_workload("verify_gqa_bf16")
    _announce(f"verify full N={w.num_seqs} T={w.num_tokens}")
    rng = np.random.default_rng(3)
    order = np.argsort(w.ctx_lens)
    seqs = sorted(set([int(order[0]), int(order[-1])] +
                      rng.choice(w.num_seqs, 30, replace=False).tolist()))
    vals = synth.make_values(w, device=DEV)
    h = host_subset(w, vals, seqs)
    out, plan = run_gpu(w, vals, "varlen", **BENCH_TILING["verify_gqa_bf16"])
    assert set(plan.table.tasks[:, 0].tolist()) == {2}
    ref = oracle_subset(h, 1.0 / math.sqrt(w.head_dim))
    check_close(to_np(out)[h["rows"]], ref, "bf16", "verify full")
    assert torch.isfinite(out).all()


# ------------------------------------------------------------------------ invariants on GPU
def test_determinism_and_block_permutation_bitwise():
    q = [1, 130, 1, 40]
    ctx = [700, 130 + 90, 33, 40]
    w = synth.custom_workload(q, ctx, 8, 2, 128, 16, seed=99, spare_blocks=6)
    _announce("determinism + permutation")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    tiling = dict(dec_split=128, pf_q_tile=64, pf_kv_split=64)
    base = {k: v.clone() for k, v in vals.items()}
    out1, _ = run_gpu(w, vals, "varlen", **tiling)
    vals2 = {k: v.clone() for k, v in base.items()}
    out2, _ = run_gpu(w, vals2, "varlen", **tiling)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    perm = np.random.default_rng(5).permutation(w.num_blocks)
    pt = torch.from_numpy(perm).to(DEV)
    kp = torch.empty_like(base["k_pages"]); vp = torch.empty_like(base["v_pages"])
    kp[pt] = base["k_pages"]; vp[pt] = base["v_pages"]
    table2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    w2 = synth.Workload(w.name, w.seed, w.q_lens, w.ctx_lens, 8, 2, 128, 16, "bf16", table2,
                        w.num_blocks)
    vals3 = dict(base, k_pages=kp, v_pages=vp)
    out3, _ = run_gpu(w2, vals3, "varlen", **tiling)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))


@pytest.mark.parametrize("pf_q_tile,pf_kv_split", [(100, 0), (128, 192)])
def test_prefill_repeat_runs_bitwise(pf_q_tile, pf_kv_split):
    """Repeated launches on the same inputs give bit-identical outputs. The batch has diagonal
    key tiles whose valid keys are loaded by waves that have no tile left to compute there
    (they only load for the others), the case where a load or barrier slip would show."""
    q = [1, 2, 31, 33, 65, 127, 129, 300, 392, 200]
    ctx = [c + p for c, p in zip(q, [0, 5, 0, 100, 17, 0, 1, 0, 0, 8])]
    w = synth.custom_workload(q, ctx, 8, 2, 128, 16, seed=pf_q_tile, spare_blocks=2)
    _announce(f"repeat runs pf_q_tile={pf_q_tile} pf_kv_split={pf_kv_split}")
    base = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    first = None
    for _ in range(6):
        vals = {k: v.clone() for k, v in base.items()}
        out, _ = run_gpu(w, vals, "varlen", dec_split=64, pf_q_tile=pf_q_tile,
                         pf_kv_split=pf_kv_split)
        if first is None:
            first = out.clone()
        assert torch.equal(first.view(torch.int16), out.view(torch.int16))


def test_empty_table_is_a_no_op():
    w = synth.custom_workload([1], [5], 2, 1, 64, 16, seed=1)
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    empty = torch.zeros(0, 8, dtype=torch.int32, device=DEV)
    out = torch.full_like(vals["q"], 7.0)
    pa.paged_attn_decode(vals["q"], vals["k_pages"], vals["v_pages"],
                         torch.from_numpy(w.block_table).to(DEV),
                         torch.from_numpy(w.ctx_lens.astype(np.int32)).to(DEV), 0.125, empty,
                         0, empty, 0, None, out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
