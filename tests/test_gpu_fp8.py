"""GPU parity for fp8 pages: the cache write bit for bit against the fp8 oracle (codes and page
scales), and decode attention over fp8 pages against the fp64 attention oracle run on the
oracle's dequantized pages. Run on an MI355X with the library built in-tree."""
import math

import numpy as np
import pytest
import torch

import synth
import paged_variable_length_amd as pa
from bench import TILING as BENCH_TILING
from paged_variable_length_amd import _abi
from oracle import attention as oa
from oracle import fp8 as of
from tests.helpers import check_close, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _oracle_write(w, vals, pages):
    """The fp8 oracle's cache write on host copies of the inputs."""
    return of.reshape_and_cache_fp8(
        to_np(vals["k_new"]), to_np(vals["v_new"]), pages["k_codes"].cpu().numpy(),
        pages["v_codes"].cpu().numpy(), pages["scales"][..., 0].cpu().numpy().astype(np.float64),
        pages["scales"][..., 1].cpu().numpy().astype(np.float64), w.block_table, w.q_lens,
        w.ctx_lens)


def _gpu_write(w, vals, pages, plan):
    plan.write_cache_fp8(vals["k_new"], vals["v_new"], pages["k_codes"], pages["v_codes"],
                         pages["scales"])
    torch.cuda.synchronize()


def _assert_pages_equal(pages, ref):
    kc, vc, ks, vs = ref
    assert np.array_equal(pages["k_codes"].cpu().numpy(), kc)
    assert np.array_equal(pages["v_codes"].cpu().numpy(), vc)
    # the page scales sit side by side per (block, kv head): K then V
    got = pages["scales"].cpu().numpy()
    assert np.array_equal(got[..., 0], ks.astype(np.float32), equal_nan=True)
    assert np.array_equal(got[..., 1], vs.astype(np.float32), equal_nan=True)


@pytest.mark.parametrize("d,bs", [(128, 16), (64, 16), (128, 64), (64, 256)])
def test_reshape_and_cache_fp8_bit_exact(d, bs):
    """Decode appends into the middle of a page and at a page boundary, a chunk spanning
    several pages over a cached prefix, and fresh prompts: codes and scales bit for bit, and
    every slot outside the written pages untouched (NaN codes stay NaN)."""
    q = [1, 1, 40, 1, 130, 3]
    ctx = [17, bs + 1, 40 + 29, 2 * bs, 130, 3 + 5]
    w = synth.custom_workload(q, ctx, 8, 4, d, bs, seed=d + bs, spare_blocks=3)
    _announce(f"fp8 cache write D={d} bs={bs}")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    pages = {k: v.to(DEV) for k, v in synth.make_fp8_pages(w).items()}
    ref = _oracle_write(w, vals, pages)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, 8, 4, d, bs, device=DEV)
    _gpu_write(w, vals, pages, plan)
    _assert_pages_equal(pages, ref)


def test_reshape_and_cache_fp8_two_steps():
    """Two decode steps in a row into the same pages: the second rescales what the first
    wrote whenever its row raises the page maximum. The block table is dealt for the second
    step's contexts, so both steps find every page they write."""
    ctx1 = [6, 17, 34, 2]
    w1 = synth.custom_workload([1] * 4, ctx1, 4, 2, 128, 16, seed=5, spare_blocks=4)
    w0 = synth.Workload(w1.name, w1.seed + 1, w1.q_lens, w1.ctx_lens - 1, 4, 2, 128, 16, "bf16",
                        w1.block_table, w1.num_blocks)
    pages = {k: v.to(DEV) for k, v in synth.make_fp8_pages(w0).items()}
    for w in (w0, w1):
        vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
        vals["k_new"] *= 40.0 if w is w1 else 1.0          # the second step raises page maxima
        ref = _oracle_write(w, vals, pages)
        plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, 4, 2, 128, 16, device=DEV)
        _gpu_write(w, vals, pages, plan)
        _assert_pages_equal(pages, ref)


def _subset(codes, scales, w, seqs):
    """Dequantized pages of the sampled sequences only, renumbered, with their table rows."""
    bs = w.block_size
    blocks, rows = [], []
    for s in seqs:
        nblk = oa.blocks_needed(int(w.ctx_lens[s]), bs)
        rows.append(np.arange(len(blocks), len(blocks) + nblk))
        blocks.extend(w.block_table[s, :nblk].tolist())
    table = np.full((len(seqs), max(len(r) for r in rows)), -1, dtype=np.int64)
    for i, r in enumerate(rows):
        table[i, :len(r)] = r
    idx = np.array(blocks)
    return of.dequantize_pages(codes[idx], scales[idx]), table


def _decode_case(w, dec_split, seqs=None, **tiling):
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    pages = {k: v.to(DEV) for k, v in synth.make_fp8_pages(w).items()}
    kc, vc, ks, vs = _oracle_write(w, vals, pages)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device=DEV, dec_split=dec_split, **tiling)
    _gpu_write(w, vals, pages, plan)
    out = torch.full_like(vals["q"], float("nan"))
    scale = 1.0 / math.sqrt(w.head_dim)
    plan.decode_fp8(vals["q"], pages["k_codes"], pages["v_codes"], pages["scales"], scale, out)
    torch.cuda.synchronize()
    seqs = list(range(w.num_seqs)) if seqs is None else seqs
    kp, table = _subset(kc, ks, w, seqs)
    vp, _ = _subset(vc, vs, w, seqs)
    q = to_np(vals["q"])[seqs]
    ref = oa.paged_attention_fast(q, kp, vp, table, w.q_lens[seqs], w.ctx_lens[seqs], scale)
    return check_close(to_np(out)[seqs], ref, "bf16", w.name), out, plan


@pytest.mark.parametrize("d,hq,hkv,bs", [(128, 8, 2, 16), (128, 32, 32, 16), (64, 16, 4, 64),
                                         (128, 16, 1, 128)])
@pytest.mark.parametrize("dec_split", [64, 512])
def test_decode_fp8_ragged(d, hq, hkv, bs, dec_split):
    ctx = [1, 2, 15, 16, 17, 33, 64, 65, 200, 513, 1400]
    w = synth.custom_workload([1] * len(ctx), ctx, hq, hkv, d, bs, seed=d + hq + bs,
                              spare_blocks=4)
    _announce(f"fp8 decode D={d} Hq={hq} Hkv={hkv} bs={bs} dec_split={dec_split}")
    _decode_case(w, dec_split)


def test_decode_fp8_full_size_sampled():
    """The 64-sequence MHA decode batch over fp8 pages in the benchmark's configuration; a
    seeded sample of sequences (shortest and longest included) against the oracle."""
    w = synth.make_workload("decode_mha_fp8")
    _announce(f"fp8 decode full N={w.num_seqs} NB={w.num_blocks}")
    rng = np.random.default_rng(4)
    order = np.argsort(w.ctx_lens)
    seqs = sorted(set([int(order[0]), int(order[-1])] +
                      rng.choice(w.num_seqs, 10, replace=False).tolist()))
    _, out, _ = _decode_case(w, BENCH_TILING["decode_mha_fp8"]["dec_split"], seqs)
    assert torch.isfinite(out).all()


def _verify_case(w, dec_split, verify_rows, seqs=None):
    """Cache write, then decode rows and drafts over fp8 pages through paged_attn_verify_fp8,
    against the fp64 oracle on the oracle's dequantized pages (all rows of `seqs`)."""
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    pages = {k: v.to(DEV) for k, v in synth.make_fp8_pages(w).items()}
    kc, vc, ks, vs = _oracle_write(w, vals, pages)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device=DEV, dec_split=dec_split,
                       verify_rows=verify_rows)
    _gpu_write(w, vals, pages, plan)
    out = torch.full_like(vals["q"], float("nan"))
    scale = 1.0 / math.sqrt(w.head_dim)
    plan.verify_fp8(vals["q"], pages["k_codes"], pages["v_codes"], pages["scales"], scale, out)
    torch.cuda.synchronize()
    seqs = list(range(w.num_seqs)) if seqs is None else seqs
    cu = oa.pack_lengths(w.q_lens)
    rows = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])
    kp, table = _subset(kc, ks, w, seqs)
    vp, _ = _subset(vc, vs, w, seqs)
    ref = oa.paged_attention_fast(to_np(vals["q"])[rows], kp, vp, table, w.q_lens[seqs],
                                  w.ctx_lens[seqs], scale)
    return check_close(to_np(out)[rows], ref, "bf16", w.name), out


@pytest.mark.parametrize("d,hq,hkv,bs", [(128, 32, 8, 16), (128, 8, 8, 64), (64, 16, 2, 16),
                                         (128, 16, 1, 128)])
@pytest.mark.parametrize("dec_split", [64, 512])
def test_verify_fp8_ragged(d, hq, hkv, bs, dec_split):
    """Drafts of 2 .. min(8, 16 / G) rows and single decode rows over ragged contexts."""
    g = hq // hkv
    longest = min(8, 16 // g)
    rng = np.random.default_rng(d + hq + bs + dec_split)
    ctx = [50, 300, 17, 1000, 4, 65, 129, 700, 2]
    q = [1 if i % 3 == 2 or longest < 2 else int(rng.integers(2, longest + 1))
         for i in range(len(ctx))]
    ctx = [max(c, ql) for c, ql in zip(ctx, q)]
    w = synth.custom_workload(q, ctx, hq, hkv, d, bs, seed=d + hq + bs, spare_blocks=3)
    _announce(f"fp8 verify D={d} Hq={hq} Hkv={hkv} bs={bs} dec_split={dec_split} q={q}")
    _verify_case(w, dec_split, max(2, longest))


def test_verify_fp8_full_size_sampled():
    """The 256-sequence GQA verify batch (4 draft rows each) over fp8 pages in the benchmark's
    configuration; a seeded sample of sequences (shortest and longest included)."""
    w = synth.make_workload("verify_gqa_fp8")
    _announce(f"fp8 verify full N={w.num_seqs} T={w.num_tokens} NB={w.num_blocks}")
    rng = np.random.default_rng(6)
    order = np.argsort(w.ctx_lens)
    seqs = sorted(set([int(order[0]), int(order[-1])] +
                      rng.choice(w.num_seqs, 10, replace=False).tolist()))
    tiling = BENCH_TILING["verify_gqa_fp8"]
    _, out = _verify_case(w, tiling["dec_split"], tiling["verify_rows"], seqs)
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("hq,hkv,d,bs,dec_split", [(8, 8, 128, 16, 64), (16, 4, 64, 32, 64),
                                                   (32, 4, 128, 16, 128)])
def test_shared_decode_fp8(hq, hkv, d, bs, dec_split):
    """Decode sequences whose tables alias a prompt's blocks, over fp8 pages: the prefix runs as
    shared-prefix tasks read once per group and kv head (their rows are the members' own)."""
    rng = np.random.default_rng(hq * 10 + bs + d)
    prefix = rng.integers(1, 40, size=5) * bs
    own = [rng.integers(1, 300, size=int(rng.integers(1, 21))) for _ in range(5)]
    w = synth.shared_prefix_workload(prefix, own, hq, hkv, d, bs, seed=int(rng.integers(1 << 30)),
                                     spare_blocks=3)
    _announce(f"fp8 shared decode Hq={hq} Hkv={hkv} D={d} bs={bs} groups={prefix.tolist()}")
    _, out, plan = _decode_case(w, dec_split, shared_min=64)
    assert np.any(plan.table.tasks[:, 0] == _abi.PA_TASK_SHARED)
