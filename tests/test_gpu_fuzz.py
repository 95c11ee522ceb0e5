"""GPU parity on seeded random batches: the parameter space the fixed cases sample by hand
(head dim, block size, GQA group, split sizes, query tile, verify rows, the mix of decode,
draft and prefill rows), drawn jointly, each batch checked against the fp64 oracle at the same
bars as the fixed cases (the unified launch over bf16 and over fp8 pages, and the decode
entry). Every case prints its seed and shapes before it runs."""
import numpy as np
import pytest

import synth
from tests.test_gpu_parity import small_case

pytestmark = pytest.mark.gpu


def _batch(rng, max_seqs, decode_only):
    n = int(rng.integers(1, max_seqs + 1))
    q, ctx = [], []
    for _ in range(n):
        kind = 0 if decode_only else int(rng.choice(3, p=[0.5, 0.2, 0.3]))
        ql = 1 if kind == 0 else (int(rng.integers(2, 5)) if kind == 1 else int(rng.integers(5, 300)))
        prefix = int(rng.integers(0 if ql > 1 else 1, 1500))
        q.append(ql)
        ctx.append(ql + prefix - (1 if ql == 1 else 0))
    return q, ctx


@pytest.mark.parametrize("seed", range(64))
def test_random_mixed_batches(seed):
    """Unified launch (bf16) over a random mix of decode rows, short drafts and prefill chunks."""
    rng = np.random.default_rng(7000 + seed)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    q, ctx = _batch(rng, 10, decode_only=False)
    tiling = dict(dec_split=int(rng.choice([64, 128, 512, 4096])),
                  pf_q_tile=int(rng.choice([16, 64, 100, 128])),
                  pf_kv_split=int(rng.choice([0, 64, 192, 512])),
                  verify_rows=int(rng.choice([0, 4, 8])))
    w = synth.custom_workload(q, ctx, hkv * g, hkv, d, bs, seed=seed,
                              spare_blocks=int(rng.integers(0, 4)))
    small_case(w, "varlen", **tiling)


@pytest.mark.parametrize("seed", range(32))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_random_decode_batches(seed, dtype):
    """Decode entry over random single-row batches (bf16 and fp32 pages)."""
    rng = np.random.default_rng(8000 + seed)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 8]))
    g = int(rng.choice([1, 4, 8, 16]))
    q, ctx = _batch(rng, 16, decode_only=True)
    w = synth.custom_workload(q, ctx, hkv * g, hkv, d, bs, dtype=dtype, seed=seed,
                              spare_blocks=int(rng.integers(0, 4)))
    small_case(w, "decode", dec_split=int(rng.choice([64, 256, 1024])))


@pytest.mark.parametrize("seed", range(48))
def test_random_mixed_batches_fp8(seed):
    """Unified launch over fp8 pages, on the same random space as the bf16 batches."""
    from tests.test_gpu_fp8_varlen import fp8_case
    rng = np.random.default_rng(9000 + seed)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    q, ctx = _batch(rng, 10, decode_only=False)
    tiling = dict(dec_split=int(rng.choice([64, 128, 512, 4096])),
                  pf_q_tile=int(rng.choice([16, 64, 100, 128])),
                  pf_kv_split=int(rng.choice([0, 64, 192, 512])),
                  verify_rows=int(rng.choice([0, 4, 8])))
    w = synth.custom_workload(q, ctx, hkv * g, hkv, d, bs, seed=seed,
                              spare_blocks=int(rng.integers(0, 4)))
    fp8_case(w, values_on="cpu", **tiling)


@pytest.mark.parametrize("seed", range(24))
def test_random_shared_prefix_batches(seed):
    """Shared-prefix groups on random shapes: decode groups through the decode entry (even
    seeds), or aliased groups between prefill and verify rows through the unified launch (odd
    seeds); group sizes, prefix lengths, G, block size, split size and grouping threshold drawn
    jointly."""
    from tests.helpers import aliased_workload
    rng = np.random.default_rng(9500 + seed)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    shared_min = int(rng.choice([64, 128, 256]))
    dec_split = int(rng.choice([64, 128, 256, 1024]))   # shared tables: multiples of 64 keys
    if seed % 2 == 0:
        n_groups = int(rng.integers(1, 5))
        prefix = rng.integers(1, 40, size=n_groups) * bs
        own = [rng.integers(1, 300, size=int(rng.integers(1, 20))) for _ in range(n_groups)]
        w = synth.shared_prefix_workload(prefix, own, hkv * g, hkv, d, bs, seed=seed,
                                         spare_blocks=int(rng.integers(0, 4)))
        small_case(w, "decode", dec_split=dec_split, shared_min=shared_min)
    else:
        w = aliased_workload(rng, bs, int(rng.integers(2, 7)), hkv * g, hkv, d, seed=seed)
        small_case(w, "varlen", dec_split=dec_split, pf_q_tile=int(rng.choice([32, 64, 128])),
                   verify_rows=int(rng.choice([0, 4])), shared_min=shared_min)


def _cache_batch(seed):
    """Random lengths and shapes of a cache-write case (host draws only)."""
    rng = np.random.default_rng(11000 + seed)
    d = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    q, ctx = _batch(rng, 12, decode_only=False)
    return rng, q, ctx, hkv, d, bs


@pytest.mark.parametrize("seed", range(16))
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_random_cache_writes(seed, dtype):
    """reshape_and_cache on random batches (decode appends, drafts, chunks over prefixes, any
    block size and head shape): the pages bit for bit against the oracle's scatter, every other
    slot untouched."""
    import torch
    import paged_variable_length_amd as pa
    from oracle import cache as oc
    from tests.helpers import to_np_raw
    rng, q, ctx, hkv, d, bs = _cache_batch(seed)
    w = synth.custom_workload(q, ctx, hkv, hkv, d, bs, dtype=dtype, seed=seed,
                              spare_blocks=int(rng.integers(0, 4)))
    print(f"\n[case] cache write {dtype} seed={seed} N={w.num_seqs} T={w.num_tokens} "
          f"Hkv={hkv} D={d} bs={bs}", flush=True)
    vals = {k: v.to("cuda") for k, v in synth.make_values(w, device="cpu").items()}
    before_k, before_v = to_np_raw(vals["k_pages"]).copy(), to_np_raw(vals["v_pages"]).copy()
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, hkv, hkv, d, bs, device="cuda")
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    torch.cuda.synchronize()
    ek, ev = oc.reshape_and_cache(to_np_raw(vals["k_new"]), to_np_raw(vals["v_new"]), before_k,
                                  before_v, w.block_table, w.q_lens, w.ctx_lens)
    assert np.array_equal(to_np_raw(vals["k_pages"]).view(np.uint8), ek.view(np.uint8))
    assert np.array_equal(to_np_raw(vals["v_pages"]).view(np.uint8), ev.view(np.uint8))


@pytest.mark.parametrize("seed", range(16))
def test_random_cache_writes_fp8(seed):
    """The fp8 cache write on random batches: codes and page scales bit for bit against the
    fp8 oracle (pages rescaled when a new row raises their maximum), other pages untouched."""
    from tests.test_gpu_fp8 import _assert_pages_equal, _gpu_write, _oracle_write
    import paged_variable_length_amd as pa
    rng, q, ctx, hkv, d, bs = _cache_batch(seed)
    w = synth.custom_workload(q, ctx, 2 * hkv, hkv, d, bs, seed=seed,
                              spare_blocks=int(rng.integers(0, 4)))
    print(f"\n[case] fp8 cache write seed={seed} N={w.num_seqs} T={w.num_tokens} "
          f"Hkv={hkv} D={d} bs={bs}", flush=True)
    vals = {k: v.to("cuda") for k, v in synth.make_values(w, device="cpu").items()}
    pages = {k: v.to("cuda") for k, v in synth.make_fp8_pages(w).items()}
    ref = _oracle_write(w, vals, pages)
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, 2 * hkv, hkv, d, bs, device="cuda")
    _gpu_write(w, vals, pages, plan)
    _assert_pages_equal(pages, ref)
