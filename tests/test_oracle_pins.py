"""Pins for the fp64 attention oracle: the pages' worked example, closed forms, invariants and a
library routine on tiny inputs. CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import synth
from oracle import attention as oa
from tests.helpers import to_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def np_inputs(w, seed=None, nan=True):
    v = synth.make_values(w, device="cpu", seed=seed, nan_sentinels=nan)
    return {k: to_np(t) for k, t in v.items()}


def run(w, vals, scale=None, fast=False):
    scale = 1.0 / math.sqrt(w.head_dim) if scale is None else scale
    f = oa.paged_attention_fast if fast else oa.paged_attention
    # the cache must already hold the new rows: write them the plain way (oracle.cache)
    from oracle.cache import reshape_and_cache
    kp, vp = reshape_and_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"],
                               w.block_table, w.q_lens, w.ctx_lens)
    return f(vals["q"], kp, vp, w.block_table, w.q_lens, w.ctx_lens, scale), kp, vp


# ---------------------------------------------------------------- packing and block counts
def test_packing_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "packing_worked_example.json")))
    cu = oa.pack_lengths(g["lengths"])
    assert cu.tolist() == g["cu_seqlens"]
    assert cu[-1] == g["packed_rows"]


def test_packing_rejects_empty_sequence():
    with pytest.raises(ValueError):
        oa.pack_lengths([3, 0, 2])


def test_block_counts_from_pages():
    g = json.load(open(os.path.join(GOLDEN, "block_counts.json")))
    for c in g["cases"]:
        assert oa.blocks_needed(c["tokens"], c["block_size"]) == c["blocks"], c["source"]


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_its_value_exactly():
    w = synth.custom_workload([1, 1], [1, 1], 4, 2, 64, 16, seed=3)
    vals = np_inputs(w)
    out, _, _ = run(w, vals)
    for t in range(2):
        for h in range(4):
            assert np.array_equal(out[t, h], vals["v_new"][t, h // 2])


def test_identical_keys_give_mean_of_values():
    w = synth.custom_workload([1], [37], 2, 1, 64, 16, seed=4)
    vals = np_inputs(w, nan=False)
    vals["k_pages"][:] = vals["k_pages"][0, 0, 0]          # every key equal
    vals["k_new"][:] = vals["k_pages"][0, 0, 0]
    out, kp, vp = run(w, vals)
    K, V = oa.gather_kv(kp, vp, w.block_table[0], 37, 16)
    assert np.allclose(out[0, 0], V[:, 0].mean(axis=0), atol=1e-13, rtol=0)
    assert np.allclose(out[0, 1], V[:, 0].mean(axis=0), atol=1e-13, rtol=0)


def test_zero_query_gives_causal_prefix_mean():
    """q = 0 makes every visible key weigh the same, so row i of a chunk over a cached prefix P
    equals the mean of V[0 .. P+i]. Pins the causal boundary and its bottom-right alignment."""
    w = synth.custom_workload([5, 1, 9], [21, 13, 9], 4, 2, 64, 16, seed=5)
    vals = np_inputs(w)
    vals["q"][:] = 0.0
    out, kp, vp = run(w, vals)
    cu = oa.pack_lengths(w.q_lens)
    for s in range(3):
        P = int(w.ctx_lens[s] - w.q_lens[s])
        K, V = oa.gather_kv(kp, vp, w.block_table[s], int(w.ctx_lens[s]), 16)
        csum = np.cumsum(V, axis=0)
        for i in range(int(w.q_lens[s])):
            for h in range(4):
                expect = csum[P + i, h // 2] / (P + i + 1)
                assert np.allclose(out[cu[s] + i, h], expect, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- invariants
def test_block_permutation_is_bitwise_invariant():
    w = synth.custom_workload([3, 1, 40], [50, 30, 40], 4, 2, 64, 16, seed=6, spare_blocks=3)
    vals = np_inputs(w)
    out, _, _ = run(w, vals)
    # move every physical block to a new id
    perm = np.random.default_rng(0).permutation(w.num_blocks)
    kp2 = np.empty_like(vals["k_pages"]); vp2 = np.empty_like(vals["v_pages"])
    kp2[perm] = vals["k_pages"]; vp2[perm] = vals["v_pages"]
    table2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1)
    w2 = synth.Workload(w.name, w.seed, w.q_lens, w.ctx_lens, 4, 2, 64, 16, "bf16",
                        table2.astype(np.int32), w.num_blocks)
    vals2 = dict(vals, k_pages=kp2, v_pages=vp2)
    out2, _, _ = run(w2, vals2)
    assert np.array_equal(out, out2)


def test_paged_equals_contiguous_bitwise():
    """Shuffled 16-token pages and one contiguous 256-token page per sequence hold the same
    logical K/V, so the outputs are bitwise equal."""
    qlen, ctx = [4, 1, 7], [60, 100, 7]
    w = synth.custom_workload(qlen, ctx, 4, 1, 64, 16, seed=7)
    vals = np_inputs(w)
    out, kp, vp = run(w, vals)
    # contiguous: sequence s occupies block s of a 256-slot pool, in order
    wc = synth.Workload("c", 0, w.q_lens, w.ctx_lens, 4, 1, 64, 256, "bf16",
                        np.arange(3, dtype=np.int32)[:, None], 3)
    kc = np.full((3, 1, 256, 64), np.nan); vc = np.full((3, 1, 256, 64), np.nan)
    for s in range(3):
        K, V = oa.gather_kv(kp, vp, w.block_table[s], ctx[s], 16)
        kc[s, :, :ctx[s]] = K.transpose(1, 0, 2); vc[s, :, :ctx[s]] = V.transpose(1, 0, 2)
    outc = oa.paged_attention(vals["q"], kc, vc, wc.block_table, wc.q_lens, wc.ctx_lens,
                              1 / 8.0)
    assert np.array_equal(out, outc)


def test_nan_in_unused_memory_leaves_output_unchanged():
    w = synth.custom_workload([2, 1], [19, 33], 2, 2, 64, 16, seed=8, spare_blocks=2, min_width=6)
    with_nan = np_inputs(w, nan=True)
    no_nan = np_inputs(w, nan=False)
    out1, _, _ = run(w, with_nan)
    out2, _, _ = run(w, no_nan)
    assert np.all(np.isfinite(out1))
    assert np.array_equal(out1, out2)


def test_gqa_equals_replicated_mha():
    w = synth.custom_workload([3, 1], [10, 20], 8, 2, 64, 16, seed=9)
    vals = np_inputs(w)
    out, kp, vp = run(w, vals)
    wr = synth.Workload("r", 0, w.q_lens, w.ctx_lens, 8, 8, 64, 16, "bf16", w.block_table,
                        w.num_blocks)
    kr = np.repeat(kp, 4, axis=1); vr = np.repeat(vp, 4, axis=1)
    outr = oa.paged_attention(vals["q"], kr, vr, wr.block_table, wr.q_lens, wr.ctx_lens, 1 / 8.0)
    assert np.array_equal(out, outr)


def test_decode_is_last_row_of_prefill_and_chunks_match_full_prefill():
    L = 45
    full = synth.custom_workload([L], [L], 2, 1, 64, 16, seed=10)
    vals = np_inputs(full, nan=False)
    out_full, kp, vp = run(full, vals)
    # decode: the last token alone over the whole (already cached) context
    d = oa.paged_attention(vals["q"][L - 1:L], kp, vp, full.block_table, [1], [L], 1 / 8.0)
    assert np.allclose(d[0], out_full[L - 1], atol=1e-14, rtol=0)
    # chunk: rows 30..44 over the cached prefix 0..29
    c = oa.paged_attention(vals["q"][30:L], kp, vp, full.block_table, [L - 30], [L], 1 / 8.0)
    assert np.allclose(c, out_full[30:L], atol=1e-14, rtol=0)


def test_packed_equals_per_sequence():
    w = synth.custom_workload([3, 1, 6], [9, 25, 6], 4, 2, 64, 16, seed=11)
    vals = np_inputs(w)
    out, kp, vp = run(w, vals)
    cu = oa.pack_lengths(w.q_lens)
    for s in range(3):
        one = oa.paged_attention(vals["q"][cu[s]:cu[s + 1]], kp, vp, w.block_table[s:s + 1],
                                 w.q_lens[s:s + 1], w.ctx_lens[s:s + 1], 1 / 8.0)
        assert np.array_equal(one, out[cu[s]:cu[s + 1]])


def test_vectorised_oracle_matches_row_loop():
    w = synth.custom_workload([7, 1, 33], [40, 70, 33], 4, 2, 64, 16, seed=12)
    vals = np_inputs(w)
    a, _, _ = run(w, vals)
    b, _, _ = run(w, vals, fast=True)
    assert np.allclose(a, b, atol=1e-13, rtol=0)


# ---------------------------------------------------------------- brute force via a library
def sdpa_reference(w, vals, kp, vp, scale):
    """Dense attention with an explicit [Lq, Lk] boolean mask through torch's float64 SDPA."""
    cu = oa.pack_lengths(w.q_lens)
    out = np.zeros_like(vals["q"])
    G = w.num_q_heads // w.num_kv_heads
    for s in range(w.num_seqs):
        ql, ctx = int(w.q_lens[s]), int(w.ctx_lens[s])
        K, V = oa.gather_kv(kp, vp, w.block_table[s], ctx, w.block_size)
        q = torch.from_numpy(vals["q"][cu[s]:cu[s + 1]]).permute(1, 0, 2)      # [Hq, Lq, D]
        k = torch.from_numpy(np.repeat(K, G, axis=1)).permute(1, 0, 2)         # [Hq, Lk, D]
        v = torch.from_numpy(np.repeat(V, G, axis=1)).permute(1, 0, 2)
        mask = torch.arange(ctx)[None, :] <= (ctx - ql + torch.arange(ql))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        out[cu[s]:cu[s + 1]] = o.permute(1, 0, 2).numpy()
    return out


@settings(max_examples=25, deadline=None, derandomize=True)
@given(st.lists(st.tuples(st.integers(1, 12), st.integers(0, 40)), min_size=1, max_size=4),
       st.sampled_from([(2, 1), (4, 2), (4, 4)]), st.sampled_from([16, 32]),
       st.integers(0, 2**16))
def test_brute_force_against_library_sdpa(lens, heads, bs, seed):
    q_lens = [a for a, _ in lens]
    ctx = [a + b for a, b in lens]
    w = synth.custom_workload(q_lens, ctx, heads[0], heads[1], 16, bs, seed=seed)
    vals = np_inputs(w, seed=seed)
    out, kp, vp = run(w, vals, scale=0.37)
    ref = sdpa_reference(w, vals, kp, vp, 0.37)
    assert np.allclose(out, ref, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- planted mistakes
def test_planted_off_by_one_causal_mistake_is_caught(monkeypatch):
    """An oracle that drops the row's own key must fail the prefix-mean pin."""
    real = oa.attend_rows

    def wrong(q_rows, K, V, first_pos, scale):
        return real(q_rows, K, V, max(first_pos - 1, 0), scale)

    monkeypatch.setattr(oa, "attend_rows", wrong)
    with pytest.raises(AssertionError):
        test_zero_query_gives_causal_prefix_mean()


def test_planted_kv_head_mixup_is_caught():
    """Reading the wrong kv head for a query head (here: the kv heads swapped) must fail the
    library brute force."""
    w = synth.custom_workload([2, 1], [6, 9], 4, 2, 16, 16, seed=1)
    vals = np_inputs(w)
    from oracle.cache import reshape_and_cache
    kp, vp = reshape_and_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"],
                               w.block_table, w.q_lens, w.ctx_lens)
    ref = sdpa_reference(w, vals, kp, vp, 0.5)
    kp_swapped = kp[:, ::-1].copy(); vp_swapped = vp[:, ::-1].copy()   # h%2 vs h//2 for Hq=4,Hkv=2
    bad = oa.paged_attention(vals["q"], kp_swapped, vp_swapped, w.block_table, w.q_lens,
                             w.ctx_lens, 0.5)
    assert not np.allclose(bad, ref, atol=1e-6)
