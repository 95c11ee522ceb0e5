"""Pins for the cache-write oracle and the task-table oracle. CPU only."""
import itertools

import numpy as np
import pytest

import synth
from oracle import attention as oa
from oracle import cache as oc
from oracle import task_table as ot
from tests.helpers import aliased_batch, to_np


# ---------------------------------------------------------------- reshape_and_cache
def test_scatter_round_trip_and_sentinels():
    w = synth.custom_workload([3, 1, 20], [40, 17, 20], 4, 2, 64, 16, seed=21, spare_blocks=4)
    v = {k: to_np(t) for k, t in synth.make_values(w, nan_sentinels=True).items()}
    kp, vp = oc.reshape_and_cache(v["k_new"], v["v_new"], v["k_pages"], v["v_pages"],
                                  w.block_table, w.q_lens, w.ctx_lens)
    cu = oa.pack_lengths(w.q_lens)
    changed = 0
    for s in range(w.num_seqs):
        ctx, ql = int(w.ctx_lens[s]), int(w.q_lens[s])
        K, V = oa.gather_kv(kp, vp, w.block_table[s], ctx, 16)
        # gather after write returns exactly the new rows at positions P .. ctx-1
        assert np.array_equal(K[ctx - ql:], v["k_new"][cu[s]:cu[s + 1]])
        assert np.array_equal(V[ctx - ql:], v["v_new"][cu[s]:cu[s + 1]])
        # and the cached prefix is untouched
        K0, V0 = oa.gather_kv(v["k_pages"], v["v_pages"], w.block_table[s], ctx - ql, 16)
        assert np.array_equal(K[:ctx - ql], K0) and np.array_equal(V[:ctx - ql], V0)
        changed += ql
    # exactly T*Hkv*D elements changed per tensor (the NaN sentinels they replaced)
    diff = ~((kp == v["k_pages"]) | (np.isnan(kp) & np.isnan(v["k_pages"])))
    assert diff.sum() == changed * 2 * 64
    # every slot outside the written ones keeps its previous content (NaN stays NaN)
    assert np.isnan(kp).sum() == np.isnan(v["k_pages"]).sum() - changed * 2 * 64


def test_scatter_never_touches_foreign_blocks():
    w = synth.custom_workload([1, 1], [16, 33], 2, 1, 64, 16, seed=22)
    v = {k: to_np(t) for k, t in synth.make_values(w, nan_sentinels=False).items()}
    kp, _ = oc.reshape_and_cache(v["k_new"], v["v_new"], v["k_pages"], v["v_pages"],
                                 w.block_table, w.q_lens, w.ctx_lens)
    own = {0: {int(w.block_table[0, 0])}, 1: set(int(b) for b in w.block_table[1, :3])}
    touched = {b for b in range(w.num_blocks) if not np.array_equal(kp[b], v["k_pages"][b])}
    # seq 0 writes slot 15 of its only block; seq 1 writes slot 0 of its third block
    assert touched == {int(w.block_table[0, 0]), int(w.block_table[1, 2])}
    assert touched <= own[0] | own[1]


# ---------------------------------------------------------------- task table
def P(**kw):
    base = dict(num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=16, dec_split=64,
                pf_q_tile=2, pf_kv_split=0, num_workers=2)
    base.update(kw)
    return ot.Params(**base)


def test_hand_derived_table():
    """One decode sequence (ctx 100) and one 3-row prefill (ctx 3), Hq=2, Hkv=1 (G=2),
    dec_split 64, pf_q_tile 2, no prefill key split. Derived by hand:
      decode seq 0, kv head 0: splits [0,64) and [64,100); 2 splits -> combine, slots 0..3;
        loads 64*2 = 128 and 36*2 = 72
      prefill seq 1 (P = 0), head h, rows [0,2): keys visible 1 + 2 = 3; rows [2,3): 3
    Emission order: d0(128), d1(72), h0r0(3), h0r2(3), h1r0(3), h1r2(3) -- already sorted."""
    tasks, comb, npart, loads, bal = ot.build_task_table(P(), [0, 1, 4], [100, 3])
    assert tasks.tolist() == [
        [0, 0, 0, 0, 1, 0, 64, 0],
        [0, 0, 0, 0, 1, 64, 100, 2],
        [1, 1, 0, 0, 2, 0, 2, -1],
        [1, 1, 0, 2, 1, 0, 3, -1],
        [1, 1, 1, 0, 2, 0, 2, -1],
        [1, 1, 1, 2, 1, 0, 3, -1]]
    assert loads.tolist() == [128, 72, 3, 3, 3, 3]
    assert comb.tolist() == [[0, 0, 1, 0, 2, 0, 2, 0]]
    assert npart == 4
    # modulo: worker0 128+3+3 = 134, worker1 72+3+3 = 78
    assert bal["modulo"] == pytest.approx(78 / 134)
    # snake: round0 -> w0 128, w1 72; round1 -> w1 3, w0 3; round2 -> w0 3, w1 3
    assert bal["snake"] == pytest.approx(78 / 134)


def test_hand_derived_verify_table():
    """A 3-row draft (ctx 100, so P = 97) with Hq=4, Hkv=2 (G=2), dec_split 64, verify_rows 4.
    Derived by hand: per kv head g, splits [0,64) and [64,100), each covering rows 0..2 and
    heads 2g, 2g+1 (6 columns); 2 splits -> one combine per g with 2*3*2 = 12 slots.
      split [0,64): rows see 98, 99, 100 keys -> 64 each -> 192 pairs x G = 384
      split [64,100): 34 + 35 + 36 = 105 pairs x G = 210
    Emission g0s0, g0s1, g1s0, g1s1; stable descending order g0s0, g1s0, g0s1, g1s1."""
    p = P(num_q_heads=4, num_kv_heads=2, verify_rows=4)
    tasks, comb, npart, loads, _ = ot.build_task_table(p, [0, 3], [100])
    assert tasks.tolist() == [
        [2, 0, 0, 0, 3, 0, 64, 0],
        [2, 0, 1, 0, 3, 0, 64, 12],
        [2, 0, 0, 0, 3, 64, 100, 6],
        [2, 0, 1, 0, 3, 64, 100, 18]]
    assert loads.tolist() == [384, 384, 210, 210]
    assert comb.tolist() == [[0, 0, 3, 0, 2, 0, 2, 0], [0, 0, 3, 2, 2, 12, 2, 0]]
    assert npart == 24


def test_verify_selection_rule():
    """verify_rows 0 keeps prefill tiles; a q_len above verify_rows, or G*q_len above 16
    columns, also stays a prefill tile; q_len 1 is always a decode task."""
    cu, ctx = [0, 3], [100]
    for p in (P(num_q_heads=4, num_kv_heads=2),                       # off
              P(num_q_heads=4, num_kv_heads=2, verify_rows=2),        # 3 rows > 2
              P(num_q_heads=16, num_kv_heads=2, verify_rows=4)):      # G*3 = 24 > 16
        tasks, *_ = ot.build_task_table(p, cu, ctx)
        assert set(tasks[:, 0].tolist()) == {1}
    tasks, *_ = ot.build_task_table(P(num_q_heads=4, num_kv_heads=1, verify_rows=4), cu, ctx)
    assert set(tasks[:, 0].tolist()) == {2}                          # G*3 = 12 columns
    tasks, *_ = ot.build_task_table(P(num_q_heads=4, num_kv_heads=2, verify_rows=4), [0, 1], [9])
    assert set(tasks[:, 0].tolist()) == {0}
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(verify_rows=1), cu, ctx)
    assert e.value.code == ot.ERR_SHAPE
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(verify_rows=17), cu, ctx)
    assert e.value.code == ot.ERR_SHAPE


def test_balance_examples():
    """Four equal-shape decode tasks with loads 4,3,2,1 (x G) on two workers:
    modulo deals w0 = 4+2, w1 = 3+1; snake deals w0 = 4+1, w1 = 3+2."""
    p = ot.Params(1, 1, 64, 16, dec_split=256, num_workers=2)   # one split per sequence
    tasks, comb, npart, loads, bal = ot.build_task_table(p, [0, 1, 2, 3, 4], [256, 192, 128, 64])
    assert loads.tolist() == [256, 192, 128, 64]
    assert bal["modulo"] == pytest.approx((192 + 64) / (256 + 128))
    assert bal["snake"] == pytest.approx(1.0)


def test_stable_descending_order_with_ties():
    p = P(num_q_heads=4, num_kv_heads=2, pf_q_tile=4)
    tasks, _, _, loads, _ = ot.build_task_table(p, [0, 1, 2, 6], [64, 64, 10])
    assert np.all(np.diff(loads) <= 0)
    for a, b, la, lb in zip(tasks[:-1], tasks[1:], loads[:-1], loads[1:]):
        if la == lb:   # ties keep emission order: (seq, head, q_row0, kv0) ascending
            assert (a[1], a[2], a[3], a[5]) < (b[1], b[2], b[3], b[5])


def coverage(p, cu, ctx, tasks):
    """Count how often each (seq, query head, row, key) pair is covered by the tasks."""
    G = p.num_q_heads // p.num_kv_heads
    cnt = {}
    for kind, s, head, r0, rows, kv0, kv1, _ in tasks.tolist():
        heads = range(head * G, head * G + G) if kind in (0, 2, 3) else [head]
        # a shared-prefix task covers row 0 of `rows` consecutive sequences
        cells = [(s + i, 0) for i in range(rows)] if kind == 3 else \
            [(s, i) for i in range(r0, r0 + rows)]
        for h, (sq, i) in itertools.product(heads, cells):
            P_ = ctx[sq] - (cu[sq + 1] - cu[sq])
            for j in range(kv0, min(kv1, P_ + i + 1)):
                cnt[(sq, h, i, j)] = cnt.get((sq, h, i, j), 0) + 1
    return cnt


@pytest.mark.parametrize("pf_kv_split,pf_q_tile,dec_split,verify_rows",
                         [(0, 3, 64, 0), (64, 5, 128, 0), (128, 128, 64, 0), (64, 5, 64, 4),
                          (0, 128, 128, 8)])
def test_coverage_and_load_identities(pf_kv_split, pf_q_tile, dec_split, verify_rows):
    rng = np.random.default_rng(pf_kv_split + pf_q_tile + verify_rows)
    q_lens = [1, 7, 1, 19, 1, 2, 4, 3]
    ctx = [int(rng.integers(1, 300)) if q == 1 else q + int(rng.integers(0, 200)) for q in q_lens]
    cu = oa.pack_lengths(q_lens).tolist()
    p = P(num_q_heads=4, num_kv_heads=2, pf_q_tile=pf_q_tile, pf_kv_split=pf_kv_split,
          dec_split=dec_split, num_workers=3, verify_rows=verify_rows)
    tasks, comb, npart, loads, _ = ot.build_task_table(p, cu, ctx)
    cnt = coverage(p, cu, ctx, tasks)
    expect = {(s, h, i, j) for s in range(len(q_lens)) for h in range(4)
              for i in range(q_lens[s]) for j in range(ctx[s] - q_lens[s] + i + 1)}
    assert set(cnt) == expect and all(v == 1 for v in cnt.values())
    # load identities: decode = sum ctx * Hq ; prefill and verify = Hq * sum_i (P + i + 1)
    dec = sum(l for t, l in zip(tasks.tolist(), loads) if t[0] == 0)
    multi = sum(l for t, l in zip(tasks.tolist(), loads) if t[0] in (1, 2))
    assert dec == sum(c * 4 for q, c in zip(q_lens, ctx) if q == 1)
    assert multi == sum(4 * sum(c - q + i + 1 for i in range(q))
                        for q, c in zip(q_lens, ctx) if q > 1)
    verify_seqs = {t[1] for t in tasks.tolist() if t[0] == 2}
    assert verify_seqs == {s for s, q in enumerate(q_lens) if 2 <= q <= verify_rows}
    # every task has at least one unmasked pair
    assert np.all(loads > 0)
    # partial rows: each used exactly once, all below num_partials, consistent with combines
    used = []
    for kind, s, head, r0, rows, kv0, kv1, part in tasks.tolist():
        if part >= 0:
            used += list(range(part, part + (rows * 2 if kind in (0, 2) else rows)))
    assert sorted(used) == list(range(npart))
    assert npart == sum(c[2] * c[4] * c[6] for c in comb.tolist())


def test_validation_codes():
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(block_size=12), [0, 1], [5])      # page size 12: rejected
    assert e.value.code == ot.ERR_BLOCK_SIZE
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(), [0, 2, 2], [5, 5])             # empty sequence
    assert e.value.code == ot.ERR_INPUT
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(), [0, 4], [3])                   # context shorter than rows
    assert e.value.code == ot.ERR_INPUT
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(num_q_heads=3, num_kv_heads=2), [0, 1], [3])
    assert e.value.code == ot.ERR_SHAPE


def test_empty_batch():
    tasks, comb, npart, loads, bal = ot.build_task_table(P(), [0], [])
    assert tasks.shape == (0, 8) and comb.shape == (0, 8) and npart == 0


# ---- shared prefixes (blocks aliased between neighbouring decode sequences) ----

def test_hand_derived_shared_table():
    """Three decode sequences, ctx 100, 90, 120, bs 16, Hq=2, Hkv=1 (G=2, 8 sequences per
    shared task), dec_split 64, shared_min 64. Block rows:
      s0: 0 1 2 3 4 5 6      s1: 0 1 2 3 4 7 8      s2: 0 1 2 3 9 10 11 12
    s0/s1 share 5 blocks (80 keys -> 64), s1/s2 share 4 (64): one group, L = 64, one column
    set of 3 members. S = 1 shared piece [0, 64); own pieces [64, 100), [64, 90), [64, 120)
    (U = 1 each); W = (1 + 1) * 2 = 4, base 0: member i owns rows 4i .. 4i+3.
    Emission: combines s0, s1, s2; shared task (load 64*3*2 = 384); s0 (36*2 = 72),
    s1 (26*2 = 52), s2 (56*2 = 112). Sorted: 384, 112, 72, 52."""
    bt = np.array([[0, 1, 2, 3, 4, 5, 6, -1], [0, 1, 2, 3, 4, 7, 8, -1],
                   [0, 1, 2, 3, 9, 10, 11, 12]])
    p = P(shared_min=64)
    tasks, comb, npart, loads, _ = ot.build_task_table(p, [0, 1, 2, 3], [100, 90, 120], bt)
    assert tasks.tolist() == [
        [3, 0, 0, 4, 3, 0, 64, 0],
        [0, 2, 0, 0, 1, 64, 120, 10],
        [0, 0, 0, 0, 1, 64, 100, 2],
        [0, 1, 0, 0, 1, 64, 90, 6]]
    assert loads.tolist() == [384, 112, 72, 52]
    assert comb.tolist() == [[0, 0, 1, 0, 2, 0, 2, 0], [1, 0, 1, 0, 2, 4, 2, 0],
                             [2, 0, 1, 0, 2, 8, 2, 0]]
    assert npart == 12
    # sharing off: the plain table, whatever the block table holds
    plain = ot.build_task_table(P(), [0, 1, 2, 3], [100, 90, 120])
    off = ot.build_task_table(P(), [0, 1, 2, 3], [100, 90, 120], bt)
    assert np.array_equal(plain[0], off[0]) and np.array_equal(plain[1], off[1])


def test_shared_rules():
    bt = np.array([[0, 1, 2, 3, 4, 5, 6, -1], [0, 1, 2, 3, 4, 7, 8, -1]])
    # below shared_min: no group
    tasks, *_ = ot.build_task_table(P(shared_min=128), [0, 1, 2], [100, 90], bt)
    assert 3 not in tasks[:, 0]
    # a prefill neighbour breaks the run
    tasks, *_ = ot.build_task_table(P(shared_min=64), [0, 1, 3], [100, 90], bt)
    assert 3 not in tasks[:, 0]
    # G = 16: one sequence per 16 columns, no sharing
    tasks, *_ = ot.build_task_table(P(num_q_heads=16, shared_min=64), [0, 1, 2], [100, 90], bt)
    assert 3 not in tasks[:, 0]
    # a shared block that receives a new row is an input error
    bad = np.array([[0, 1, 2], [0, 1, 5]])
    tasks, *_ = ot.build_task_table(P(shared_min=32 * 2), [0, 1, 2], [40, 48], bad)
    assert 3 not in tasks[:, 0]                   # each writes its own block 2; 32 keys shared
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(shared_min=64), [0, 1, 2], [40, 48], np.array([[0, 1, 2]] * 2))
    assert e.value.code == ot.ERR_INPUT           # both write physical block 2
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(shared_min=64), [0, 1, 2], [32, 48], bad)   # s0 writes block 1
    assert e.value.code == ot.ERR_INPUT
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(shared_min=64), [0, 1, 2], [100, 90])       # no block table
    assert e.value.code == ot.ERR_INPUT
    with pytest.raises(ot.TaskTableError) as e:
        ot.build_task_table(P(shared_min=32), [0, 1, 2], [100, 90], bt)
    assert e.value.code == ot.ERR_SHAPE


def test_shared_column_sets_are_balanced():
    """G = 4 gives 4 sequences per shared task: a group of 9 becomes sets of 3, 3, 3 and a
    group of 6 sets of 3 and 3."""
    for n, sizes in ((9, [3, 3, 3]), (6, [3, 3]), (4, [4]), (5, [3, 2])):
        bt = np.array([[0, 1, 2, 3, 100 + s] for s in range(n)])
        p = P(num_q_heads=4, shared_min=64)
        tasks, *_ = ot.build_task_table(p, list(range(n + 1)), [70] * n, bt)
        got = sorted(((t[1], t[4]) for t in tasks.tolist() if t[0] == 3))
        assert [r for _, r in got] == sizes
        assert [f for f, _ in got] == list(np.cumsum([0] + sizes[:-1]))


@pytest.mark.parametrize("seed,G,bs,dec_split,shared_min",
                         [(1, 1, 16, 64, 64), (2, 2, 16, 128, 64), (3, 4, 32, 64, 128),
                          (4, 8, 64, 64, 64), (5, 1, 16, 64, 192)])
def test_shared_coverage_and_partials(seed, G, bs, dec_split, shared_min):
    rng = np.random.default_rng(seed)
    q_lens, ctx, bt = aliased_batch(rng, bs, 8)
    cu = oa.pack_lengths(q_lens).tolist()
    hkv = 2
    p = P(num_q_heads=hkv * G, num_kv_heads=hkv, block_size=bs, dec_split=dec_split,
          pf_q_tile=3, verify_rows=4, shared_min=shared_min, num_workers=5)
    _check_shared_table(p, cu, ctx, bt, q_lens, G)


def _check_shared_table(p, cu, ctx, bt, q_lens, G):
    bs, hkv = p.block_size, p.num_kv_heads
    tasks, comb, npart, loads, _ = ot.build_task_table(p, cu, ctx, bt)
    assert 3 in tasks[:, 0]
    cnt = coverage(p, cu, ctx, tasks)
    hq = hkv * G
    expect = {(s, h, i, j) for s in range(len(q_lens)) for h in range(hq)
              for i in range(q_lens[s]) for j in range(ctx[s] - q_lens[s] + i + 1)}
    assert set(cnt) == expect and all(v == 1 for v in cnt.values())
    # loads: pairs x heads, whatever task covers them
    assert int(loads.sum()) == len(expect)
    # shared tasks: members are consecutive decode sequences that really alias [0, kv1)
    for kind, s, head, W, rows, kv0, kv1, part in tasks.tolist():
        if kind == 3:
            for m in range(s, s + rows):
                assert q_lens[m] == 1 and kv1 <= ctx[m] - 1
                nb = -(-kv1 // bs)
                assert np.array_equal(bt[m, :nb], bt[s, :nb])
    # partial rows: written once each; every combine slot reads exactly the written rows
    written = []
    for kind, s, head, W, rows, kv0, kv1, part in tasks.tolist():
        if part < 0:
            continue
        if kind == 3:
            written += [part + i * W + j for i in range(rows) for j in range(G)]
        elif kind in (0, 2):
            written += list(range(part, part + rows * G))
        else:
            written += list(range(part, part + rows))
    assert len(written) == len(set(written)) and max(written) < npart
    read = []
    for sq, r0, rows, head, heads, first, n, _ in comb.tolist():
        read += [first + k * rows * heads + i for k in range(n) for i in range(rows * heads)]
    assert sorted(read) == sorted(written)


def test_planted_shared_length_mistake_is_caught(monkeypatch):
    """An oracle whose pairwise shared length runs one 64-key step past the aliased blocks
    must fail the aliasing pin."""
    rng = np.random.default_rng(1)
    q_lens, ctx, bt = aliased_batch(rng, 16, 8)
    cu = oa.pack_lengths(q_lens).tolist()
    p = P(num_q_heads=2, num_kv_heads=2, block_size=16, dec_split=64, pf_q_tile=3,
          verify_rows=4, shared_min=64, num_workers=5)
    _check_shared_table(p, cu, ctx, bt, q_lens, 1)
    real = ot.shared_keys_with_previous
    monkeypatch.setattr(ot, "shared_keys_with_previous",
                        lambda *a: [v + 64 if v > 0 else v for v in real(*a)])
    with pytest.raises(AssertionError):
        _check_shared_table(p, cu, ctx, bt, q_lens, 1)
