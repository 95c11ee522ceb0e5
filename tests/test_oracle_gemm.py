"""Pins for the SmoothGEMM oracle (product definition and task decomposition). CPU only."""
import numpy as np
import pytest

from oracle import gemm as og


def test_matmul_is_the_triple_loop():
    rng = np.random.default_rng(0)
    for M, N, K in ((1, 1, 1), (7, 13, 5), (3, 4, 9)):
        a = rng.standard_normal((M, K))
        w = rng.standard_normal((N, K))
        ref = np.zeros((M, N))
        for i in range(M):
            for j in range(N):
                for k in range(K):
                    ref[i, j] += a[i, k] * w[j, k]
        assert np.allclose(og.matmul(a, w), ref, rtol=0, atol=1e-12)


def test_matmul_closed_forms():
    a = np.arange(12.0).reshape(3, 4)
    assert np.array_equal(og.matmul(a, np.eye(4)), a)                 # W = I
    u, v = np.array([1.0, 2.0, 3.0]), np.array([4.0, 5.0])
    # rank one: A = u 1^T, W = v 1^T over K = 6 gives C = 6 u v^T
    assert np.array_equal(og.matmul(np.outer(u, np.ones(6)), np.outer(v, np.ones(6))),
                          6 * np.outer(u, v))
    assert og.matmul(a, a)[1, 2] == sum(a[1, k] * a[2, k] for k in range(4))   # W not = A^T


def test_hand_derived_table():
    """M=300, N=200, K=200, tile 256, k_split 128. Output blocks: rows [0,256) and [256,300)
    (44 rows), one column block of 200; K pieces [0,128), [128,200).
      block (0,0): loads 256*200*128 = 6553600 and 256*200*72 = 3686400, slots 0, 1
      block (256,0): 44*200*128 = 1126400 and 44*200*72 = 633600, slots 2, 3
    Sorted: 6553600, 3686400, 1126400, 633600 (already in emission order)."""
    tasks, red, slots, loads, bal = og.decompose_linear(og.GemmParams(256, 128, 2), 300, 200, 200)
    assert tasks.tolist() == [[0, 256, 0, 200, 0, 128, 0, 0], [0, 256, 0, 200, 128, 200, 1, 0],
                              [256, 44, 0, 200, 0, 128, 2, 0], [256, 44, 0, 200, 128, 200, 3, 0]]
    assert loads.tolist() == [6553600, 3686400, 1126400, 633600]
    assert red.tolist() == [[0, 256, 0, 200, 0, 2, 0, 0], [256, 44, 0, 200, 2, 2, 0, 0]]
    assert slots == 4
    # modulo on 2 workers: w0 = 6553600 + 1126400, w1 = 3686400 + 633600
    assert bal["modulo"] == pytest.approx((3686400 + 633600) / (6553600 + 1126400))


def test_no_split_writes_directly_and_sorts_edges_last():
    tasks, red, slots, loads, _ = og.decompose_linear(og.GemmParams(128, 0), 130, 260, 70)
    assert red.shape == (0, 8) and slots == 0 and np.all(tasks[:, 6] == -1)
    assert np.all(np.diff(loads) <= 0)
    assert tasks[0].tolist() == [0, 128, 0, 128, 0, 70, -1, 0]
    assert tasks[-1].tolist() == [128, 2, 256, 4, 0, 70, -1, 0]     # the 2 x 4 corner


@pytest.mark.parametrize("M,N,K,tile,k_split", [(1, 1, 1, 128, 0), (257, 129, 300, 128, 64),
                                                (513, 700, 1000, 256, 192), (64, 1000, 65, 256, 64)])
def test_coverage_and_loads(M, N, K, tile, k_split):
    tasks, red, slots, loads, _ = og.decompose_linear(og.GemmParams(tile, k_split, 7), M, N, K)
    cover = np.zeros((M, N, K), dtype=np.int32)
    for m0, rows, n0, cols, k0, k1, slot, _ in tasks.tolist():
        assert rows == min(tile, M - m0) and cols == min(tile, N - n0)
        cover[m0:m0 + rows, n0:n0 + cols, k0:k1] += 1
    assert np.all(cover == 1)
    assert int(loads.sum()) == M * N * K
    used = sorted(t[6] for t in tasks.tolist() if t[6] >= 0)
    assert used == list(range(slots))
    assert slots == sum(r[5] for r in red.tolist())
    # every output block with a split has one reduce record over exactly its slots
    for m0, rows, n0, cols, first, n, _, _ in red.tolist():
        mine = sorted(t[6] for t in tasks.tolist() if t[0] == m0 and t[2] == n0)
        assert mine == list(range(first, first + n))


def test_hand_derived_tail_split():
    """M=N=512, K=1000, tile 256, 3 workers, tail_split. Four equal blocks: one full round of 3
    whole blocks, r = 4 mod 3 = 1 left over, p = min(3 // 1, ceil(1000/64) = 16) = 3 pieces of
    ceil(1000/3) = 334 -> 384 keys: [0,384), [384,768), [768,1000). The tail block is the last
    of the load-sorted whole blocks: all loads tie, so the last in emission order, (256, 256).
    Loads: whole 256*256*1000 = 65536000; pieces 25165824, 25165824, 15204352."""
    tasks, red, slots, loads, _ = og.decompose_linear(og.GemmParams(256, 0, 3, 1), 512, 512, 1000)
    assert tasks.tolist() == [[0, 256, 0, 256, 0, 1000, -1, 0], [0, 256, 256, 256, 0, 1000, -1, 0],
                              [256, 256, 0, 256, 0, 1000, -1, 0],
                              [256, 256, 256, 256, 0, 384, 0, 0],
                              [256, 256, 256, 256, 384, 768, 1, 0],
                              [256, 256, 256, 256, 768, 1000, 2, 0]]
    assert loads.tolist() == [65536000] * 3 + [25165824, 25165824, 15204352]
    assert red.tolist() == [[256, 256, 256, 256, 0, 3, 0, 0]] and slots == 3


def test_tail_split_cases():
    # a whole number of rounds: nothing to cut
    t, r, ns, _, _ = og.decompose_linear(og.GemmParams(128, 0, 4, 1), 256, 256, 512)
    assert len(t) == 4 and ns == 0
    # r > W / 2: p = 1, nothing to cut
    t, r, ns, _, _ = og.decompose_linear(og.GemmParams(128, 0, 5, 1), 384, 384, 512)
    assert len(t) == 9 and ns == 0
    # fewer blocks than workers: all are cut; pieces capped by ceil(K / 64)
    t, r, ns, _, _ = og.decompose_linear(og.GemmParams(128, 0, 64, 1), 128, 256, 100)
    assert sorted((x[4], x[5]) for x in t.tolist()) == [(0, 64), (0, 64), (64, 100), (64, 100)]
    # edge blocks are lighter, sort last and are the ones cut: 3 x 2 blocks, 4 workers
    t, r, ns, _, _ = og.decompose_linear(og.GemmParams(256, 0, 4, 1), 600, 512, 640)
    cut = {(x[0], x[2]) for x in t.tolist() if x[6] >= 0}
    assert cut == {(512, 0), (512, 256)}


@pytest.mark.parametrize("M,N,K,tile,W", [(1, 1, 1, 128, 7), (257, 129, 300, 128, 5),
                                          (513, 700, 1000, 256, 3), (1000, 64, 4097, 128, 40)])
def test_tail_split_coverage(M, N, K, tile, W):
    """Every (m, n, k) is covered once, pieces are multiples of 64 but the last, and the tasks
    after the last whole round number at most W."""
    tasks, red, slots, loads, _ = og.decompose_linear(og.GemmParams(tile, 0, W, 1), M, N, K)
    cover = np.zeros((M, N, K), dtype=np.int32)
    for m0, rows, n0, cols, k0, k1, slot, _ in tasks.tolist():
        cover[m0:m0 + rows, n0:n0 + cols, k0:k1] += 1
        assert k0 % 64 == 0 and (k1 == K or (k1 - k0) % 64 == 0)
    assert np.all(cover == 1) and int(loads.sum()) == M * N * K
    T = -(-M // tile) * -(-N // tile)
    assert len(tasks) - (T // W) * W <= W
    assert slots == sum(x[5] for x in red.tolist())


def test_errors():
    for p in (og.GemmParams(64, 0), og.GemmParams(256, 32), og.GemmParams(256, 0, 0),
              og.GemmParams(256, 64, 4, 1), og.GemmParams(256, 0, 4, 2)):
        with pytest.raises(og.GemmTableError) as e:
            og.decompose_linear(p, 4, 4, 4)
        assert e.value.code == og.ERR_SHAPE
    with pytest.raises(og.GemmTableError) as e:
        og.decompose_linear(og.GemmParams(), 4, 4, 0)
    assert e.value.code == og.ERR_SHAPE
    tasks, red, slots, _, _ = og.decompose_linear(og.GemmParams(), 0, 5, 5)
    assert tasks.shape == (0, 8) and slots == 0
