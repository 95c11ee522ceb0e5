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


def test_errors():
    for p in (og.GemmParams(64, 0), og.GemmParams(256, 32), og.GemmParams(256, 0, 0)):
        with pytest.raises(og.GemmTableError) as e:
            og.decompose_linear(p, 4, 4, 4)
        assert e.value.code == og.ERR_SHAPE
    with pytest.raises(og.GemmTableError) as e:
        og.decompose_linear(og.GemmParams(), 4, 4, 0)
    assert e.value.code == og.ERR_SHAPE
    tasks, red, slots, _, _ = og.decompose_linear(og.GemmParams(), 0, 5, 5)
    assert tasks.shape == (0, 8) and slots == 0
