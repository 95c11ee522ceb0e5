"""Host-side checks of SmoothGEMM's C ABI (no GPU needed): the Linear decomposition must match
the oracle's bit for bit, errors must agree with it, and the launcher's scalar checks run
before any HIP call."""
import ctypes

import numpy as np
import pytest

import synth
import paged_variable_length_amd as pa
from paged_variable_length_amd import _abi
from oracle import gemm as og


def _both(M, N, K, tile, k_split, workers, tail=False):
    g = pa.build_gemm_table(M, N, K, tile, k_split, workers, tail)
    t, r, ns, _, bal = og.decompose_linear(og.GemmParams(tile, k_split, workers, int(tail)),
                                           M, N, K)
    return g, (t, r, ns, bal)


@pytest.mark.parametrize("M,N,K,tile,k_split", [
    (300, 200, 200, 256, 128), (130, 260, 70, 128, 0), (513, 700, 1000, 256, 192),
    (1, 1, 1, 128, 0), (1024, 1024, 1024, 256, 0), (512, 2048, 1024, 128, 256),
    (2048, 512, 2048, 256, 64), (0, 5, 5, 256, 0), (7, 0, 3, 128, 64)])
def test_gemm_table_bit_exact(M, N, K, tile, k_split):
    g, (t, r, ns, bal) = _both(M, N, K, tile, k_split, 7)
    assert np.array_equal(g.tasks, t) and np.array_equal(g.reduces, r) and g.num_slots == ns
    assert g.balance_snake == pytest.approx(bal["snake"], abs=1e-12)
    assert g.balance_modulo == pytest.approx(bal["modulo"], abs=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_gemm_table_bit_exact_random(seed):
    rng = np.random.default_rng(seed)
    for _ in range(8):
        M, N, K = (int(x) for x in rng.integers(1, 3000, size=3))
        tile = int(rng.choice([128, 256]))
        k_split = int(rng.choice([0, 64, 192, 1024]))
        g, (t, r, ns, _) = _both(M, N, K, tile, k_split, int(rng.integers(1, 600)))
        assert np.array_equal(g.tasks, t) and np.array_equal(g.reduces, r) and g.num_slots == ns


@pytest.mark.parametrize("seed", range(4))
def test_gemm_table_tail_split_bit_exact_random(seed):
    rng = np.random.default_rng(100 + seed)
    for _ in range(12):
        M, N, K = (int(x) for x in rng.integers(1, 4000, size=3))
        tile = int(rng.choice([128, 256]))
        g, (t, r, ns, bal) = _both(M, N, K, tile, 0, int(rng.integers(1, 700)), tail=True)
        assert np.array_equal(g.tasks, t) and np.array_equal(g.reduces, r) and g.num_slots == ns
        assert g.balance_snake == pytest.approx(bal["snake"], abs=1e-12)


def test_gemm_table_tail_split_on_the_bench_shapes():
    for name in synth.GEMM_SHAPES:
        M, N, K = synth.gemm_shape(name)
        for tile in (128, 256):
            g, (t, r, ns, _) = _both(M, N, K, tile, 0, 256, tail=True)
            assert np.array_equal(g.tasks, t) and np.array_equal(g.reduces, r) and g.num_slots == ns


def test_gemm_table_on_the_bench_shapes():
    for name in synth.GEMM_SHAPES:
        M, N, K = synth.gemm_shape(name)
        g, (t, r, ns, _) = _both(M, N, K, 256, 0, 256)
        assert np.array_equal(g.tasks, t) and ns == 0 and len(r) == 0


def test_gemm_table_errors_match_oracle():
    L = _abi.lib()
    cases = [(64, 0, 1, 4, 4, 4), (256, 32, 1, 4, 4, 4), (256, 0, 0, 4, 4, 4),
             (256, 0, 1, 4, 4, 0), (256, 0, 1, -1, 4, 4)]
    for tile, ks, W, M, N, K in cases:
        with pytest.raises(og.GemmTableError) as e:
            og.decompose_linear(og.GemmParams(tile, ks, W), M, N, K)
        nt, nr, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        rc = L.build_gemm_table(ctypes.byref(_abi.PaGemmParams(tile, ks, W, 0)), M, N, K, None, 0,
                                ctypes.byref(nt), None, 0, ctypes.byref(nr), ctypes.byref(ns),
                                None)
        assert rc == e.value.code == _abi.PA_ERR_SHAPE
    nt, nr, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    for bad in (_abi.PaGemmParams(256, 0, 1, 2), _abi.PaGemmParams(256, 64, 1, 1)):
        rc = L.build_gemm_table(ctypes.byref(bad), 4, 4, 4, None, 0, ctypes.byref(nt), None, 0,
                                ctypes.byref(nr), ctypes.byref(ns), None)
        assert rc == _abi.PA_ERR_SHAPE  # tail_split is 0, or 1 with k_split 0
    assert L.build_gemm_table(None, 4, 4, 4, None, 0, None, None, 0, None, None, None) == \
        _abi.PA_ERR_NULL


def test_gemm_table_capacity_sizing():
    L = _abi.lib()
    nt, nr, ns = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = L.build_gemm_table(ctypes.byref(_abi.PaGemmParams(128, 64, 4, 0)), 300, 200, 200, None, 0,
                            ctypes.byref(nt), None, 0, ctypes.byref(nr), ctypes.byref(ns), None)
    assert rc == _abi.PA_ERR_CAPACITY
    # 3 x 2 output blocks, 4 K pieces each
    assert (nt.value, nr.value, ns.value) == (24, 6, 24)


def test_gemm_workspace_bytes():
    assert pa.gemm_workspace_bytes(0, 256) == 0
    assert pa.gemm_workspace_bytes(3, 256) == 3 * 256 * 256 * 4
    assert pa.gemm_workspace_bytes(1, 128) == 128 * 128 * 4
    assert pa.gemm_workspace_bytes(2, 64) == 0


def test_gemm_launcher_scalar_errors_need_no_gpu():
    L = _abi.lib()
    nul = None
    assert L.smooth_gemm(nul, nul, nul, 4, 4, 4, 64, nul, 1, nul, 0, 0, nul, 0, nul) == \
        _abi.PA_ERR_SHAPE                                                  # tile 64
    assert L.smooth_gemm(nul, nul, nul, -1, 4, 4, 256, nul, 1, nul, 0, 0, nul, 0, nul) == \
        _abi.PA_ERR_SHAPE                                                  # negative M
    assert L.smooth_gemm(nul, nul, nul, 4, 4, 4, 256, nul, 0, nul, 0, 0, nul, 0, nul) == \
        _abi.PA_OK                                                         # no tasks: no-op
    assert L.smooth_gemm(nul, nul, nul, 4, 4, 4, 256, nul, 1, nul, 0, 0, nul, 0, nul) == \
        _abi.PA_ERR_NULL
    p = ctypes.c_void_p(256)
    assert L.smooth_gemm(p, p, p, 4, 4, 4, 256, p, 2, p, 1, 2, p, 16, nul) == \
        _abi.PA_ERR_CAPACITY                                               # workspace too small
    assert b"workspace" in L.pa_last_error()
    # launch limits: 2^23 tasks, or reduces whose 64 workgroups each (tile 256) pass 2^23 - 1
    assert L.smooth_gemm(p, p, p, 4, 4, 4, 256, p, 1 << 23, nul, 0, 0, nul, 0, nul) == \
        _abi.PA_ERR_SHAPE
    assert L.smooth_gemm(p, p, p, 4, 4, 4, 256, p, 1, p, 1 << 17, 1, p, 1 << 40, nul) == \
        _abi.PA_ERR_SHAPE
    assert L.smooth_gemm(p, p, p, 4, 4, 4, 128, p, 1, p, 1 << 17, 1, p, 0, nul) == \
        _abi.PA_ERR_CAPACITY                                               # 16 per record: fits
