"""GPU parity of SmoothGEMM (C = A W^T, bf16 in, fp32 accumulation, bf16 out) through the C ABI
against the fp64 oracle product on the same seeded operands.

Tolerance (a reading: the pages state none for the Linear kernel). The kernel's result is the
exact product up to fp32 accumulation over K terms, at most K * 2^-24 * sum_k |a_k w_k|, and the
final rounding to bf16, at most 2^-9 |C|. The test allows 2^-8 |C| + 2^-20 sum_k |a_k w_k|:
twice the rounding term, and for K <= 16384 at least four times the accumulation term. A
dropped, repeated or zero-filled reduction chunk of 8 terms moves an element by about
sqrt(8) * 1 while 2^-8 |C| stays below 1 for |C| < 256, so such a mistake fails.

Every C sits inside a larger buffer whose guard region is filled with a sentinel, so a store
outside [M, N] (the virtual padding must never write there) shows up.
"""

import numpy as np
import pytest
import torch

import synth
import paged_variable_length_amd as pa
from oracle import gemm as og

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 4096
SENTINEL = 0x7FC1  # a bf16 NaN pattern no product produces


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _out_buffer(M, N):
    buf = torch.full((M * N + GUARD,), SENTINEL, dtype=torch.int16, device=DEV)
    c = buf[: M * N].view(torch.bfloat16).view(M, N)
    return buf, c


def _check(c, a, w, rows=None, what=""):
    """Compare C (device) with the oracle product; `rows` samples rows of C and A (indexed on
    the device before the copy)."""
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long)
        a = a.index_select(0, idx.to(a.device))
        c = c.index_select(0, idx.to(c.device))
    af = a.float().cpu().numpy().astype(np.float64)
    wf = w.float().cpu().numpy().astype(np.float64)
    ref = og.matmul(af, wf)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * (np.abs(af) @ np.abs(wf).T)
    got = c.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    worst = float((err / bound).max())
    assert worst <= 1.0, f"{what}: error {err.max():.3e} exceeds the bound (ratio {worst:.2f})"
    return worst


def _run(M, N, K, tile, k_split, seed, a_offset=0, w_offset=0, workers=256, tail=False):
    _announce(f"smooth_gemm M={M} N={N} K={K} tile={tile} k_split={k_split} "
              f"offsets={a_offset},{w_offset} workers={workers} tail={tail}")
    a0, w0 = synth.make_gemm_operands(M, N, K, device="cpu", seed=seed)
    # operands optionally start a few elements into a larger allocation (unaligned bases)
    abuf = torch.zeros(M * K + a_offset, dtype=torch.bfloat16, device=DEV)
    wbuf = torch.zeros(N * K + w_offset, dtype=torch.bfloat16, device=DEV)
    a = abuf[a_offset:].view(M, K)
    w = wbuf[w_offset:].view(N, K)
    a.copy_(a0.to(DEV))
    w.copy_(w0.to(DEV))
    plan = pa.GemmPlan(M, N, K, tile=tile, k_split=k_split, num_workers=workers, device=DEV,
                       tail_split=tail)
    buf, c = _out_buffer(M, N)
    plan.run(a, w, c)
    torch.cuda.synchronize()
    assert bool((buf[M * N:] == SENTINEL).all()), "store past the end of C"
    return c, a0, w0, plan


@pytest.mark.parametrize("tile", [256, 128])
@pytest.mark.parametrize("M,N,K,k_split", [
    (1, 1, 8, 0), (1, 300, 64, 0), (37, 19, 200, 0), (256, 256, 64, 0),
    (257, 513, 136, 0), (300, 200, 200, 128), (640, 384, 1000, 192), (513, 129, 4104, 1024),
    (100, 700, 72, 64), (512, 384, 1024, 0), (384, 256, 1088, 320)])
def test_gemm_ragged(M, N, K, k_split, tile):
    c, a, w, plan = _run(M, N, K, tile, k_split, seed=M + N + K)
    assert (len(plan.table.reduces) > 0) == (0 < k_split < K)
    _check(c, a, w, what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,tile,k_split", [(33, 70, 13, 256, 0), (300, 129, 77, 128, 0),
                                                (129, 257, 301, 256, 128), (5, 9, 1, 128, 0)])
def test_gemm_unaligned_k(M, N, K, tile, k_split):
    """K not a multiple of 8: rows are not 16-byte aligned, so stages load element by element."""
    c, a, w, _ = _run(M, N, K, tile, k_split, seed=7 * K)
    _check(c, a, w, what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,tile,workers", [(600, 512, 640, 256, 4), (1000, 64, 4097, 128, 40),
                                                (1024, 1024, 1024, 128, 256),
                                                (513, 700, 1000, 256, 3), (130, 260, 70, 128, 5)])
def test_gemm_tail_split(M, N, K, tile, workers):
    """Tables whose last partial round is cut into K pieces (reading of the page's balancing)."""
    c, a, w, plan = _run(M, N, K, tile, 0, seed=M + K, workers=workers, tail=True)
    _check(c, a, w, what=f"tail {M}x{N}x{K}")


def test_gemm_unaligned_bases():
    """Operands that start one element into their allocations take the element-wise path."""
    c, a, w, _ = _run(200, 300, 256, 256, 0, seed=3, a_offset=1, w_offset=3)
    _check(c, a, w, what="offset bases")


def test_gemm_split_matches_unsplit_closely():
    """The same product with and without K splits: both within the bound, and their
    difference is only summation order (a few bf16 ulps at most)."""
    M, N, K = 384, 512, 2048
    c0, a, w, _ = _run(M, N, K, 256, 0, seed=11)
    c1, _, _, _ = _run(M, N, K, 256, 512, seed=11)
    _check(c0, a, w, what="unsplit")
    _check(c1, a, w, what="split")
    d = (c0.float() - c1.float()).abs()
    assert float(d.max()) <= float(c0.float().abs().max()) * 2.0 ** -6


def test_gemm_closed_forms():
    """W = I (exact: each output is one bf16 input times 1) and a rank-one product
    A = u 1^T, W = v 1^T over K = 64, whose entries 64 u_i v_j are exact in fp32."""
    M, K = 300, 256
    a, _ = synth.make_gemm_operands(M, K, K, device="cpu", seed=5)
    eye = torch.eye(K, dtype=torch.bfloat16)
    plan = pa.GemmPlan(M, K, K, tile=256, device=DEV)
    buf, c = _out_buffer(M, K)
    plan.run(a.to(DEV), eye.to(DEV), c)
    torch.cuda.synchronize()
    assert torch.equal(c.cpu(), a), "A I^T must return A exactly"
    u = torch.tensor([1.0, -2.0, 0.5, 3.0, 0.25], dtype=torch.bfloat16)
    v = torch.tensor([2.0, -1.0, 4.0], dtype=torch.bfloat16)
    A = u[:, None].expand(5, 64).contiguous()
    W = v[:, None].expand(3, 64).contiguous()
    plan = pa.GemmPlan(5, 3, 64, tile=128, device=DEV)
    buf, c = _out_buffer(5, 3)
    plan.run(A.to(DEV), W.to(DEV), c)
    torch.cuda.synchronize()
    exp = (64.0 * u.double()[:, None] * v.double()[None, :]).to(torch.bfloat16)
    assert torch.equal(c.cpu(), exp)


@pytest.mark.parametrize("name", ["linear_mixed_oproj", "linear_prefill_qproj"])
def test_gemm_full_size_sampled(name):
    """The bench's Linear shapes at full size, in its launch configuration (tile 256, the last
    partial round cut into K pieces for 256 workers): sampled rows (first, last and random rows)
    checked against the oracle, every element finite."""
    M, N, K = synth.gemm_shape(name)
    _announce(f"smooth_gemm full {name} {M}x{N}x{K}")
    a, w = synth.make_gemm_operands(M, N, K, device=DEV, seed=1)
    plan = pa.GemmPlan(M, N, K, tile=256, k_split=0, num_workers=256, device=DEV,
                       tail_split=True)
    buf, c = _out_buffer(M, N)
    plan.run(a, w, c)
    torch.cuda.synchronize()
    assert bool((buf[M * N:] == SENTINEL).all()), "store past the end of C"
    assert bool(torch.isfinite(c).all())
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, M - 1, M // 2], rng.integers(0, M, size=45)]))
    _check(c, a, w, rows=rows, what=name)


def test_gemm_empty_and_errors():
    a = torch.zeros(4, 8, dtype=torch.bfloat16, device=DEV)
    w = torch.zeros(0, 8, dtype=torch.bfloat16, device=DEV)
    c = torch.zeros(4, 0, dtype=torch.bfloat16, device=DEV)
    plan = pa.GemmPlan(4, 0, 8, device=DEV)
    assert len(plan.table.tasks) == 0
    plan.run(a, w, c)                      # empty table: a no-op
    with pytest.raises(pa.PagedAttnError):
        pa.smooth_gemm(a, torch.zeros(3, 8, dtype=torch.bfloat16, device=DEV),
                       torch.zeros(4, 3, dtype=torch.bfloat16, device=DEV), 64,
                       plan.tasks, plan.reduces, 0, None)


def _random_gemm_case(seed):
    """Shape, tile, split, balancing and base offsets of random case `seed` (host draws only)."""
    rng = np.random.default_rng(12000 + seed)
    M, N = int(rng.integers(1, 1100)), int(rng.integers(1, 900))
    K = int(rng.choice([int(rng.integers(1, 2100)), 8 * int(rng.integers(1, 260))]))
    tile = int(rng.choice([128, 256]))
    k_split = int(rng.choice([0, 0, 64, 192, 512]))
    tail = bool(k_split == 0 and rng.integers(0, 2))
    workers = int(rng.choice([3, 40, 256]))
    off = int(rng.choice([0, 0, 0, 1]))
    return M, N, K, tile, k_split, tail, workers, off


@pytest.mark.parametrize("seed", range(32))
def test_gemm_random(seed):
    """Random shapes (ragged M and N, K aligned or not), tiles, K splits, tail splits and
    operand bases drawn jointly; every element against the oracle, nothing stored past C."""
    M, N, K, tile, k_split, tail, workers, off = _random_gemm_case(seed)
    c, a, w, _ = _run(M, N, K, tile, k_split, seed=seed, a_offset=off, w_offset=2 * off,
                      workers=workers, tail=tail)
    _check(c, a, w, what=f"random {seed}: {M}x{N}x{K}")
