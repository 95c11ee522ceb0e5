"""Small test helpers: tensor <-> numpy conversion and tolerance checks (no method arithmetic)."""
from __future__ import annotations

import numpy as np

# Attention outputs in bf16 (bf16 inputs, fp32 accumulation) versus the fp64 oracle.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
# fp32 inputs (a reading; only the bf16 bounds are stated): fp32 accumulation over <= 64 keys and
# 128-term dots plus a ~1 ulp exp2 gives O(1e-6) errors on O(1) outputs, so 1e-4 / 1e-5 leaves
# two orders of margin while a dropped key (weight >= 1/ctx) still fails.
FP32_MAX_ABS = 1e-4
FP32_MEAN_ABS = 1e-5


def to_np(t):
    """torch tensor (any float dtype, any device) -> fp64 numpy (exact for bf16/fp32)."""
    import torch
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def to_np_raw(t):
    """torch tensor -> numpy holding the same bits (bf16 as uint16) for bit-exact comparisons."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def tolerance(dtype: str):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == "bf16" else (FP32_MAX_ABS, FP32_MEAN_ABS)


def check_close(got, ref, dtype, what=""):
    """Assert max-abs and mean-abs error bounds over the finite reference entries."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    sel = ~np.isnan(ref)
    assert sel.any(), f"{what}: nothing to compare"
    assert np.all(np.isfinite(got[sel])), f"{what}: non-finite output"
    err = np.abs(got[sel] - ref[sel])
    mx, mean = tolerance(dtype)
    assert err.max() <= mx, f"{what}: max-abs {err.max():.3e} > {mx}"
    assert err.mean() <= mean, f"{what}: mean-abs {err.mean():.3e} > {mean}"
    return float(err.max()), float(err.mean())


def aliased_batch(rng, bs, n_groups):
    """Decode sequences in runs that share a random number of leading blocks, a prefill and a
    verify sequence in between, and private blocks for everything else."""
    rows, ctx, q = [], [], []
    nxt = 1000
    for g in range(n_groups):
        shared = [nxt + i for i in range(int(rng.integers(0, 17)))]
        nxt += len(shared)
        for m in range(int(rng.integers(1, 6))):
            c = len(shared) * bs + int(rng.integers(1, 200))
            need = -(-c // bs)
            row = shared + list(range(nxt, nxt + need - len(shared)))
            nxt += need - len(shared)
            rows.append(row)
            ctx.append(c)
            q.append(1)
        if g % 2:
            c = int(rng.integers(5, 90))
            rows.append(list(range(nxt, nxt + -(-c // bs))))
            nxt += -(-c // bs)
            ctx.append(c)
            q.append(int(rng.integers(2, 5)))
    width = max(len(r) for r in rows)
    bt = np.full((len(rows), width), -1, dtype=np.int64)
    for i, r in enumerate(rows):
        bt[i, :len(r)] = r
    return q, ctx, bt


def aliased_workload(rng, bs, n_groups, num_q_heads, num_kv_heads, head_dim, dtype="bf16",
                     seed=0, spare_blocks=2):
    """aliased_batch as a synth.Workload: the block ids mapped onto a dense, shuffled pool."""
    import synth
    q, ctx, bt = aliased_batch(rng, bs, n_groups)
    ids = np.unique(bt[bt >= 0])
    nb = len(ids) + spare_blocks
    new = rng.permutation(nb)[:len(ids)]
    table = np.full(bt.shape, -1, dtype=np.int32)
    table[bt >= 0] = new[np.searchsorted(ids, bt[bt >= 0])]
    return synth.Workload("aliased", seed, np.asarray(q, np.int64), np.asarray(ctx, np.int64),
                          num_q_heads, num_kv_heads, head_dim, bs, dtype, table, nb)
