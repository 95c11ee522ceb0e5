"""GPU parity for shared-prefix attention: decode sequences whose block tables alias their
leading blocks run PA_TASK_SHARED tasks (the prefix read once for several sequences) plus their
own decode splits, merged by the combine; outputs against the fp64 oracle, which reads every
sequence's keys through its own table row. Run on an MI355X with the library built in-tree."""
import numpy as np
import pytest

import synth
from bench import TILING as BENCH_TILING
from paged_variable_length_amd import _abi
from tests.helpers import aliased_workload
from tests.test_gpu_parity import _announce, small_case

pytestmark = pytest.mark.gpu


def _has_shared(plan):
    return bool(np.any(plan.table.tasks[:, 0] == _abi.PA_TASK_SHARED))


def _decode_groups(rng, n_groups, bs, hq, hkv, d, dtype="bf16", max_members=20):
    prefix = rng.integers(1, 40, size=n_groups) * bs
    own = [rng.integers(1, 300, size=int(rng.integers(1, max_members + 1)))
           for _ in range(n_groups)]
    return synth.shared_prefix_workload(prefix, own, hq, hkv, d, bs, dtype=dtype,
                                        seed=int(rng.integers(1 << 30)), spare_blocks=3)


@pytest.mark.parametrize("hq,hkv,d,bs,dec_split", [(8, 8, 128, 16, 64), (8, 4, 128, 16, 128),
                                                   (16, 4, 64, 32, 64), (16, 2, 128, 64, 192),
                                                   (32, 4, 128, 16, 64)])
def test_shared_decode_small(hq, hkv, d, bs, dec_split):
    rng = np.random.default_rng(hq * 100 + hkv * 10 + bs)
    w = _decode_groups(rng, 5, bs, hq, hkv, d)
    _announce(f"shared decode groups={w.extra['prefix_lens']}")
    (mx, _), out, _, plan = small_case(w, "decode", dec_split=dec_split, shared_min=64)
    assert _has_shared(plan)


def test_shared_decode_fp32():
    rng = np.random.default_rng(5)
    w = _decode_groups(rng, 3, 16, 4, 2, 64, dtype="fp32", max_members=9)
    _, _, _, plan = small_case(w, "decode", dec_split=64, shared_min=64)
    assert _has_shared(plan)


@pytest.mark.parametrize("seed,G", [(1, 1), (2, 2), (3, 4), (4, 8)])
def test_shared_in_mixed_launch(seed, G):
    """Groups between prefill and verify sequences, through the unified launch."""
    rng = np.random.default_rng(40 + seed)
    w = aliased_workload(rng, 16, 8, 2 * G, 2, 128, seed=seed)
    (mx, _), out, _, plan = small_case(w, "varlen", dec_split=64, pf_q_tile=64, verify_rows=4,
                                       shared_min=64)
    assert _has_shared(plan)


def test_shared_decode_full_size_sampled():
    """The 128-request agent batch (8 prompts x 16 requests) in the launch configuration
    bench.py times (its TILING: key splits of 4096, groups from 64 shared keys); a seeded sample
    of requests from every group against the oracle."""
    w = synth.make_workload("decode_shared_mha_bf16")
    rng = np.random.default_rng(9)
    seqs = sorted(set((16 * np.arange(8) + rng.integers(0, 16, size=8)).tolist() + [0, 127]))
    _announce(f"shared decode full N={w.num_seqs} sampled {seqs}")
    _, out, _, plan = small_case(w, "decode", seqs=seqs, **BENCH_TILING["decode_shared_mha_bf16"])
    assert _has_shared(plan)
    import torch
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("shared_min", [0, 64])
def test_decode_entry_and_unified_launch_agree_bitwise(shared_min):
    """The decode entry (one chunk of page reads in flight per wave on tables with shared-prefix
    tasks, two otherwise) and the unified launch (always two) run the same arithmetic in the same
    order in every wave, so on one decode table, with or without shared-prefix groups, their
    outputs agree bit for bit."""
    import math
    import torch
    import paged_variable_length_amd as pa
    rng = np.random.default_rng(77 + shared_min)
    w = _decode_groups(rng, 4, 16, 16, 4, 128)
    _announce(f"decode entry vs unified launch, shared_min={shared_min} N={w.num_seqs}")
    vals = {k: v.to("cuda") for k, v in synth.make_values(w, device="cpu").items()}
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, w.num_q_heads, w.num_kv_heads,
                       w.head_dim, w.block_size, device="cuda", dec_split=128,
                       shared_min=shared_min)
    assert _has_shared(plan) == bool(shared_min)
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    scale = 1.0 / math.sqrt(w.head_dim)
    out_d = torch.full_like(vals["q"], float("nan"))
    out_v = torch.full_like(vals["q"], float("nan"))
    plan.decode(vals["q"], vals["k_pages"], vals["v_pages"], scale, out_d)
    plan.varlen(vals["q"], vals["k_pages"], vals["v_pages"], scale, out_v)
    torch.cuda.synchronize()
    assert torch.isfinite(out_d).all()
    assert torch.equal(out_d.view(torch.int16), out_v.view(torch.int16))
