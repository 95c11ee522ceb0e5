"""GPU test of paged_attn_varlen_prefill_noalloc (partial rows in the library's own device
scratch) against paged_attn_varlen_prefill (partial rows in a caller workspace): both run the
same kernels over the same table, so their outputs must agree bit for bit, and both must meet
the oracle's bars. Two calls in a row, the second on a smaller batch, so the second reuses the
scratch the first left behind."""
import math

import numpy as np
import pytest
import torch

import synth
import paged_variable_length_amd as pa
from tests.helpers import check_close, to_np
from tests.test_gpu_parity import _announce, host_subset, oracle_subset

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(q, ctx, seed, **tiling):
    w = synth.custom_workload(q, ctx, 16, 4, 128, 16, seed=seed, spare_blocks=3)
    _announce(f"no-alloc entry N={w.num_seqs} T={w.num_tokens} {tiling}")
    vals = {k: v.to(DEV) for k, v in synth.make_values(w, device="cpu").items()}
    h = host_subset(w, vals, list(range(w.num_seqs)))
    plan = pa.StepPlan(w.q_lens, w.ctx_lens, w.block_table, 16, 4, 128, 16, device=DEV, **tiling)
    assert plan.num_partials > 0 and len(plan.table.combines) > 0
    plan.write_cache(vals["k_new"], vals["v_new"], vals["k_pages"], vals["v_pages"])
    scale = 1.0 / math.sqrt(128)
    ref_out = torch.full_like(vals["q"], float("nan"))
    plan.varlen(vals["q"], vals["k_pages"], vals["v_pages"], scale, ref_out)
    out = torch.full_like(vals["q"], float("nan"))
    pa.paged_attn_varlen_prefill_noalloc(vals["q"], vals["k_pages"], vals["v_pages"],
                                         plan.block_table, plan.cu, plan.ctx, scale, plan.tasks,
                                         plan.table.kinds, plan.combines, plan.num_partials, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    ref = oracle_subset(h, scale)
    check_close(to_np(out)[h["rows"]], ref, "bf16", "no-alloc entry")
    return plan.num_partials


def test_noalloc_entry_matches_workspace_entry_twice():
    # decode rows with key splits, a verify draft, and prefill chunks with key splits
    first = _case([1, 3, 200, 1, 130, 1], [900, 3 + 500, 200 + 700, 2000, 130 + 64, 300], 21,
                  dec_split=128, pf_q_tile=64, pf_kv_split=128, verify_rows=4)
    # the second call: a smaller batch over the scratch the first call left behind
    second = _case([1, 40, 1], [700, 40 + 300, 129], 22, dec_split=64, pf_q_tile=128,
                   pf_kv_split=64)
    assert second < first
