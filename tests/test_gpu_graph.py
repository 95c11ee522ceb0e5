"""GPU test of the benchmark's captured step: the per-slot HIP graphs (cache write, attention
launch, combine) replayed after each step's host table build and copy give outputs bit-identical
to eager launches of the same step, replay after replay, with eager work and synchronisations
between the replays. The library records no memset into the graphs (its launches are kernels
only), and the replays are checked one by one."""
import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["decode_mha_bf16", "verify_gqa_fp8", "prefill_varlen_bf16",
                                  "decode_shared_mha_bf16", "mixed_fp8"])
def test_graph_replays_match_eager_step(name):
    print(f"\n[case] graph replay {name}", flush=True)
    r = bench.Runner(name)
    sizes = r.build_table(0)
    r.launch(0, *sizes)
    torch.cuda.synchronize()
    ref = r.out.clone()
    assert torch.isfinite(ref).all()
    r.capture()
    for i in range(6):
        r.out.fill_(float("nan"))               # eager work on the launch stream between replays
        torch.cuda.synchronize()
        r.step()                                # host table, its copy, the slot's graph replay
        torch.cuda.synchronize()
        assert torch.equal(r.out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"
    # eager launches still give the same result after the replays
    r.out.zero_()
    sizes = r.build_table(1)
    r.launch(1, *sizes)
    torch.cuda.synchronize()
    assert torch.equal(r.out.view(torch.int16), ref.view(torch.int16))
