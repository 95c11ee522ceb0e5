"""CPU oracle for paged, variable-length attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 NumPy statement of what the GPU path computes. Only the
test suite, the package's smoke check and the benchmark's CPU-baseline leg may import it; the
library itself never does, and it shares no code with the HIP kernels or their host code.

Contents:
  attention.pack_lengths        per-sequence lengths -> cumulative offsets
  attention.blocks_needed       blocks a context occupies
  attention.gather_kv           logical K/V of one sequence, read through its block table
  attention.paged_attention     full-row softmax attention per sequence, causal, GQA
  cache.reshape_and_cache       scatter of new K/V rows into their pages (bit-exact)
  task_table.build_task_table   the load-sorted task decomposition (bit-exact)

Every function is pinned in the CPU tests to something other than itself: the pages' worked
example, closed forms, invariants and a library routine on tiny inputs. No function is
"parity unpinned".
"""
from . import attention, cache, task_table  # noqa: F401
