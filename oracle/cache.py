"""Oracle for writing new K/V rows into the paged cache -- test infrastructure only.

cann-recipes-infer Paged KV / Packed Sequence page: section 3.2 grows a sequence by taking free
pages and writing the page table; section 5.2 copies the packed new keys into kv_pages. The ATB
page ("KV缓存复用") appends the K/V of a new turn's tokens to the blocks a session already owns.
This is that write, stated plainly: packed new token t of sequence s (row i = t - cu[s]) sits at
absolute position P_s + i, where P_s = context_lens[s] - q_len_s, and its K/V rows are copied
unchanged into slot (P_s + i) % block_size of physical block
block_table[s][(P_s + i) // block_size]. A pure copy, so it is bit-exact.
"""
from __future__ import annotations

import numpy as np

from .attention import pack_lengths


def reshape_and_cache(k_new, v_new, k_pages, v_pages, block_table, q_lens, context_lens):
    """Return copies of (k_pages, v_pages) with every new token's K/V written into its slot.

    k_new, v_new     [T, Hkv, D]
    k_pages, v_pages [NB, Hkv, bs, D]  (any dtype; copied, never modified in place)
    """
    k_out = np.array(k_pages, copy=True)
    v_out = np.array(v_pages, copy=True)
    bs = k_pages.shape[2]
    cu = pack_lengths(q_lens)
    for s in range(len(q_lens)):
        prefix = int(context_lens[s]) - int(q_lens[s])
        for i in range(int(q_lens[s])):
            t = int(cu[s]) + i
            pos = prefix + i
            b = int(block_table[s][pos // bs])
            k_out[b, :, pos % bs, :] = k_new[t]
            v_out[b, :, pos % bs, :] = v_new[t]
    return k_out, v_out
