"""The seeded input generators (shared by both sides; they hold none of the
method's arithmetic): shapes, budgets and slot positions of the named
workloads."""
import numpy as np

import workloads as W


def test_mixed_batch_structure():
    x = W.mixed_batch()
    lq = np.diff(x.cu_seqlens_q)
    lk = np.diff(x.cu_seqlens_k)
    assert int(x.cu_seqlens_q[-1]) <= W.MIXED_BATCH_TOKENS
    assert (lq[:48] == 1).all() and (lq[48:] > 1).all()          # decode first, then chunks
    assert (lk == x.context_lens).all() and (lk >= lq).all()
    pref = lk[48:] - lq[48:]
    assert (pref % x.block_size == 0).all() and (pref <= 4 * x.block_size).all()
    # each new token is stored at its own position (slot of position P + i)
    bs = x.block_size
    k = 0
    for b in range(len(lq)):
        for pos in range(int(lk[b]) - int(lq[b]), int(lk[b])):
            blk = x.block_tables[b, pos // bs]
            assert x.slot_mapping[k] == blk * bs + pos % bs
            k += 1
    assert k == len(x.slot_mapping) == x.q.shape[0]
    # the table rows are disjoint (one permutation of the blocks)
    used = [x.block_tables[b, : -(-int(lk[b]) // bs)] for b in range(len(lq))]
    flat = np.concatenate(used)
    assert len(np.unique(flat)) == len(flat)
