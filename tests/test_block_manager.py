"""Host-side KV block manager (pk_bm_* through the Python binding), on the CPU.

The manager has no arithmetic to compare with an oracle; its contract is
checked directly:
  * cache semantics: a simulated cache records, for every slot written, the
    token prefix whose K/V it holds (in a model the K/V of position p depend on
    tokens[0..p]); reading any live sequence through its block table must give
    exactly that sequence's prefixes, whatever was shared, freed or evicted;
  * bookkeeping: reference counts equal the number of live tables holding a
    block; free blocks are those with none; only full blocks are shared;
  * prefix reuse: a prompt that starts with the full blocks of a live sequence
    reuses them (the same block ids), up to its last token;
  * eviction order: least recently freed first, a sequence's tail first;
  * blocks filled in a step are found only after that step's commit, so no
    batch reuses a prefix block that the same batch writes;
  * errors leave the manager unchanged.
"""
import random

import pytest

import paged_kv_cache_236_amd as pk


def table_of(m, sid, mb=64):
    tables, _, _, _ = m.prepare([sid], [0], mb)
    return [int(b) for b in tables[0] if b >= 0]


def write_new_tokens(m, cache, seqs, ids, num_new, mb=64):
    """Store the K/V (here: the prefix tuple) of the new tokens at slot_mapping."""
    _, cu_q, cu_k, slots = m.prepare(ids, num_new, mb)
    k = 0
    for i, sid in enumerate(ids):
        toks = seqs[sid]
        L = len(toks)
        assert int(cu_k[i + 1] - cu_k[i]) == L
        assert int(cu_q[i + 1] - cu_q[i]) == num_new[i]
        for pos in range(L - num_new[i], L):
            cache[int(slots[k])] = tuple(toks[:pos + 1])
            k += 1
    assert k == len(slots)


def check_state(m, cache, seqs, mb=64):
    bs = m.block_size
    refs = {}
    owner_of_partial = {}
    for sid, toks in seqs.items():
        L, nb, _ = m.seq_info(sid)
        assert L == len(toks)
        tbl = table_of(m, sid, mb)
        assert len(tbl) == nb == (L + bs - 1) // bs
        for pos in range(L):
            slot = tbl[pos // bs] * bs + pos % bs
            assert cache.get(slot) == tuple(toks[:pos + 1]), (sid, pos)
        for b in tbl:
            refs[b] = refs.get(b, 0) + 1
        if L % bs:
            owner_of_partial.setdefault(tbl[-1], []).append(sid)
    for b, owners in owner_of_partial.items():
        assert refs[b] == 1, f"partial block {b} is shared by {owners}"
    nfree = 0
    for b in range(m.num_blocks):
        ref, _ = m.block_info(b)
        assert ref == refs.get(b, 0)
        nfree += ref == 0
    assert m.num_free_blocks == nfree


def test_fresh_allocation_and_free():
    with pk.BlockManager(16, 4) as m:
        assert m.num_free_blocks == 16
        assert m.allocate(7, list(range(10))) == 0
        assert m.seq_info(7) == (10, 3, 0)
        tbl = table_of(m, 7)
        assert len(set(tbl)) == 3
        assert m.num_free_blocks == 13
        # full blocks are pending (not findable) until the step is committed
        assert [m.block_info(b) for b in tbl] == [(1, False)] * 3
        assert m.commit() == 2
        assert [m.block_info(b) for b in tbl] == [(1, True), (1, True), (1, False)]
        assert m.commit() == 0
        m.free(7)
        assert m.num_free_blocks == 16
        # freed full blocks stay registered until their space is reused
        assert [m.block_info(b)[1] for b in tbl] == [True, True, False]


def test_prefix_reuse_shares_block_ids():
    with pk.BlockManager(32, 4) as m:
        sys_prompt = [5, 6, 7, 8, 9, 10, 11, 12]          # two full blocks
        assert m.allocate(1, sys_prompt + [1, 2, 3]) == 0
        m.commit()
        assert m.allocate(2, sys_prompt + [4, 4, 4, 4, 4]) == 8
        t1, t2 = table_of(m, 1), table_of(m, 2)
        assert t1[:2] == t2[:2] and t1[2] != t2[2]
        assert m.block_info(t1[0]) == (2, True)
        # a prompt diverging inside the second block reuses only the first
        assert m.allocate(3, sys_prompt[:6] + [0, 0, 0]) == 4
        assert table_of(m, 3)[0] == t1[0] and table_of(m, 3)[1] != t1[1]


def test_equal_block_after_different_prefix_is_not_shared():
    with pk.BlockManager(32, 4) as m:
        m.allocate(1, [1, 1, 1, 1, 2, 2, 2, 2, 9])
        m.commit()
        # same second block, different first block: the chain hash differs
        assert m.allocate(2, [3, 3, 3, 3, 2, 2, 2, 2, 9]) == 0
        assert set(table_of(m, 1)).isdisjoint(table_of(m, 2))


def test_prompt_cached_in_full_recomputes_last_block():
    with pk.BlockManager(32, 4) as m:
        m.allocate(1, list(range(8)))
        m.commit()
        # 8 tokens, both blocks cached: the last block is recomputed
        assert m.allocate(2, list(range(8))) == 4
        m.commit()
        t1, t2 = table_of(m, 1), table_of(m, 2)
        assert t1[0] == t2[0] and t1[1] != t2[1]
        # 9 tokens: both full blocks reused, the ninth token computed
        assert m.allocate(3, list(range(9))) == 8
        assert table_of(m, 3)[:2] == t1
        # a single-block prompt cached in full still computes its block
        m.allocate(4, [1, 2, 3, 4])
        m.commit()
        assert m.allocate(5, [1, 2, 3, 4]) == 0


def test_freed_blocks_are_reused_from_cache_and_evicted_lru():
    with pk.BlockManager(6, 4) as m:
        m.allocate(1, list(range(12)))                      # blocks a b c
        m.commit()
        a, b, c = table_of(m, 1)
        m.free(1)                                           # freed c, b, a (tail first)
        assert m.num_free_blocks == 6
        # a cache hit revives the freed prefix
        assert m.allocate(2, list(range(8)) + [99]) == 8
        assert table_of(m, 2)[:2] == [a, b]
        assert m.num_free_blocks == 3
        m.free(2)
        # the untouched blocks go first, then c (freed first), ...
        m.allocate(3, [50] * 4)
        m.allocate(4, [51] * 4)
        m.allocate(5, [52] * 4)
        m.allocate(6, [53] * 4)
        used = [table_of(m, s)[0] for s in (3, 4, 5, 6)]
        assert c in used
        assert a not in used                                # freed last: still cached
        assert m.allocate(7, list(range(4)) + [0]) == 4
        assert table_of(m, 7)[0] == a


def test_append_crosses_blocks_and_registers_them():
    with pk.BlockManager(16, 4) as m:
        m.allocate(1, [1, 2, 3])
        assert m.seq_info(1) == (3, 1, 0)
        m.append(1, 4)                                      # fills block 0
        assert m.seq_info(1) == (4, 1, 0)
        m.append(1, 5)                                      # opens block 1
        assert m.seq_info(1) == (5, 2, 0)
        for t in (6, 7, 8):
            m.append(1, t)
        # the appended blocks are pending until the step is committed
        assert m.allocate(3, [1, 2, 3, 4, 5, 6, 7, 8, 0]) == 0
        assert m.commit() == 4                              # seq 1's two, seq 3's two
        assert m.allocate(2, [1, 2, 3, 4, 5, 6, 7, 8, 0]) == 8
        assert table_of(m, 2)[:2] == table_of(m, 1)


def test_prepare_outputs():
    with pk.BlockManager(16, 4) as m:
        m.allocate(1, list(range(6)))
        m.allocate(2, list(range(4)) + [9])
        tables, cu_q, cu_k, slots = m.prepare([2, 1], [1, 6], 3)
        t1, t2 = table_of(m, 1), table_of(m, 2)
        assert tables.tolist() == [t2 + [-1], t1 + [-1]]
        assert cu_q.tolist() == [0, 1, 7] and cu_k.tolist() == [0, 5, 11]
        want = [t2[1] * 4 + 0] + [t1[p // 4] * 4 + p % 4 for p in range(6)]
        assert slots.tolist() == want
        tables, cu_q, cu_k, slots = m.prepare([], [], 3)
        assert tables.shape == (0, 3) and cu_q.tolist() == [0] and slots.numel() == 0


def test_errors_leave_manager_unchanged():
    with pk.BlockManager(4, 4) as m:
        m.allocate(1, list(range(9)))                       # 3 blocks
        before = (m.num_free_blocks, table_of(m, 1), m.seq_info(1))
        with pytest.raises(pk.PagedKVError, match="WORKSPACE"):
            m.allocate(2, list(range(100, 109)))            # needs 3, 1 free
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.allocate(1, [1])                              # id in use
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.allocate(3, [])
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.free(42)
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.prepare([1], [10], 4)                         # more new tokens than tokens
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.prepare([1], [1], 2)                          # table longer than capacity
        with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
            m.block_info(4)
        assert (m.num_free_blocks, table_of(m, 1), m.seq_info(1)) == before
        for t in (9, 10, 11):                               # fills the third block
            m.append(1, t)
        m.allocate(5, [7])                                  # takes the last free block
        with pytest.raises(pk.PagedKVError, match="WORKSPACE"):
            m.append(1, 12)                                 # would open a fifth block
        assert m.seq_info(1) == (12, 3, 0)
    with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
        pk.BlockManager(0, 16)
    with pytest.raises(pk.PagedKVError, match="INVALID_ARG"):
        pk.BlockManager(1 << 20, 4096)                      # slots overflow int32


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("bs", [1, 4, 16])
def test_random_workload_keeps_cache_semantics(seed, bs):
    """Random admissions (prompts sharing a few system prompts), decode steps
    and frees under memory pressure; after every step each live sequence reads
    exactly its own prefixes through its table."""
    rnd = random.Random(seed * 100 + bs)
    nblocks = 48 if bs == 16 else 160
    m = pk.BlockManager(nblocks, bs)
    systems = [[rnd.randrange(5) for _ in range(rnd.randrange(1, 3 * bs + 2))] for _ in range(3)]
    cache, seqs = {}, {}
    next_id = 0
    hits = 0
    for step in range(120):
        op = rnd.random()
        if op < 0.35 or not seqs:
            batch = []
            for _ in range(rnd.randrange(1, 4)):
                prompt = list(rnd.choice(systems)) if rnd.random() < 0.8 else []
                prompt += [rnd.randrange(5) for _ in range(rnd.randrange(1, 2 * bs + 2))]
                free_before = m.num_free_blocks
                try:
                    cached = m.allocate(next_id, prompt)
                except pk.PagedKVError as e:
                    assert "WORKSPACE" in str(e)
                    assert m.num_free_blocks == free_before
                    continue
                assert cached % bs == 0 and 0 <= cached < len(prompt)
                hits += cached > 0
                seqs[next_id] = prompt
                batch.append((next_id, len(prompt) - cached))
                next_id += 1
            if batch:
                write_new_tokens(m, cache, seqs, [s for s, _ in batch], [n for _, n in batch])
            m.commit()
        elif op < 0.8:
            ids = []
            for sid in list(seqs):
                tok = rnd.randrange(5)
                try:
                    m.append(sid, tok)
                except pk.PagedKVError as e:
                    assert "WORKSPACE" in str(e)
                    continue
                seqs[sid].append(tok)
                ids.append(sid)
            write_new_tokens(m, cache, seqs, ids, [1] * len(ids))
            m.commit()
        else:
            sid = rnd.choice(list(seqs))
            m.free(sid)
            del seqs[sid]
        check_state(m, cache, seqs)
    assert hits > 0
    for sid in list(seqs):
        m.free(sid)
    assert m.num_free_blocks == nblocks
    m.close()


def test_reuse_is_maximal_against_live_sequences():
    """A new prompt reuses every leading full block that a live sequence
    (whose blocks cannot have been evicted) has with the same prefix."""
    rnd = random.Random(7)
    bs = 4
    with pk.BlockManager(400, bs) as m:
        live = {}
        for sid in range(60):
            base = rnd.choice(list(live.values())) if live and rnd.random() < 0.7 else []
            cut = rnd.randrange(0, len(base) + 1)
            prompt = base[:cut] + [rnd.randrange(3) for _ in range(rnd.randrange(1, 10))]
            best = 0
            for toks in live.values():
                n = 0
                while n < min(len(toks), len(prompt)) and toks[n] == prompt[n]:
                    n += 1
                best = max(best, n // bs * bs)
            best = min(best, (len(prompt) - 1) // bs * bs)
            assert m.allocate(sid, prompt) >= best
            m.commit()
            live[sid] = prompt
            if rnd.random() < 0.3:
                victim = rnd.choice(list(live))
                m.free(victim)
                del live[victim]


def test_same_step_blocks_are_not_found_before_commit():
    """A prompt's full blocks are written by the step that admits it; a second
    prompt of the same step must not take them as its cached prefix (a fused
    store + prefill would read them before they are written)."""
    with pk.BlockManager(32, 4) as m:
        sys_prompt = [5, 6, 7, 8, 9, 10, 11, 12]
        assert m.allocate(1, sys_prompt + [1]) == 0
        assert m.allocate(2, sys_prompt + [2]) == 0         # same step: no hit
        t1, t2 = table_of(m, 1), table_of(m, 2)
        assert set(t1).isdisjoint(t2)
        # every block a batch reads as a prefix was filled before the batch
        _, cu_q, cu_k, slots = m.prepare([1, 2], [9, 9], 8)
        assert cu_q.tolist() == [0, 9, 18]
        assert m.commit() == 4
        # the next step finds them (the first copy registered under the hash)
        assert m.allocate(3, sys_prompt + [3]) == 8
        assert table_of(m, 3)[:2] in (t1[:2], t2[:2])
        written = {int(s) // 4 for s in slots}
        _, cu_q, _, slots3 = m.prepare([3], [1], 8)
        assert set(table_of(m, 3)[:2]) <= written           # filled by the committed step
        assert {int(s) // 4 for s in slots3}.isdisjoint(table_of(m, 3)[:2])


def test_pending_block_freed_before_commit_is_dropped():
    with pk.BlockManager(8, 4) as m:
        m.allocate(1, list(range(9)))                       # two full blocks pending
        tbl = table_of(m, 1)
        m.free(1)
        assert m.commit() == 0                              # nothing registered
        assert [m.block_info(b) for b in tbl] == [(0, False)] * 3
        assert m.allocate(2, list(range(9))) == 0           # no stale hit
        assert m.commit() == 2
    # a block freed and refilled before the commit is registered once, under
    # its new content
    with pk.BlockManager(2, 4) as m:
        m.allocate(9, [1])                                  # holds the other block
        m.allocate(3, [7, 7, 7, 7])
        (b,) = table_of(m, 3)
        m.free(3)
        m.allocate(4, [8, 8, 8, 8])
        assert table_of(m, 4) == [b]
        assert m.commit() == 1
        m.free(9)
        assert m.allocate(5, [8, 8, 8, 8, 2]) == 4
        assert table_of(m, 5)[0] == b
        m.free(5)
        m.free(4)
        assert m.allocate(6, [7, 7, 7, 7, 2]) == 0
