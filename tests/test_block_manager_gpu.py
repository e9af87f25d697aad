"""The block manager driving the HIP path: block tables and slot mappings from
pk_bm_prepare feed kv_store, paged_prefill and paged_decode on the GPU, with
prompts that share a system prompt (prefix-cache hits, a freed sequence's
blocks revived and evicted).  The oracle computes every sequence on its own
dense layout (blocks laid out in order), so the manager's tables are checked
by the results and not reused by the reference.

The K/V and query rows of position p are drawn from a generator seeded by the
token prefix tokens[0..p], as in a model, so a shared block is only right if
the prefix it was computed for is the same."""
import hashlib
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import bits_of, normal_bf16

pytestmark = pytest.mark.gpu

HQ, HKV, D = 16, 8, 128
SCALE = 1 / math.sqrt(D)
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def rows_for(prefix, what):
    """[HKV or HQ, D] bf16 bits for the last token of ``prefix``."""
    digest = hashlib.blake2b(np.asarray(prefix, np.int32).tobytes() + what.encode(),
                             digest_size=8).digest()
    rng = np.random.default_rng(int.from_bytes(digest, "little"))
    return normal_bf16(rng, (HQ if what == "q" else HKV, D))


def bf(a, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def dense_reference(seqs, ids, num_new, bs):
    """Oracle attention of the new tokens of each sequence, on a private dense
    layout: sequence i owns blocks i*mb .. i*mb+mb-1 in order."""
    mb = max(math.ceil(len(seqs[s]) / bs) for s in ids)
    kc = np.zeros((len(ids) * mb, bs, HKV, D), np.uint16)
    vc = np.zeros_like(kc)
    q_rows, cu_q, cu_k = [], [0], [0]
    for i, s in enumerate(ids):
        toks = seqs[s]
        for p in range(len(toks)):
            kc[i * mb + p // bs, p % bs] = rows_for(toks[:p + 1], "k")
            vc[i * mb + p // bs, p % bs] = rows_for(toks[:p + 1], "v")
        for p in range(len(toks) - num_new[i], len(toks)):
            q_rows.append(rows_for(toks[:p + 1], "q"))
        cu_q.append(cu_q[-1] + num_new[i])
        cu_k.append(cu_k[-1] + len(toks))
    tables = np.arange(len(ids) * mb, dtype=np.int32).reshape(len(ids), mb)
    q = np.stack(q_rows)
    return q, oracle.paged_prefill(q, kc, vc, tables, np.array(cu_q), np.array(cu_k), SCALE)


def assert_close(got, ref):
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (float(err.max()), float(err.mean()))


@pytest.mark.parametrize("fused", [False, True], ids=["store_then_attend", "fused_store"])
@pytest.mark.parametrize("bs", [16, 64])
def test_block_manager_end_to_end(gpu_lib, bs, fused):
    """Admissions sharing a system prompt, a free, cross-block decode steps.
    Unfused: kv_store then paged_prefill / paged_decode.  Fused:
    paged_prefill_store / paged_decode_store, which read prefix blocks in the
    same launch that writes the new rows; the manager's commit rule (blocks
    filled in a step are found only after it) keeps every prefix block they
    read written by an earlier launch."""
    pk = gpu_lib
    rng = np.random.default_rng(2024 + bs)
    vocab = 50
    # Exactly enough blocks (one spare at block 16) for the end state, so the
    # freed sequence's blocks are evicted by the last decode steps.
    num_blocks = 10 if bs == 16 else 9
    mb = 16
    k_cache = torch.zeros(num_blocks, bs, HKV, D, dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    m = pk.BlockManager(num_blocks, bs)
    system = list(rng.integers(0, vocab, 2 * bs + bs // 2))
    seqs = {}

    def step(ids, num_new, decode):
        tables, cu_q, cu_k, slots = m.prepare(ids, num_new, mb)
        key, val, q = [], [], []
        for i, s in enumerate(ids):
            toks = seqs[s]
            for p in range(len(toks) - num_new[i], len(toks)):
                key.append(rows_for(toks[:p + 1], "k"))
                val.append(rows_for(toks[:p + 1], "v"))
                q.append(rows_for(toks[:p + 1], "q"))
        q_ref, ref = dense_reference(seqs, ids, num_new, bs)
        assert np.array_equal(np.stack(q), q_ref)
        kt, vt, qt = bf(np.stack(key)), bf(np.stack(val)), bf(np.stack(q))
        if not fused:
            pk.kv_store(kt, vt, slots.cuda(), k_cache, v_cache)
        if decode:
            ctx = (cu_k[1:] - cu_k[:-1]).cuda()
            if fused:
                out = pk.paged_decode_store(qt, kt, vt, k_cache, v_cache, tables.cuda(), ctx, SCALE)
            else:
                out = pk.paged_decode(qt, k_cache, v_cache, tables.cuda(), ctx, SCALE)
        else:
            args = (tables.cuda(), cu_q.cuda(), cu_k.cuda(), SCALE)
            if fused:
                out = pk.paged_prefill_store(qt, kt, vt, k_cache, v_cache, *args,
                                             max_seqlen_q=int(max(num_new)))
            else:
                out = pk.paged_prefill(qt, k_cache, v_cache, *args, max_seqlen_q=int(max(num_new)))
        m.commit()   # the step is enqueued: its full blocks may now be reused
        torch.cuda.synchronize()
        assert_close(out, ref)

    # One prefill batch: A and B share the system prompt but are admitted in
    # the same step, so B computes it too (A's blocks are not committed yet).
    seqs[0] = system + list(rng.integers(0, vocab, bs + 3))
    seqs[1] = system + list(rng.integers(0, vocab, 5))
    new = [len(seqs[0]) - m.allocate(0, seqs[0]), len(seqs[1]) - m.allocate(1, seqs[1])]
    assert new[0] == len(seqs[0]) and new[1] == len(seqs[1])
    step([0, 1], new, decode=False)
    # A finishes; C reuses the committed system prompt, D (no shared prefix) takes space.
    m.free(0)
    seqs[2] = system + list(rng.integers(0, vocab, 7))
    seqs[3] = list(rng.integers(0, vocab, bs + 1))
    new = [len(seqs[2]) - m.allocate(2, seqs[2]), len(seqs[3]) - m.allocate(3, seqs[3])]
    assert new[0] == len(seqs[2]) - 2 * bs and new[1] == len(seqs[3])
    step([2, 3], new, decode=False)
    # Decode steps across block boundaries.
    for _ in range(bs + 2):
        for s in (1, 2, 3):
            tok = int(rng.integers(0, vocab))
            m.append(s, tok)
            seqs[s].append(tok)
        step([1, 2, 3], [1, 1, 1], decode=True)
    # Every live sequence reads its own K/V rows through its table, bit for bit.
    kc, vc = bits_of(k_cache), bits_of(v_cache)
    tables, _, _, _ = m.prepare([1, 2, 3], [0, 0, 0], mb)
    for i, s in enumerate((1, 2, 3)):
        for p, _ in enumerate(seqs[s]):
            blk = int(tables[i, p // bs])
            assert np.array_equal(kc[blk, p % bs], rows_for(seqs[s][:p + 1], "k"))
            assert np.array_equal(vc[blk, p % bs], rows_for(seqs[s][:p + 1], "v"))
    m.close()
