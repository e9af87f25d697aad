"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

kv_store must be bit-exact.  Attention output (bf16) must be within max-abs
2e-2 and mean-abs 2e-3 of the oracle's float64 result: the output's own bf16
rounding is up to 2^-8 relative (|out| <~ 3 gives <= 7.8e-3), fp32
accumulation over <= 8192 keys adds ~1e-5, so 2e-2 max-abs leaves room only
for rounding, not for a dropped term or a wrong index.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from workloads import bits_of, to_torch

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def assert_close(got, ref, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert err.max() <= max_abs and err.mean() <= mean_abs, (float(err.max()), float(err.mean()))
    return float(err.max()), float(err.mean())


def run_decode(pk, t, x, **kw):
    return pk.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["context_lens"], x.scale, sliding_window=x.sliding_window,
                           max_context_len=kw.pop("max_context_len", x.max_context_len), **kw)


def oracle_decode(x, k_cache=None, v_cache=None):
    return oracle.paged_decode(x.q, x.k_cache if k_cache is None else k_cache,
                               x.v_cache if v_cache is None else v_cache,
                               x.block_tables, x.context_lens, x.scale, x.sliding_window)


# --- kv_store ------------------------------------------------------------------

@pytest.mark.parametrize("nb,bs,hkv,n", [(40, 16, 8, 100), (9, 256, 8, 700), (5, 32, 2, 33)])
def test_kv_store_bit_exact(gpu_lib, nb, bs, hkv, n):
    rng = np.random.default_rng([21, nb, bs, n])
    kc = rng.integers(0, 1 << 16, size=(nb, bs, hkv, 128), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(nb, bs, hkv, 128), dtype=np.uint16)
    key = rng.integers(0, 1 << 16, size=(n, hkv, 128), dtype=np.uint16)
    value = rng.integers(0, 1 << 16, size=(n, hkv, 128), dtype=np.uint16)
    slots = rng.choice(nb * bs, size=n, replace=False).astype(np.int32)
    slots[::7] = -1                          # padding tokens
    slots[3] = nb * bs + 5                   # outside the cache: not stored
    x = W.PagedInputs(q=key[:1], k_cache=kc, v_cache=vc, block_tables=np.zeros((1, 1), np.int32),
                      context_lens=np.zeros(1, np.int32), block_size=bs, scale=1.0,
                      key=key, value=value, slot_mapping=slots)
    t = to_torch(x, "cuda")
    gpu_lib.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    oracle_slots = np.where(slots >= nb * bs, -1, slots)
    ek, ev = oracle.kv_store(kc, vc, key, value, oracle_slots)
    assert np.array_equal(bits_of(t["k_cache"]), ek)
    assert np.array_equal(bits_of(t["v_cache"]), ev)


def test_kv_store_no_tokens(gpu_lib):
    kc = torch.zeros(2, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    e = torch.empty(0, 8, 128, dtype=torch.bfloat16, device="cuda")
    gpu_lib.kv_store(e, e, torch.empty(0, dtype=torch.int32, device="cuda"), kc, vc)
    assert not kc.any() and not vc.any()


# --- decode on the named workloads ---------------------------------------------

def test_small_decode(gpu_lib):
    """8 seqs, ctx U{1..128}, block 16, 64 blocks in a random permutation."""
    x = W.small_decode()
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    assert_close(out, oracle_decode(x))


def test_store_then_decode(gpu_lib):
    """16 seqs, ctx U{256..512}, block 256: store the new token, then attend."""
    x = W.store_decode()
    t = to_torch(x, "cuda")
    gpu_lib.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    out = run_decode(gpu_lib, t, x)
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert np.array_equal(bits_of(t["k_cache"]), kc)
    assert np.array_equal(bits_of(t["v_cache"]), vc)
    assert_close(out, oracle_decode(x, kc, vc))


@pytest.mark.parametrize("layer", [0, 27])
def test_deep_decode_layer(gpu_lib, layer):
    """64 seqs, ctx U{512..1024}, block 256, q pre-scaled, scale 1.0 (one layer
    of the 28, at its full size)."""
    x = W.deep_decode_layer(layer)
    t = to_torch(x, "cuda")
    gpu_lib.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    out = run_decode(gpu_lib, t, x)
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert_close(out, oracle_decode(x, kc, vc))


def _sampled_long(gpu_lib, window, sample):
    """64 seqs, ctx U{4096..8192}, block 256, caches of 2048 blocks drawn on the
    GPU; the sampled sequences' blocks are copied to the host before any kernel
    runs and the oracle checks those sequences."""
    meta = W.long_decode_meta(window)
    dev = W.long_decode_device_caches("cuda")
    x = meta
    sub = {}
    for b in sample:
        nblk = math.ceil(int(x.context_lens[b]) / x.block_size)
        blocks = torch.from_numpy(x.block_tables[b, :nblk].astype(np.int64)).cuda()
        sub[b] = (bits_of(dev[0][blocks]), bits_of(dev[1][blocks]))
    t = to_torch(W.PagedInputs(q=x.q, k_cache=x.q[:0], v_cache=x.q[:0],
                               block_tables=x.block_tables, context_lens=x.context_lens,
                               block_size=x.block_size, scale=x.scale), "cuda")
    out = gpu_lib.paged_decode(t["q"], dev[0], dev[1], t["block_tables"], t["context_lens"],
                               x.scale, sliding_window=window, max_context_len=x.max_context_len)
    for b in sample:
        kb, vb = sub[b]
        tables = np.arange(kb.shape[0], dtype=np.int32)[None]
        ref = oracle.paged_decode(x.q[b:b + 1], kb, vb, tables, x.context_lens[b:b + 1],
                                  x.scale, window)
        assert_close(out[b:b + 1], ref)


def test_long_decode_sampled(gpu_lib):
    _sampled_long(gpu_lib, 0, [0, 17, 42, 63])


def test_long_decode_full_batch(gpu_lib):
    """64 seqs, ctx U{4096..8192} over all 64 sequences, in the planner's plan
    (one partition per sequence, longest first) and split into 2048-key
    partitions merged in the same launch: both 1 GiB caches are copied to the
    host before the launches, and the oracle walks the same block tables."""
    x = W.long_decode_meta(0)
    dev = W.long_decode_device_caches("cuda")
    kc, vc = bits_of(dev[0]), bits_of(dev[1])
    t = to_torch(W.PagedInputs(q=x.q, k_cache=x.q[:0], v_cache=x.q[:0],
                               block_tables=x.block_tables, context_lens=x.context_lens,
                               block_size=x.block_size, scale=x.scale), "cuda")
    ref = oracle.paged_decode(x.q, kc, vc, x.block_tables, x.context_lens, x.scale)
    assert gpu_lib.decode_plan(64, 8, x.max_context_len)[1] == 1
    assert gpu_lib.decode_plan(64, 8, x.max_context_len, 0, 2048)[1] == 4
    for ps in (0, 2048):
        out = gpu_lib.paged_decode(t["q"], dev[0], dev[1], t["block_tables"], t["context_lens"],
                                   x.scale, max_context_len=x.max_context_len, partition_size=ps)
        torch.cuda.synchronize()
        assert_close(out, ref)


def test_long_decode_window_sampled(gpu_lib):
    _sampled_long(gpu_lib, 256, [1, 5, 33, 60])


def test_long_decode_window_full_batch(gpu_lib):
    """The window-256 variant over all 64 sequences (its keys are few enough
    for the oracle): only the windowed blocks are copied to the host."""
    x = W.long_decode_meta(256)
    dev = W.long_decode_device_caches("cuda")
    t = to_torch(W.PagedInputs(q=x.q, k_cache=x.q[:0], v_cache=x.q[:0],
                               block_tables=x.block_tables, context_lens=x.context_lens,
                               block_size=x.block_size, scale=x.scale), "cuda")
    out = gpu_lib.paged_decode(t["q"], dev[0], dev[1], t["block_tables"], t["context_lens"],
                               x.scale, sliding_window=256, max_context_len=x.max_context_len)
    ref = np.zeros((64, 16, 128))
    for b in range(64):
        L = int(x.context_lens[b])
        lb0, lb1 = (L - 256) // 256, (L - 1) // 256
        blocks = torch.from_numpy(x.block_tables[b, lb0:lb1 + 1].astype(np.int64)).cuda()
        kb, vb = bits_of(dev[0][blocks]), bits_of(dev[1][blocks])
        # rebase: logical block lb0 becomes block 0 of a small table
        tables = np.arange(lb1 - lb0 + 1, dtype=np.int32)[None]
        L_local = L - lb0 * 256
        ref[b:b + 1] = oracle.paged_decode(x.q[b:b + 1], kb, vb, tables,
                                           np.array([L_local], np.int32), x.scale, 256)
    assert_close(out, ref)


# --- decode edge cases and invariants ------------------------------------------

def _random_case(seed, lens, bs=16, hq=16, hkv=8, mb=None, window=0, scale=None):
    rng = np.random.default_rng(seed)
    if mb is None:
        mb = max(1, max(math.ceil(L / bs) for L in lens))
    nb = len(lens) * mb + 3
    tables = rng.permutation(nb)[:len(lens) * mb].reshape(len(lens), mb).astype(np.int32)
    return W.PagedInputs(
        q=W.normal_bf16(rng, (len(lens), hq, 128)),
        k_cache=W.normal_bf16(rng, (nb, bs, hkv, 128)),
        v_cache=W.normal_bf16(rng, (nb, bs, hkv, 128)),
        block_tables=tables, context_lens=np.array(lens, np.int32), block_size=bs,
        scale=(1 / math.sqrt(128)) if scale is None else scale, sliding_window=window)


EDGE_LENS = [0, 1, 2, 15, 16, 17, 63, 64, 65, 255, 256, 257, 500, 1023, 1024]


@pytest.mark.parametrize("bs", [16, 32, 48, 64, 128, 256, 512, 1024])
@pytest.mark.parametrize("window", [0, 1, 17, 256])
def test_decode_edge_lengths(gpu_lib, bs, window):
    x = _random_case([31, bs, window], EDGE_LENS, bs=bs, window=window)
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    ref = oracle_decode(x)
    assert_close(out, ref)
    assert not out[0].any()                        # L = 0 -> zero row


@pytest.mark.parametrize("ps", [64, 128, 192, 512, 1024, 4096])
def test_decode_partition_sizes(gpu_lib, ps):
    """Every split (including one partition for everything) meets the bar."""
    x = _random_case([32], [1, 100, 700, 1500, 3000, 4096], bs=64)
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x, partition_size=ps)
    assert_close(out, oracle_decode(x))


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8), (4, 2)])
def test_decode_group_sizes(gpu_lib, hq, hkv):
    x = _random_case([33, hq, hkv], [5, 300, 1000], bs=32, hq=hq, hkv=hkv)
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    assert_close(out, oracle_decode(x))


# With at most 64 sequences, one partition each and more (seq, KV head) items
# than CUs, workgroups take the items in order of context length (ranked inside
# the kernel): ties, a partial second round of items and empty sequences.
@pytest.mark.parametrize("case", ["ties", "all_equal", "partial_round", "with_empty"])
def test_decode_length_ordered_batches(gpu_lib, case):
    rng = np.random.default_rng([41, len(case)])
    if case == "ties":
        lens = rng.choice([1, 17, 300, 300, 1024], size=40).tolist()
    elif case == "all_equal":
        lens = [512] * 64
    elif case == "partial_round":
        lens = rng.integers(1, 1025, size=33).tolist()      # 264 items for 256 CUs
    else:
        lens = rng.choice([0, 0, 5, 700], size=48).tolist()
    x = _random_case([42, len(case)], lens, bs=256)
    assert gpu_lib.decode_plan(len(lens), 8, max(lens))[1] == 1
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    assert_close(out, oracle_decode(x))
    for b, L in enumerate(lens):
        if L == 0:
            assert not out[b].any()


@pytest.mark.parametrize("bs", [16, 32, 48, 64])
def test_decode_length_ordered_small_blocks(gpu_lib, bs):
    """Ranked decode (40 seqs, one partition each) at block sizes where some
    wavefronts' first chunk lies past block 0: those read their table entry in
    the loop, the others take the one the ranking loaded."""
    lens = np.random.default_rng([46, bs]).integers(1, 700, size=40).tolist()
    x = _random_case([47, bs], lens, bs=bs)
    assert gpu_lib.decode_plan(len(lens), 8, max(lens))[1] == 1
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    assert_close(out, oracle_decode(x))


def test_decode_length_ordered_bad_first_block(gpu_lib):
    """Ranked decode with block 0 of some sequences outside the cache (the
    entry the ranking preloads): those 64 keys contribute nothing."""
    rng = np.random.default_rng(48)
    lens = rng.integers(65, 700, size=40).tolist()
    x = _random_case([49], lens, bs=64)
    nb = x.k_cache.shape[0]
    bad = {3: -5, 17: nb, 30: 1 << 30}
    good_tables = x.block_tables.copy()
    for b, e in bad.items():
        x.block_tables[b, 0] = e
    assert gpu_lib.decode_plan(len(lens), 8, max(lens))[1] == 1
    out = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    ref = oracle_decode(W.PagedInputs(**{**x.__dict__, "block_tables": good_tables}))
    for b in bad:
        # keys 64 .. L-1 only: the sequence's blocks from the second on
        tb = np.ascontiguousarray(good_tables[b:b + 1, 1:])
        ref[b:b + 1] = oracle.paged_decode(x.q[b:b + 1], x.k_cache, x.v_cache, tb,
                                           np.array([lens[b] - 64], np.int32), x.scale)
    assert_close(out, ref)


def test_decode_block_permutation_bit_exact(gpu_lib):
    x = _random_case([34], [37, 513, 900, 1024], bs=64)
    out1 = run_decode(gpu_lib, to_torch(x, "cuda"), x, partition_size=256)
    perm = np.random.default_rng(35).permutation(x.k_cache.shape[0])
    y = W.PagedInputs(**{**x.__dict__})
    y.k_cache = np.empty_like(x.k_cache)
    y.v_cache = np.empty_like(x.v_cache)
    y.k_cache[perm] = x.k_cache
    y.v_cache[perm] = x.v_cache
    y.block_tables = perm[x.block_tables].astype(np.int32)
    out2 = run_decode(gpu_lib, to_torch(y, "cuda"), y, partition_size=256)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    out3 = run_decode(gpu_lib, to_torch(x, "cuda"), x, partition_size=256)
    assert torch.equal(out1.view(torch.int16), out3.view(torch.int16))   # deterministic


def test_decode_unused_table_entries_never_used(gpu_lib):
    """Entries past ceil(L/block_size) hold a sentinel far outside the cache
    (the kernel may read the entry, but never uses it as a block id); the
    result is bit-identical to a table with valid entries there."""
    x = _random_case([36], [10, 200, 64], bs=32, mb=8)
    out1 = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    y = W.PagedInputs(**{**x.__dict__})
    y.block_tables = x.block_tables.copy()
    for b, L in enumerate(x.context_lens):
        y.block_tables[b, math.ceil(L / 32):] = np.iinfo(np.int32).max
    out2 = run_decode(gpu_lib, to_torch(y, "cuda"), y)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_decode_out_of_range_block_contributes_nothing(gpu_lib):
    """A used table entry outside [0, num_blocks) is skipped (no access)."""
    x = _random_case([37], [64, 64], bs=16, mb=4)
    t = to_torch(x, "cuda")
    x.block_tables[1, 2] = -5
    x.block_tables[0, 0] = 1 << 30
    t["block_tables"] = torch.from_numpy(x.block_tables).cuda()
    out = run_decode(gpu_lib, t, x)
    # oracle over the admitted blocks only: drop logical block 2 of seq 1 and 0 of seq 0
    keep = {0: [1, 2, 3], 1: [0, 1, 3]}
    ref = np.zeros((2, 16, 128))
    for b in range(2):
        tb = x.block_tables[b, keep[b]][None].astype(np.int32)
        ref[b:b + 1] = oracle.paged_decode(x.q[b:b + 1], x.k_cache, x.v_cache, tb,
                                           np.array([48], np.int32), x.scale)
    assert_close(out, ref)


def test_decode_prescaled_q_matches_scaled(gpu_lib):
    """q pre-scaled by 1/sqrt(d) with scale 1 agrees with raw q and scale 1/sqrt(d)
    (up to the bf16 rounding of the pre-scaled q)."""
    x = _random_case([38], [300, 700], bs=64)
    out1 = run_decode(gpu_lib, to_torch(x, "cuda"), x)
    y = W.PagedInputs(**{**x.__dict__})
    y.q = W.bf16_bits(oracle.bf16_to_f64(x.q).astype(np.float32) * np.float32(x.scale))
    y.scale = 1.0
    out2 = run_decode(gpu_lib, to_torch(y, "cuda"), y)
    assert_close(out2, out1.double().cpu().numpy(), max_abs=3e-2, mean_abs=4e-3)


# --- fused store + decode -------------------------------------------------------

def _fused_vs_unfused(pk, x, partition_size=0):
    t1 = to_torch(x, "cuda")
    pk.kv_store(t1["key"], t1["value"], t1["slot_mapping"], t1["k_cache"], t1["v_cache"])
    ref = run_decode(pk, t1, x, partition_size=partition_size)
    t2 = to_torch(x, "cuda")
    got = pk.paged_decode_store(t2["q"], t2["key"], t2["value"], t2["k_cache"], t2["v_cache"],
                                t2["block_tables"], t2["context_lens"], x.scale,
                                sliding_window=x.sliding_window, max_context_len=x.max_context_len,
                                partition_size=partition_size)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    assert torch.equal(t1["k_cache"].view(torch.int16), t2["k_cache"].view(torch.int16))
    assert torch.equal(t1["v_cache"].view(torch.int16), t2["v_cache"].view(torch.int16))
    return got, t2


def test_decode_store_fused_workload(gpu_lib):
    """16 seqs, ctx U{256..512}: one launch == store then decode, bit for bit,
    and within the bar of the oracle."""
    x = W.store_decode()
    got, _ = _fused_vs_unfused(gpu_lib, x)
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert_close(got, oracle_decode(x, kc, vc))


@pytest.mark.parametrize("window,ps", [(0, 0), (0, 64), (0, 256), (17, 0), (256, 64), (1, 0)])
def test_decode_store_fused_edges(gpu_lib, window, ps):
    lens = [1, 2, 15, 16, 17, 64, 65, 255, 256, 257, 1000]
    x = _random_case([39, window, ps], lens, bs=32, window=window)
    rng = np.random.default_rng([40, window])
    x.key = W.normal_bf16(rng, (len(lens), 8, 128))
    x.value = W.normal_bf16(rng, (len(lens), 8, 128))
    x.slot_mapping = np.array([W.slot_of(x.block_tables, b, L - 1, 32) for b, L in enumerate(lens)],
                              np.int32)
    _fused_vs_unfused(gpu_lib, x, partition_size=ps)


def test_decode_store_fused_length_ordered(gpu_lib):
    """40 seqs with tied lengths, one partition each: the fused store under the
    length-ordered work assignment."""
    lens = np.random.default_rng(43).choice([1, 16, 300, 300, 1024], size=40).tolist()
    x = _random_case([44], lens, bs=256)
    rng = np.random.default_rng(45)
    x.key = W.normal_bf16(rng, (len(lens), 8, 128))
    x.value = W.normal_bf16(rng, (len(lens), 8, 128))
    x.slot_mapping = np.array([W.slot_of(x.block_tables, b, L - 1, 256) for b, L in enumerate(lens)],
                              np.int32)
    got, _ = _fused_vs_unfused(gpu_lib, x)
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert_close(got, oracle_decode(x, kc, vc))


def test_decode_store_fused_deep_layer(gpu_lib):
    """A full 64-seq layer of the 28-layer workload, in the bench's launch plan."""
    x = W.deep_decode_layer(3)
    got, _ = _fused_vs_unfused(gpu_lib, x)
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert_close(got, oracle_decode(x, kc, vc))


@pytest.mark.parametrize("mcl", [80, 0])
def test_decode_store_fused_clamped_lengths(gpu_lib, mcl):
    """context_lens beyond max_context_len (a graph captured with a smaller
    bound) or beyond the table row: the new row goes to position L-1 when the
    table has an entry for it, else nowhere; attention covers the clamped
    range.  Equal, bit for bit, to kv_store (slot -1 where no slot exists) then
    paged_decode, and the caches change only at those slots."""
    pk = gpu_lib
    lens = [10, 100, 200, 64, 128, 129]
    bs, mb = 32, 4                                   # the table covers 128 positions
    x = _random_case([46, mcl], lens, bs=bs, mb=mb)
    rng = np.random.default_rng([47, mcl])
    x.key = W.normal_bf16(rng, (len(lens), 8, 128))
    x.value = W.normal_bf16(rng, (len(lens), 8, 128))
    x.slot_mapping = np.array([W.slot_of(x.block_tables, b, L - 1, bs) if L <= mb * bs else -1
                               for b, L in enumerate(lens)], np.int32)
    t1 = to_torch(x, "cuda")
    pk.kv_store(t1["key"], t1["value"], t1["slot_mapping"], t1["k_cache"], t1["v_cache"])
    ref = run_decode(pk, t1, x, max_context_len=mcl)
    t2 = to_torch(x, "cuda")
    got = pk.paged_decode_store(t2["q"], t2["key"], t2["value"], t2["k_cache"], t2["v_cache"],
                                t2["block_tables"], t2["context_lens"], x.scale, max_context_len=mcl)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    assert np.array_equal(bits_of(t2["k_cache"]), kc)
    assert np.array_equal(bits_of(t2["v_cache"]), vc)
    clamped = np.minimum(np.array(lens), min(mcl, mb * bs)).astype(np.int32)
    ref_o = oracle.paged_decode(x.q, kc, vc, x.block_tables, clamped, x.scale)
    assert_close(got, ref_o)
    if mcl == 0:
        assert not got.any()
