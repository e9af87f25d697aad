"""GPU parity of the varlen prefill over a cached prefix (through the C ABI)
against the CPU oracle: the named 16-sequence workload in full, and edge
cases (ragged tails, prefixes not aligned to tiles, windows, head groups,
block sizes, empty sequences, sentinel table padding)."""
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


def assert_close(got, ref, rows=None, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.isfinite(g).all()
    err = np.abs(g - ref)
    assert err.max() <= max_abs and err.mean() <= mean_abs, (float(err.max()), float(err.mean()))


def prefill_case(seed, shapes, bs=64, hq=16, hkv=8, window=0, spare=2, mb=None):
    """shapes: list of (cached prefix P, new tokens Lq).  The cache is N(0,1)
    everywhere; new K/V are drawn separately and stored at positions P.."""
    rng = np.random.default_rng(seed)
    need = [max(1, math.ceil((p + n) / bs)) for p, n in shapes]
    mb = mb or max(need)
    nb = len(shapes) * mb + spare
    tables = rng.permutation(nb)[:len(shapes) * mb].reshape(len(shapes), mb).astype(np.int32)
    lq = np.array([n for p, n in shapes], np.int32)
    lk = np.array([p + n for p, n in shapes], np.int32)
    cuq = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    total = int(cuq[-1])
    slots = np.concatenate([W.slot_of(tables, b, np.arange(p, p + n), bs)
                            for b, (p, n) in enumerate(shapes)] + [np.zeros(0)]).astype(np.int32)
    return W.PagedInputs(
        q=W.normal_bf16(rng, (total, hq, 128)),
        k_cache=W.normal_bf16(rng, (nb, bs, hkv, 128)),
        v_cache=W.normal_bf16(rng, (nb, bs, hkv, 128)),
        block_tables=tables, context_lens=lk, block_size=bs, scale=1 / math.sqrt(128),
        sliding_window=window,
        key=W.normal_bf16(rng, (total, hkv, 128)), value=W.normal_bf16(rng, (total, hkv, 128)),
        slot_mapping=slots, cu_seqlens_q=cuq, cu_seqlens_k=cuk)


def run_store_prefill(pk, x, t=None, max_seqlen_q=None):
    t = t or to_torch(x, "cuda")
    pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    msq = max_seqlen_q or int(np.diff(x.cu_seqlens_q).max())
    out = pk.paged_prefill(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                           t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale,
                           max_seqlen_q=msq, sliding_window=x.sliding_window)
    return out, t


def oracle_prefill(x):
    kc, vc = oracle.kv_store(x.k_cache, x.v_cache, x.key, x.value, x.slot_mapping)
    return oracle.paged_prefill(x.q, kc, vc, x.block_tables, x.cu_seqlens_q, x.cu_seqlens_k,
                                x.scale, x.sliding_window), kc, vc


def test_prefix_prefill_workload(gpu_lib):
    """16 seqs, new U{64..512}, prefix 0-2 full 256-token blocks, block 256."""
    x = W.prefix_prefill()
    out, t = run_store_prefill(gpu_lib, x)
    ref, kc, vc = oracle_prefill(x)
    assert np.array_equal(bits_of(t["k_cache"]), kc)
    assert np.array_equal(bits_of(t["v_cache"]), vc)
    assert_close(out, ref)


SHAPES = [(0, 1), (0, 63), (0, 64), (0, 65), (100, 1), (100, 37), (5, 130), (256, 200),
          (0, 300), (513, 64)]


@pytest.mark.parametrize("bs", [16, 32, 48, 64, 128, 256, 512, 1024])
def test_prefill_shapes_block_sizes(gpu_lib, bs):
    x = prefill_case([41, bs], SHAPES, bs=bs)
    out, _ = run_store_prefill(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


@pytest.mark.parametrize("window", [1, 17, 64, 100, 256])
def test_prefill_window(gpu_lib, window):
    x = prefill_case([42, window], SHAPES, bs=32, window=window)
    out, _ = run_store_prefill(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8), (4, 2)])
def test_prefill_group_sizes(gpu_lib, hq, hkv):
    x = prefill_case([43, hq, hkv], [(0, 40), (70, 90), (3, 129)], bs=32, hq=hq, hkv=hkv)
    out, _ = run_store_prefill(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


def test_prefill_empty_sequences(gpu_lib):
    """Sequences with no new tokens own no output rows; neighbours are exact."""
    x = prefill_case([44], [(10, 0), (0, 50), (64, 0), (30, 70)], bs=16)
    out, _ = run_store_prefill(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


def test_prefill_single_token_equals_decode(gpu_lib):
    """Lq = 1 after a prefix of L-1 tokens is one decode step."""
    x = prefill_case([45], [(0, 1), (99, 1), (700, 1), (255, 1)], bs=64)
    out, t = run_store_prefill(gpu_lib, x)
    dec = gpu_lib.paged_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                               torch.from_numpy(x.context_lens).cuda(), x.scale,
                               max_context_len=int(x.context_lens.max()))
    ref = oracle_prefill(x)[0]
    assert_close(out, ref)
    assert_close(dec, ref)


def test_mixed_batch_workload(gpu_lib):
    """A chunked-prefill step in one varlen launch: 48 decode sequences (one
    new token each) then 4 prefill chunks over cached prefixes, block 256."""
    x = W.mixed_batch()
    out, t = run_store_prefill(gpu_lib, x)
    ref, kc, vc = oracle_prefill(x)
    assert np.array_equal(bits_of(t["k_cache"]), kc)
    assert np.array_equal(bits_of(t["v_cache"]), vc)
    assert_close(out, ref)
    # The decode rows are one decode step of those sequences.
    nd = int(np.sum(np.diff(x.cu_seqlens_q) == 1))
    dec = gpu_lib.paged_decode(t["q"][:nd].contiguous(), t["k_cache"], t["v_cache"],
                               t["block_tables"][:nd].contiguous(),
                               torch.from_numpy(x.context_lens[:nd]).cuda(), x.scale,
                               max_context_len=int(x.context_lens[:nd].max()))
    assert_close(dec, ref[:nd])
    assert_close(out[:nd], dec.double().cpu().numpy(), max_abs=2e-2, mean_abs=2e-3)


def test_prefill_chunked_matches_whole(gpu_lib):
    """Two chunks (the second one over a prefix that includes the first) give
    the same rows as one pass, within the bf16 bar."""
    whole = prefill_case([46], [(0, 200), (64, 150)], bs=32)
    out_whole, t = run_store_prefill(gpu_lib, whole)
    c = [80, 33]
    rows1 = np.concatenate([np.arange(0, c[0]), np.arange(200, 200 + c[1])])
    rows2 = np.concatenate([np.arange(c[0], 200), np.arange(200 + c[1], 350)])
    for rows, cuq, cuk in (
            (rows1, [0, c[0], c[0] + c[1]], [0, c[0], c[0] + 64 + c[1]]),
            (rows2, [0, 200 - c[0], 350 - c[0] - c[1]], [0, 200, 200 + 214])):
        q = t["q"][torch.from_numpy(rows).cuda()].contiguous()
        out = gpu_lib.paged_prefill(q, t["k_cache"], t["v_cache"], t["block_tables"],
                                    torch.tensor(cuq, dtype=torch.int32, device="cuda"),
                                    torch.tensor(cuk, dtype=torch.int32, device="cuda"),
                                    whole.scale, max_seqlen_q=int(np.diff(cuq).max()))
        d = (out.float() - out_whole[torch.from_numpy(rows).cuda()].float()).abs()
        assert d.max().item() <= 2e-2 and d.mean().item() <= 2e-3


def test_prefill_permutation_bit_exact_and_deterministic(gpu_lib):
    x = prefill_case([47], [(100, 120), (0, 77)], bs=32, spare=5)
    out1, t = run_store_prefill(gpu_lib, x)
    out1b = gpu_lib.paged_prefill(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                  t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale, max_seqlen_q=120)
    assert torch.equal(out1.view(torch.int16), out1b.view(torch.int16))
    perm = np.random.default_rng(48).permutation(x.k_cache.shape[0])
    y = W.PagedInputs(**{**x.__dict__})
    y.k_cache = np.empty_like(x.k_cache)
    y.v_cache = np.empty_like(x.v_cache)
    y.k_cache[perm] = x.k_cache
    y.v_cache[perm] = x.v_cache
    y.block_tables = perm[x.block_tables].astype(np.int32)
    y.slot_mapping = (perm[x.slot_mapping // 32] * 32 + x.slot_mapping % 32).astype(np.int32)
    out2, _ = run_store_prefill(gpu_lib, y)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_prefill_work_order_invariant(gpu_lib):
    """Which workgroup takes which (sequence, query tile) item does not change a bit
    of the output.  The same batch with max_seqlen_q 448 / 512 / 576 has 112 / 128
    / 144 items: the first two are taken in order of key-tile count (ranked inside
    the kernel, 128 being the most it ranks), the last latest query tile first.
    Three prefixes pass 63 key tiles, where ranked counts tie; empty sequences
    and single tokens sit between them."""
    shapes = [(2100, 100), (2150, 90), (2300, 64), (0, 448), (0, 0), (5, 1), (256, 200),
              (700, 0), (31, 33), (64, 64), (1000, 5), (0, 129), (512, 300), (3, 3),
              (1500, 17), (0, 2)]
    x = prefill_case([53], shapes, bs=256)
    outs = []
    t = None
    for msq in (448, 512, 576):
        out, t = run_store_prefill(gpu_lib, x, t=t, max_seqlen_q=msq)
        outs.append(out.clone())
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    assert_close(outs[0], oracle_prefill(x)[0])
    # The fused store under both orders: output and caches as store-then-prefill.
    for msq in (512, 576):
        out, tf = run_fused(gpu_lib, x, max_seqlen_q=msq)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), outs[0].view(torch.int16))
        assert torch.equal(tf["k_cache"].view(torch.int16), t["k_cache"].view(torch.int16))
        assert torch.equal(tf["v_cache"].view(torch.int16), t["v_cache"].view(torch.int16))


def test_prefill_sentinel_padding_never_read(gpu_lib):
    x = prefill_case([49], [(10, 30), (0, 5)], bs=16, mb=8)
    out1, _ = run_store_prefill(gpu_lib, x)
    y = W.PagedInputs(**{**x.__dict__})
    y.block_tables = x.block_tables.copy()
    for b, L in enumerate(x.context_lens):
        y.block_tables[b, math.ceil(L / 16):] = np.iinfo(np.int32).max
    out2, _ = run_store_prefill(gpu_lib, y)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_prefill_long_prefix_window(gpu_lib):
    """A long cached prefix (1800 tokens) with a window of 256 and with none."""
    for window in (0, 256):
        x = prefill_case([50, window], [(1800, 300), (1000, 17)], bs=256, window=window)
        out, _ = run_store_prefill(gpu_lib, x)
        assert_close(out, oracle_prefill(x)[0])


# ---- fused store + prefill (pk_paged_prefill_store) ---------------------------

def run_fused(pk, x, max_seqlen_q=None):
    """The fused entry on fresh copies of the inputs: (out, tensors)."""
    t = to_torch(x, "cuda")
    msq = max_seqlen_q or int(np.diff(x.cu_seqlens_q).max())
    out = pk.paged_prefill_store(t["q"], t["key"], t["value"], t["k_cache"], t["v_cache"],
                                 t["block_tables"], t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale,
                                 max_seqlen_q=msq, sliding_window=x.sliding_window)
    return out, t


def assert_fused_equals_unfused(pk, x):
    """Output and both caches bit-identical to kv_store then paged_prefill."""
    ref_out, tr = run_store_prefill(pk, x)
    out, tf = run_fused(pk, x)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(tf["k_cache"].view(torch.int16), tr["k_cache"].view(torch.int16))
    assert torch.equal(tf["v_cache"].view(torch.int16), tr["v_cache"].view(torch.int16))
    return out, tf


def test_prefill_store_workload(gpu_lib):
    """The 16-sequence prefix workload: fused == store + prefill, bit for bit,
    and both match the oracle (caches bit-exact)."""
    x = W.prefix_prefill()
    out, t = assert_fused_equals_unfused(gpu_lib, x)
    ref, kc, vc = oracle_prefill(x)
    assert np.array_equal(bits_of(t["k_cache"]), kc)
    assert np.array_equal(bits_of(t["v_cache"]), vc)
    assert_close(out, ref)


@pytest.mark.parametrize("bs", [16, 32, 48, 64, 256])
def test_prefill_store_block_sizes(gpu_lib, bs):
    """Every block-addressing mode (division for 48, shifts below a tile,
    tiles inside a block), prefixes off the tile grid."""
    x = prefill_case([51, bs], SHAPES, bs=bs)
    out, _ = assert_fused_equals_unfused(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


@pytest.mark.parametrize("window", [17, 256])
def test_prefill_store_window(gpu_lib, window):
    x = prefill_case([52, window], SHAPES, bs=64, window=window)
    out, _ = assert_fused_equals_unfused(gpu_lib, x)
    assert_close(out, oracle_prefill(x)[0])


def test_prefill_store_mixed_and_empty(gpu_lib):
    """The mixed decode + chunk batch, and sequences with no new tokens."""
    assert_fused_equals_unfused(gpu_lib, W.mixed_batch())
    assert_fused_equals_unfused(gpu_lib, prefill_case([53], [(10, 0), (0, 50), (64, 0), (30, 70)], bs=16))


def test_prefill_store_bad_table_entry(gpu_lib):
    """A block-table entry outside the cache inside a sequence's range: its
    positions are neither stored nor attended, exactly as kv_store (which
    skips the slot) then paged_prefill."""
    x = prefill_case([54], [(40, 100), (0, 70)], bs=32, mb=6)
    x.block_tables = x.block_tables.copy()
    x.block_tables[0, 3] = x.k_cache.shape[0] + 5      # new positions 96..127 of sequence 0
    x.block_tables[1, 0] = -7                          # new positions 0..31 of sequence 1
    bad = np.zeros(len(x.slot_mapping), bool)
    x.slot_mapping = x.slot_mapping.copy()
    for b, (p, n) in enumerate([(40, 100), (0, 70)]):
        q0 = int(x.cu_seqlens_q[b])
        for i in range(n):
            blk = x.block_tables[b, (p + i) // 32]
            if not 0 <= blk < x.k_cache.shape[0]:
                x.slot_mapping[q0 + i] = -1
                bad[q0 + i] = True
    assert bad.any()
    out, _ = assert_fused_equals_unfused(gpu_lib, x)
    assert torch.isfinite(out.float()).all()


# ---- mixed batch split by kind (pk_paged_prefill_decode) ---------------------

def run_mixed(pk, x, nd, out=None):
    t = to_torch(x, "cuda")
    pk.kv_store(t["key"], t["value"], t["slot_mapping"], t["k_cache"], t["v_cache"])
    lq = np.diff(x.cu_seqlens_q)
    lk = np.diff(x.cu_seqlens_k)
    res = pk.paged_prefill_decode(t["q"], t["k_cache"], t["v_cache"], t["block_tables"],
                                  t["cu_seqlens_q"], t["cu_seqlens_k"], x.scale,
                                  num_decode_seqs=nd,
                                  max_seqlen_q=int(lq[nd:].max()) if nd < len(lq) else 1,
                                  max_decode_context_len=int(lk[:nd].max()) if nd else 0,
                                  sliding_window=x.sliding_window, out=out)
    return res, t


def check_split_matches_parts(pk, x, nd):
    """Decode rows bit-identical to pk_paged_decode of those sequences, the
    other rows bit-identical to pk_paged_prefill of the remaining ones."""
    out, t = run_mixed(pk, x, nd)
    lk = np.diff(x.cu_seqlens_k)
    if nd:
        dec = pk.paged_decode(t["q"][:nd].contiguous(), t["k_cache"], t["v_cache"],
                              t["block_tables"][:nd].contiguous(),
                              torch.from_numpy(lk[:nd].astype(np.int32)).cuda(), x.scale,
                              max_context_len=int(lk[:nd].max()), sliding_window=x.sliding_window)
        assert torch.equal(out[:nd].view(torch.int16), dec.view(torch.int16))
    if nd < x.num_seqs:
        pre = pk.paged_prefill(t["q"], t["k_cache"], t["v_cache"], t["block_tables"][nd:].contiguous(),
                               t["cu_seqlens_q"][nd:].contiguous(), t["cu_seqlens_k"][nd:].contiguous(),
                               x.scale, max_seqlen_q=int(np.diff(x.cu_seqlens_q)[nd:].max()),
                               sliding_window=x.sliding_window)
        r0 = int(x.cu_seqlens_q[nd])
        assert torch.equal(out[r0:].view(torch.int16), pre[r0:].view(torch.int16))
    return out


def test_mixed_split_workload(gpu_lib):
    """The chunked-prefill step (48 decode rows + 4 chunks): decode rows on the
    decode kernel, chunks on the prefill kernel, all within the bar of the oracle."""
    x = W.mixed_batch()
    nd = int(np.sum(np.diff(x.cu_seqlens_q) == 1))
    assert nd == 48
    out = check_split_matches_parts(gpu_lib, x, nd)
    assert_close(out, oracle_prefill(x)[0])


@pytest.mark.parametrize("window", [0, 100])
def test_mixed_split_extremes_and_long(gpu_lib, window):
    """All prefill, all decode, and decode contexts long enough to be split
    over partitions (merged in their own launch, workspace) next to prefill chunks."""
    shapes = [(5000, 1), (1, 1), (3000, 1), (700, 1), (0, 90), (300, 33)]
    x = prefill_case([55, window], shapes, bs=64, window=window)
    for nd in (0, 4):
        out = check_split_matches_parts(gpu_lib, x, nd)
        assert_close(out, oracle_prefill(x)[0])
    y = prefill_case([56, window], shapes[:4], bs=64, window=window)
    out = check_split_matches_parts(gpu_lib, y, 4)
    assert_close(out, oracle_prefill(y)[0])


@pytest.mark.parametrize("bs", [16, 32, 256])
def test_mixed_split_block_sizes(gpu_lib, bs):
    """Decode rows in one partition next to prefill chunks: one combined launch
    for power-of-two blocks of >= 32 keys, two launches for block 16; either
    way bit-identical to the separate kernels and within the oracle's bar."""
    shapes = [(300, 1), (40, 1), (700, 1), (129, 1), (100, 200), (0, 77), (513, 64)]
    x = prefill_case([58, bs], shapes, bs=bs)
    out = check_split_matches_parts(gpu_lib, x, 4)
    assert_close(out, oracle_prefill(x)[0])


@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8), (64, 8)])
def test_mixed_split_group_sizes(gpu_lib, hq, hkv):
    """The combined launch for 1 and 4 query heads per KV head (2 is the
    workload above); 8 takes two launches.  Bit-identical either way."""
    shapes = [(200, 1), (517, 1), (64, 1), (100, 150), (0, 70)]
    x = prefill_case([59, hq], shapes, bs=64, hq=hq, hkv=hkv)
    out = check_split_matches_parts(gpu_lib, x, 3)
    assert_close(out, oracle_prefill(x)[0])


def test_mixed_split_bad_leading_sequence_untouched(gpu_lib):
    """A leading 'decode' sequence with two new tokens is left unwritten."""
    x = prefill_case([57], [(50, 1), (60, 2), (70, 1), (0, 40)], bs=32)
    t = to_torch(x, "cuda")
    sentinel = torch.full_like(t["q"], 7.0)
    out, _ = run_mixed(gpu_lib, x, 3, out=sentinel.clone())
    rows = slice(int(x.cu_seqlens_q[1]), int(x.cu_seqlens_q[2]))
    assert torch.equal(out[rows].view(torch.int16), sentinel[rows].view(torch.int16))
    ref = oracle_prefill(x)[0]
    keep = np.ones(len(ref), bool)
    keep[rows] = False
    assert_close(out, ref, rows=np.nonzero(keep)[0])
