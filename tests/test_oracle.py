"""Pins for the CPU oracle, against things other than itself.

* brute force: dense, unpaged attention from torch's scaled_dot_product_attention
  (float64, CPU) on tiny inputs whose K/V were laid into a paged cache by a
  scatter written here;
* closed forms (one key, zero query, constant V, equal keys, one dominant key,
  a hand-derived golden fixture);
* invariants (physical-block permutation, kv_store round trip and canaries,
  decode == last prefill row, prefill chunking, window reductions, split-K
  merge over any partition).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return bf16_bits(np.asarray(x, dtype=np.float32))


def val(b):
    """bf16 bits -> float64, written independently of the oracle's decoder."""
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


def scatter_contiguous(seqs_k, seqs_v, block_size, rng, spare_blocks=2):
    """Lay contiguous per-sequence K/V [L_b, Hkv, d] into a paged cache whose
    physical blocks are a random permutation.  Written here, apart from the
    oracle, so that the oracle's table walk is checked, not reused."""
    hkv, d = seqs_k[0].shape[1:]
    need = [math.ceil(k.shape[0] / block_size) for k in seqs_k]
    mb = max(max(need), 1)
    nb = len(seqs_k) * mb + spare_blocks
    perm = rng.permutation(nb)
    tables = perm[: len(seqs_k) * mb].reshape(len(seqs_k), mb).astype(np.int32)
    kc = bits(rng.standard_normal((nb, block_size, hkv, d)))  # junk elsewhere
    vc = bits(rng.standard_normal((nb, block_size, hkv, d)))
    for b, (k, v) in enumerate(zip(seqs_k, seqs_v)):
        for j in range(k.shape[0]):
            blk = tables[b][j // block_size]
            kc[blk, j % block_size] = k[j]
            vc[blk, j % block_size] = v[j]
    return kc, vc, tables


def sdpa(q, k, v, scale, **kw):
    """q [Hq, n, d], k/v [Hkv, m, d] float64 -> [Hq, n, d]"""
    o = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None],
        torch.from_numpy(v)[None], scale=scale, enable_gqa=True, **kw)
    return o[0].numpy()


@pytest.mark.parametrize("hq,hkv,d,bs", [(16, 8, 128, 16), (4, 2, 16, 4), (8, 1, 8, 4), (4, 4, 8, 1)])
@pytest.mark.parametrize("window", [0, 5])
def test_decode_matches_dense_sdpa(hq, hkv, d, bs, window):
    rng = np.random.default_rng([7, hq, d, bs, window])
    lens = [1, 3, 17, 40]
    ks = [bits(rng.standard_normal((L, hkv, d))) for L in lens]
    vs = [bits(rng.standard_normal((L, hkv, d))) for L in lens]
    kc, vc, tables = scatter_contiguous(ks, vs, bs, rng)
    q = bits(rng.standard_normal((len(lens), hq, d)))
    scale = 1.0 / math.sqrt(d)
    out = oracle.paged_decode(q, kc, vc, tables, np.array(lens, np.int32), scale, window)
    for b, L in enumerate(lens):
        lo = max(0, L - window) if window else 0
        # the window taken by slicing K/V, not by a mask
        ref = sdpa(val(q[b])[:, None, :], val(ks[b][lo:]).transpose(1, 0, 2),
                   val(vs[b][lo:]).transpose(1, 0, 2), scale)[:, 0, :]
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,d,bs", [(16, 8, 128, 16), (4, 2, 16, 4), (2, 2, 8, 3)])
def test_prefill_matches_full_causal_sdpa(hq, hkv, d, bs):
    """Prefill over a cached prefix of P tokens == rows P.. of a full causal
    prefill of the whole sequence (torch's is_causal, which is exact for a
    square mask), so bottom-right alignment is checked by a library routine."""
    rng = np.random.default_rng([11, hq, d, bs])
    shapes = [(0, 5), (7, 1), (12, 9), (3, 20)]   # (prefix, new)
    ks, vs, qs_full = [], [], []
    for p, n in shapes:
        ks.append(bits(rng.standard_normal((p + n, hkv, d))))
        vs.append(bits(rng.standard_normal((p + n, hkv, d))))
        qs_full.append(bits(rng.standard_normal((p + n, hq, d))))
    kc, vc, tables = scatter_contiguous(ks, vs, bs, rng)
    q = np.concatenate([qf[p:] for qf, (p, n) in zip(qs_full, shapes)])
    cuq = np.concatenate([[0], np.cumsum([n for p, n in shapes])]).astype(np.int32)
    cuk = np.concatenate([[0], np.cumsum([p + n for p, n in shapes])]).astype(np.int32)
    scale = 0.3
    out = oracle.paged_prefill(q, kc, vc, tables, cuq, cuk, scale)
    for b, (p, n) in enumerate(shapes):
        ref = sdpa(val(qs_full[b]).transpose(1, 0, 2), val(ks[b]).transpose(1, 0, 2),
                   val(vs[b]).transpose(1, 0, 2), scale, is_causal=True)
        np.testing.assert_allclose(out[cuq[b]:cuq[b + 1]], ref[:, p:, :].transpose(1, 0, 2),
                                   rtol=0, atol=1e-12)


def test_prefill_window_matches_banded_sdpa():
    rng = np.random.default_rng(5)
    hq, hkv, d, bs, W = 4, 2, 16, 4, 6
    shapes = [(8, 10), (0, 13)]
    ks = [bits(rng.standard_normal((p + n, hkv, d))) for p, n in shapes]
    vs = [bits(rng.standard_normal((p + n, hkv, d))) for p, n in shapes]
    qf = [bits(rng.standard_normal((p + n, hq, d))) for p, n in shapes]
    kc, vc, tables = scatter_contiguous(ks, vs, bs, rng)
    q = np.concatenate([x[p:] for x, (p, n) in zip(qf, shapes)])
    cuq = np.array([0, 10, 23], np.int32)
    cuk = np.array([0, 18, 31], np.int32)
    out = oracle.paged_prefill(q, kc, vc, tables, cuq, cuk, 0.25, sliding_window=W)
    for b, (p, n) in enumerate(shapes):
        T = p + n
        band = torch.ones(T, T, dtype=torch.bool).tril().triu(-(W - 1))
        ref = sdpa(val(qf[b]).transpose(1, 0, 2), val(ks[b]).transpose(1, 0, 2),
                   val(vs[b]).transpose(1, 0, 2), 0.25, attn_mask=band)
        np.testing.assert_allclose(out[cuq[b]:cuq[b + 1]], ref[:, p:, :].transpose(1, 0, 2),
                                   rtol=0, atol=1e-12)


def test_golden_three_keys():
    with open(os.path.join(GOLDEN, "decode_three_keys.json")) as f:
        g = json.load(f)
    d, hq, hkv, bs, nb = g["head_dim"], g["num_q_heads"], g["num_kv_heads"], g["block_size"], g["num_blocks"]
    tables = np.array(g["block_tables"], np.int32)
    L = g["context_lens"][0]
    q = np.zeros((1, hq, d), np.float32)
    for h, dim, x in g["q_nonzero"]:
        q[0, h, dim] = x
    kc = np.full((nb, bs, hkv, d), 99.0, np.float32)   # junk outside the sequence
    vc = np.full((nb, bs, hkv, d), 99.0, np.float32)
    for j in range(L):
        blk, row = tables[0][j // bs], j % bs
        kc[blk, row] = 0.0
        for dim, x in g["k_rows"][str(j)].items():
            kc[blk, row, 0, int(dim)] = x
        vc[blk, row] = g["v_rows"][str(j)]
    out = oracle.paged_decode(bits(q), bits(kc), bits(vc), tables,
                              np.array(g["context_lens"], np.int32), g["scale"])
    for h, e in enumerate(g["expected_out"]):
        np.testing.assert_allclose(out[0, h], e, rtol=0, atol=1e-12)


def _case(rng, B=3, hq=4, hkv=2, d=16, bs=4, lens=(5, 1, 11)):
    mb = max(math.ceil(L / bs) for L in lens)
    nb = B * mb + 1
    tables = rng.permutation(nb)[: B * mb].reshape(B, mb).astype(np.int32)
    kc = bits(rng.standard_normal((nb, bs, hkv, d)))
    vc = bits(rng.standard_normal((nb, bs, hkv, d)))
    q = bits(rng.standard_normal((B, hq, d)))
    return q, kc, vc, tables, np.array(lens, np.int32)


def test_one_key_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    q, kc, vc, tables, _ = _case(rng)
    ctx = np.array([1, 1, 1], np.int32)
    out = oracle.paged_decode(q, kc, vc, tables, ctx, 0.7)
    for b in range(3):
        blk = tables[b][0]
        for h in range(4):
            assert np.array_equal(out[b, h], val(vc[blk, 0, h // 2]))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    q, kc, vc, tables, ctx = _case(rng)
    q[:] = 0
    out = oracle.paged_decode(q, kc, vc, tables, ctx, 0.5)
    for b, L in enumerate(ctx):
        for h in range(4):
            rows = [val(vc[tables[b][j // 4], j % 4, h // 2]) for j in range(L)]
            np.testing.assert_allclose(out[b, h], np.mean(rows, axis=0), atol=1e-12)


def test_constant_values_and_equal_keys():
    rng = np.random.default_rng(3)
    q, kc, vc, tables, ctx = _case(rng)
    vc2 = np.full_like(vc, bits(np.float32(1.5))[()])
    out = oracle.paged_decode(q, kc, vc2, tables, ctx, 0.5)
    np.testing.assert_allclose(out, 1.5, atol=1e-12)
    kc2 = np.broadcast_to(kc[:1, :1], kc.shape).copy()
    out = oracle.paged_decode(q, kc2, vc, tables, ctx, 0.5)
    ref = oracle.paged_decode(np.zeros_like(q), kc, vc, tables, ctx, 0.5)
    np.testing.assert_allclose(out, ref, atol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    q, kc, vc, tables, ctx = _case(rng, lens=(9, 9, 9))
    q[:] = 0
    q[:, :, 0] = bits(np.float32(1.0))
    kc[:, :, :, 0] = 0
    j = 6
    kc[tables[1][j // 4], j % 4, :, 0] = bits(np.float32(64.0))
    out = oracle.paged_decode(q, kc, vc, tables, ctx, 1.0)   # score gap 64 -> e^-64
    for h in range(4):
        np.testing.assert_allclose(out[1, h], val(vc[tables[1][j // 4], j % 4, h // 2]),
                                   rtol=0, atol=1e-20)


def test_block_permutation_invariance_bit_exact():
    rng = np.random.default_rng(5)
    q, kc, vc, tables, ctx = _case(rng, lens=(13, 7, 16))
    out = oracle.paged_decode(q, kc, vc, tables, ctx, 0.3)
    perm = rng.permutation(kc.shape[0])          # new physical position of each block
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    out2 = oracle.paged_decode(q, kc2, vc2, perm[tables].astype(np.int32), ctx, 0.3)
    assert np.array_equal(out, out2)


def test_kv_store_round_trip_and_canaries():
    rng = np.random.default_rng(6)
    nb, bs, hkv, d = 6, 4, 2, 8
    kc = bits(rng.standard_normal((nb, bs, hkv, d)))
    vc = bits(rng.standard_normal((nb, bs, hkv, d)))
    n = 9
    slots = rng.choice(nb * bs, size=n, replace=False).astype(np.int32)
    slots[3] = -1
    key = rng.integers(0, 1 << 16, size=(n, hkv, d), dtype=np.uint16)  # any bit pattern
    value = rng.integers(0, 1 << 16, size=(n, hkv, d), dtype=np.uint16)
    kc2, vc2 = oracle.kv_store(kc, vc, key, value, slots)
    flat_k, flat_v = kc2.reshape(nb * bs, hkv, d), vc2.reshape(nb * bs, hkv, d)
    for i, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(flat_k[s], key[i]) and np.array_equal(flat_v[s], value[i])
    untouched = np.setdiff1d(np.arange(nb * bs), slots[slots >= 0])
    assert np.array_equal(flat_k[untouched], kc.reshape(nb * bs, hkv, d)[untouched])
    assert np.array_equal(flat_v[untouched], vc.reshape(nb * bs, hkv, d)[untouched])
    # slot s is block s // block_size, row s % block_size
    s = int(slots[0])
    assert np.array_equal(kc2[s // bs, s % bs], key[0])
    with pytest.raises(AssertionError):
        oracle.kv_store(kc, vc, key[:2], value[:2], np.array([5, 5], np.int32))


def test_decode_equals_last_prefill_row():
    rng = np.random.default_rng(8)
    q, kc, vc, tables, ctx = _case(rng, lens=(5, 1, 11))
    dec = oracle.paged_decode(q, kc, vc, tables, ctx, 0.4, sliding_window=3)
    cuq = np.arange(4, dtype=np.int32)                    # one query per sequence
    cuk = np.concatenate([[0], np.cumsum(ctx)]).astype(np.int32)
    pre = oracle.paged_prefill(q, kc, vc, tables, cuq, cuk, 0.4, sliding_window=3)
    np.testing.assert_allclose(pre, dec, atol=1e-13)


def test_prefill_chunk_invariance():
    """Prefill of Lq tokens after prefix P == prefill of the first c tokens
    after P, then of the remaining tokens after P + c."""
    rng = np.random.default_rng(9)
    B, hq, hkv, d, bs = 2, 4, 2, 16, 4
    P, Lq, c = [4, 0], [9, 6], [5, 2]
    q, kc, vc, tables, _ = _case(rng, B=B, lens=(16, 16))
    qn = bits(rng.standard_normal((sum(Lq), hq, d)))
    cuq = np.array([0, Lq[0], sum(Lq)], np.int32)
    cuk = np.array([0, P[0] + Lq[0], P[0] + Lq[0] + P[1] + Lq[1]], np.int32)
    whole = oracle.paged_prefill(qn, kc, vc, tables, cuq, cuk, 0.3)
    rows1 = np.concatenate([qn[cuq[b]:cuq[b] + c[b]] for b in range(B)])
    rows2 = np.concatenate([qn[cuq[b] + c[b]:cuq[b + 1]] for b in range(B)])
    o1 = oracle.paged_prefill(rows1, kc, vc, tables, np.array([0, c[0], c[0] + c[1]], np.int32),
                              np.array([0, P[0] + c[0], P[0] + c[0] + P[1] + c[1]], np.int32), 0.3)
    n2 = [Lq[b] - c[b] for b in range(B)]
    o2 = oracle.paged_prefill(rows2, kc, vc, tables, np.array([0, n2[0], n2[0] + n2[1]], np.int32), cuk, 0.3)
    for b in range(B):
        np.testing.assert_allclose(whole[cuq[b]:cuq[b] + c[b]], o1[sum(c[:b]):sum(c[:b + 1])], atol=1e-13)
        np.testing.assert_allclose(whole[cuq[b] + c[b]:cuq[b + 1]], o2[sum(n2[:b]):sum(n2[:b + 1])], atol=1e-13)


def test_window_reductions():
    rng = np.random.default_rng(10)
    q, kc, vc, tables, ctx = _case(rng, lens=(5, 1, 11))
    full = oracle.paged_decode(q, kc, vc, tables, ctx, 0.4)
    big = oracle.paged_decode(q, kc, vc, tables, ctx, 0.4, sliding_window=11)
    assert np.array_equal(full, big)
    one = oracle.paged_decode(q, kc, vc, tables, ctx, 0.4, sliding_window=1)
    for b, L in enumerate(ctx):
        j = L - 1
        for h in range(4):
            assert np.array_equal(one[b, h], val(vc[tables[b][j // 4], j % 4, h // 2]))


def test_gqa_equal_queries_give_equal_outputs():
    rng = np.random.default_rng(12)
    q, kc, vc, tables, ctx = _case(rng)
    q[:, 1] = q[:, 0]
    q[:, 3] = q[:, 2]
    out = oracle.paged_decode(q, kc, vc, tables, ctx, 0.5)
    assert np.array_equal(out[:, 0], out[:, 1]) and np.array_equal(out[:, 2], out[:, 3])
    assert not np.allclose(out[:, 0], out[:, 2])


def test_merge_partials_any_split():
    rng = np.random.default_rng(13)
    d, n = 16, 37
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    qv = rng.standard_normal(d)
    whole = oracle.attention_rows(qv[None], k, v, 0.6, np.ones((1, n), bool))[0]
    for cuts in ([0, n], [0, 10, 10, 37], [0, 1, 2, 30, 37], [0, 0, 37, 37]):
        parts = [oracle.partial_attention(qv, k[a:b], v[a:b], 0.6)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_allclose(oracle.merge_partials(parts), whole, atol=1e-13)
    empty = [oracle.partial_attention(qv, k[:0], v[:0], 0.6)] * 2
    assert np.array_equal(oracle.merge_partials(empty), np.zeros(d))


def test_empty_sequence_is_zero():
    rng = np.random.default_rng(14)
    q, kc, vc, tables, _ = _case(rng)
    out = oracle.paged_decode(q, kc, vc, tables, np.array([0, 3, 0], np.int32), 0.5)
    assert not out[0].any() and not out[2].any() and out[1].any()


def test_bf16_decoder_matches_torch():
    x = np.random.default_rng(15).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    x = x[((x >> 7) & 0xFF) != 0xFF]                 # skip Inf/NaN patterns
    assert np.array_equal(oracle.bf16_to_f64(x), val(x))
