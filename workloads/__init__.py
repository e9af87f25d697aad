"""Seeded synthetic inputs for paged KV-cache attention.

This module only draws inputs: random values, random lengths, random block
tables and slot maps.  It holds none of the attention arithmetic, so both the
CPU oracle and the HIP path can take their inputs from it without sharing any
of the method.

bf16 tensors are carried on the host as ``numpy.uint16`` bit patterns, so a
round trip through the cache can be compared bit for bit.

Shapes follow a Qwen3-0.6B-shaped grouped-query attention layer: 16 query
heads, 8 KV heads, head_dim 128.  The five named workloads are shaped like the
bench tiers and long-context settings of the nano-vLLM pages (nano-vllm-rs
README, "Benchmark" tiers fast / normal / heavy; nano-vllm-sansho README,
max_model_len 8192 and the SWA-256 export).  Every random draw is seeded from
``numpy.random.default_rng([ROOT_SEED, workload_id, ...])``; the root seed 0
matches the ``--seed 0`` of the nano-vllm-rs bench command.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

ROOT_SEED = 0
NUM_Q_HEADS = 16
NUM_KV_HEADS = 8
HEAD_DIM = 128

# Workload ids, used as the second seed word.
SMALL_DECODE = 1        # 8 seqs, ctx U{1..128}, block 16, 64 blocks permuted
STORE_DECODE = 2        # 16 seqs, ctx U{256..512}, block 256, store new token first
DEEP_DECODE = 3         # 64 seqs, ctx U{512..1024}, block 256, 28 layers, q pre-scaled
PREFIX_PREFILL = 4      # 16 seqs, new U{64..512} + prefix of 0-2 full blocks
LONG_DECODE = 5         # 64 seqs, ctx U{4096..8192}, block 256 (+ window 256 variant)
MIXED_BATCH = 6         # chunked-prefill step: 48 decode seqs + 4 prefill chunks, block 256


def rng_for(workload_id: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([ROOT_SEED, workload_id, *sub])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even); return uint16 bits.

    Inputs are drawn in float32 and rounded once here, so both sides see the
    same bf16 numbers.  No NaN or Inf is ever drawn.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, mul: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if mul != 1.0:
        x = x * np.float32(mul)
    return bf16_bits(x)


@dataclasses.dataclass
class PagedInputs:
    """One batch of paged-cache inputs.

    k_cache / v_cache: uint16 [num_blocks, block_size, num_kv_heads, head_dim]
    q:                 uint16 [num_seqs, num_q_heads, head_dim] (decode) or
                       uint16 [total_q, num_q_heads, head_dim] (prefill)
    block_tables:      int32 [num_seqs, max_blocks_per_seq]
    context_lens:      int32 [num_seqs]  (decode: keys including the new token;
                                          prefill: prefix + new tokens)
    key / value / slot_mapping: new tokens to store before attention, or None
    cu_seqlens_q / cu_seqlens_k: int32 [num_seqs + 1] (prefill only)
    """
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    block_size: int
    scale: float
    sliding_window: int = 0
    key: Optional[np.ndarray] = None
    value: Optional[np.ndarray] = None
    slot_mapping: Optional[np.ndarray] = None
    cu_seqlens_q: Optional[np.ndarray] = None
    cu_seqlens_k: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0


def permuted_block_tables(rng: np.random.Generator, num_seqs: int,
                          blocks_per_seq: int) -> np.ndarray:
    """A random permutation of num_seqs*blocks_per_seq physical blocks,
    row b of the result being the blocks sequence b owns."""
    perm = rng.permutation(num_seqs * blocks_per_seq).astype(np.int32)
    return perm.reshape(num_seqs, blocks_per_seq)


def slot_of(block_tables: np.ndarray, b: int, pos, block_size: int):
    """Physical slot of logical position(s) ``pos`` of sequence b.

    Used only to say where the workload's new tokens go (an input), not by
    either implementation.
    """
    pos = np.asarray(pos, dtype=np.int64)
    return block_tables[b, pos // block_size].astype(np.int64) * block_size + pos % block_size


def decode_inputs(workload_id: int, num_seqs: int, ctx_lo: int, ctx_hi: int,
                  block_size: int, *, blocks_per_seq: Optional[int] = None,
                  layer: int = 0, q_mul: float = 1.0, scale: Optional[float] = None,
                  sliding_window: int = 0, store_new_token: bool = False,
                  with_caches: bool = True,
                  heads=(NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)) -> PagedInputs:
    """Decode batch: one query token per sequence over a paged cache.

    context_lens ~ U{ctx_lo..ctx_hi} inclusive.  Each sequence owns
    ``blocks_per_seq`` blocks (default: enough for ctx_hi) taken from one random
    permutation of all blocks.  With ``store_new_token`` the token at position
    L_b - 1 is drawn separately and stored through slot_mapping before
    attention.  The lengths and tables depend only on ``workload_id``; the
    values also on ``layer``.  With ``with_caches=False`` the caches are left
    empty (shape [0, ...]) for drawing on the GPU with ``device_caches``.
    """
    hq, hkv, d = heads
    if blocks_per_seq is None:
        blocks_per_seq = math.ceil(ctx_hi / block_size)
    meta = rng_for(workload_id, 0)
    ctx = meta.integers(ctx_lo, ctx_hi, endpoint=True, size=num_seqs).astype(np.int32)
    tables = permuted_block_tables(meta, num_seqs, blocks_per_seq)
    nb = num_seqs * blocks_per_seq
    vals = rng_for(workload_id, 1, layer)
    q = normal_bf16(vals, (num_seqs, hq, d), mul=q_mul)
    cshape = (nb if with_caches else 0, block_size, hkv, d)
    kc = normal_bf16(vals, cshape)
    vc = normal_bf16(vals, cshape)
    out = PagedInputs(q=q, k_cache=kc, v_cache=vc, block_tables=tables,
                      context_lens=ctx, block_size=block_size,
                      scale=(1.0 / math.sqrt(d)) if scale is None else scale,
                      sliding_window=sliding_window)
    if store_new_token:
        out.key = normal_bf16(vals, (num_seqs, hkv, d))
        out.value = normal_bf16(vals, (num_seqs, hkv, d))
        out.slot_mapping = np.array(
            [slot_of(tables, b, int(ctx[b]) - 1, block_size) for b in range(num_seqs)],
            dtype=np.int32)
    return out


def prefill_inputs(workload_id: int, num_seqs: int, new_lo: int, new_hi: int,
                   prefix_blocks_max: int, block_size: int, *,
                   blocks_per_seq: Optional[int] = None, sliding_window: int = 0,
                   heads=(NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)) -> PagedInputs:
    """Varlen prefill batch over a partly cached prefix.

    New lengths Lq_b ~ U{new_lo..new_hi}; cached prefix P_b = 0..prefix_blocks_max
    full blocks (uniform).  The prefix K/V are already in the cache (the cache
    is filled with N(0,1) everywhere); the new tokens' K/V are drawn separately
    and stored through slot_mapping at positions P_b .. P_b + Lq_b - 1.
    """
    hq, hkv, d = heads
    meta = rng_for(workload_id, 0)
    lq = meta.integers(new_lo, new_hi, endpoint=True, size=num_seqs).astype(np.int32)
    pref = (meta.integers(0, prefix_blocks_max, endpoint=True, size=num_seqs)
            * block_size).astype(np.int32)
    lk = (pref + lq).astype(np.int32)
    if blocks_per_seq is None:
        blocks_per_seq = math.ceil((prefix_blocks_max * block_size + new_hi) / block_size)
    tables = permuted_block_tables(meta, num_seqs, blocks_per_seq)
    nb = num_seqs * blocks_per_seq
    cuq = np.zeros(num_seqs + 1, np.int32)
    cuq[1:] = np.cumsum(lq)
    cuk = np.zeros(num_seqs + 1, np.int32)
    cuk[1:] = np.cumsum(lk)
    total_q = int(cuq[-1])
    vals = rng_for(workload_id, 1)
    q = normal_bf16(vals, (total_q, hq, d))
    kc = normal_bf16(vals, (nb, block_size, hkv, d))
    vc = normal_bf16(vals, (nb, block_size, hkv, d))
    key = normal_bf16(vals, (total_q, hkv, d))
    value = normal_bf16(vals, (total_q, hkv, d))
    slots = np.concatenate([
        slot_of(tables, b, np.arange(pref[b], lk[b]), block_size) for b in range(num_seqs)
    ]).astype(np.int32)
    return PagedInputs(q=q, k_cache=kc, v_cache=vc, block_tables=tables,
                       context_lens=lk, block_size=block_size,
                       scale=1.0 / math.sqrt(d), sliding_window=sliding_window,
                       key=key, value=value, slot_mapping=slots,
                       cu_seqlens_q=cuq, cu_seqlens_k=cuk)


def mixed_inputs(workload_id: int, decode_seqs: int, ctx_lo: int, ctx_hi: int,
                 prefill_seqs: int, new_lo: int, new_hi: int, prefix_blocks_max: int,
                 block_size: int, heads=(NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)) -> PagedInputs:
    """One mixed step of a chunked-prefill scheduler: decode sequences first
    (one new token each, context L ~ U{ctx_lo..ctx_hi}, i.e. a cached prefix of
    L - 1), then prefill chunks (new tokens ~ U{new_lo..new_hi} over a cached
    prefix of 0..prefix_blocks_max full blocks).  The layout is the varlen
    prefill's: cu_seqlens_q / cu_seqlens_k, new K/V stored through slot_mapping."""
    hq, hkv, d = heads
    meta = rng_for(workload_id, 0)
    dec_ctx = meta.integers(ctx_lo, ctx_hi, endpoint=True, size=decode_seqs)
    chunk = meta.integers(new_lo, new_hi, endpoint=True, size=prefill_seqs)
    pref = meta.integers(0, prefix_blocks_max, endpoint=True, size=prefill_seqs) * block_size
    lq = np.concatenate([np.ones(decode_seqs, np.int64), chunk]).astype(np.int32)
    lk = np.concatenate([dec_ctx, pref + chunk]).astype(np.int32)
    n = decode_seqs + prefill_seqs
    blocks_per_seq = int(max(math.ceil(int(L) / block_size) for L in lk))
    tables = permuted_block_tables(meta, n, blocks_per_seq)
    nb = n * blocks_per_seq
    cuq = np.zeros(n + 1, np.int32)
    cuq[1:] = np.cumsum(lq)
    cuk = np.zeros(n + 1, np.int32)
    cuk[1:] = np.cumsum(lk)
    total_q = int(cuq[-1])
    vals = rng_for(workload_id, 1)
    q = normal_bf16(vals, (total_q, hq, d))
    kc = normal_bf16(vals, (nb, block_size, hkv, d))
    vc = normal_bf16(vals, (nb, block_size, hkv, d))
    key = normal_bf16(vals, (total_q, hkv, d))
    value = normal_bf16(vals, (total_q, hkv, d))
    slots = np.concatenate([
        slot_of(tables, b, np.arange(int(lk[b]) - int(lq[b]), int(lk[b])), block_size) for b in range(n)
    ]).astype(np.int32)
    return PagedInputs(q=q, k_cache=kc, v_cache=vc, block_tables=tables,
                       context_lens=lk, block_size=block_size,
                       scale=1.0 / math.sqrt(d), sliding_window=0,
                       key=key, value=value, slot_mapping=slots,
                       cu_seqlens_q=cuq, cu_seqlens_k=cuk)


# --- the five named workloads -------------------------------------------------

def small_decode() -> PagedInputs:
    """8 seqs, ctx U{1..128}, block 16, 64 blocks in a random permutation."""
    return decode_inputs(SMALL_DECODE, 8, 1, 128, 16, blocks_per_seq=8)


def store_decode() -> PagedInputs:
    """16 seqs, ctx U{256..512}, block 256; the new token is stored first."""
    return decode_inputs(STORE_DECODE, 16, 256, 512, 256, store_new_token=True)


DEEP_DECODE_LAYERS = 28


def deep_decode_layer(layer: int, num_seqs: int = 64) -> PagedInputs:
    """One of 28 independent layers: 64 seqs, ctx U{512..1024}, block 256.

    q is drawn N(0,1), multiplied by 1/sqrt(128) in float32 and rounded to
    bf16 ("q pre-scaled"), and the kernel scale is 1.0.  Lengths and tables
    are shared by all layers; q, K and V are drawn per layer.
    """
    return decode_inputs(DEEP_DECODE, num_seqs, 512, 1024, 256, layer=layer,
                         q_mul=1.0 / math.sqrt(HEAD_DIM), scale=1.0,
                         store_new_token=True)


def prefix_prefill() -> PagedInputs:
    """16 seqs, new U{64..512}, prefix 0-2 full 256-token blocks."""
    return prefill_inputs(PREFIX_PREFILL, 16, 64, 512, 2, 256)


def long_decode(sliding_window: int = 0, num_seqs: int = 64) -> PagedInputs:
    """64 seqs, ctx U{4096..8192}, block 256; optional window of 256."""
    return decode_inputs(LONG_DECODE, num_seqs, 4096, 8192, 256,
                         sliding_window=sliding_window)


LONG_DECODE_BLOCKS = 64 * 32


MIXED_BATCH_TOKENS = 4096   # the scheduler's token budget for one step


def mixed_batch() -> PagedInputs:
    """A chunked-prefill step under a 4096-token budget: 48 decode sequences
    (context U{256..2048}) and 4 prefill chunks (U{256..1024} new tokens over a
    prefix of 0-4 full blocks), block 256."""
    x = mixed_inputs(MIXED_BATCH, 48, 256, 2048, 4, 256, 1024, 4, 256)
    assert int(x.cu_seqlens_q[-1]) <= MIXED_BATCH_TOKENS
    return x


def long_decode_meta(sliding_window: int = 0) -> PagedInputs:
    """The long-context workload without its 2 GiB of caches (q, tables and
    lengths only); draw the caches with long_decode_device_caches()."""
    return decode_inputs(LONG_DECODE, 64, 4096, 8192, 256,
                         sliding_window=sliding_window, with_caches=False)


def long_decode_device_caches(device):
    return device_caches(LONG_DECODE, LONG_DECODE_BLOCKS, 256, device)


def deep_decode_layer_meta(layer: int) -> PagedInputs:
    """One layer of the 28-layer workload without its caches."""
    return decode_inputs(DEEP_DECODE, 64, 512, 1024, 256, layer=layer,
                         q_mul=1.0 / math.sqrt(HEAD_DIM), scale=1.0,
                         store_new_token=True, with_caches=False)


def device_caches(workload_id: int, num_blocks: int, block_size: int, device, layer: int = 0,
                  heads=(NUM_Q_HEADS, NUM_KV_HEADS, HEAD_DIM)):
    """(k_cache, v_cache) bf16 N(0,1) [num_blocks, block_size, Hkv, d] drawn on
    the GPU (see device_normal_bf16)."""
    shape = (num_blocks, block_size, heads[1], heads[2])
    return (device_normal_bf16(shape, [workload_id, 2, layer, 0], device),
            device_normal_bf16(shape, [workload_id, 2, layer, 1], device))


# --- device-side drawing for the full-size workloads ---------------------------

def device_normal_bf16(shape, seed_words, device, mul: float = 1.0):
    """N(0,1) bf16 drawn on the GPU with torch's seeded generator.

    Used for the multi-GiB caches of the full-size workloads, where drawing on
    the host would take minutes.  The seed is derived from the same seed words
    as the host draws.  A test that checks such an input copies it to the host
    before any kernel runs on it.
    """
    import torch
    seed = int(np.random.SeedSequence([ROOT_SEED, *seed_words]).generate_state(1)[0])
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if mul != 1.0:
        x.mul_(mul)
    return x.to(torch.bfloat16)


def to_torch(x: PagedInputs, device) -> dict:
    """The same arrays as torch tensors on ``device`` (bf16 bits reinterpreted
    as torch.bfloat16, index arrays as int32)."""
    import torch

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    t = {
        "q": bf(x.q), "k_cache": bf(x.k_cache), "v_cache": bf(x.v_cache),
        "block_tables": i32(x.block_tables), "context_lens": i32(x.context_lens),
    }
    if x.key is not None:
        t["key"] = bf(x.key)
        t["value"] = bf(x.value)
        t["slot_mapping"] = i32(x.slot_mapping)
    if x.cu_seqlens_q is not None:
        t["cu_seqlens_q"] = i32(x.cu_seqlens_q)
        t["cu_seqlens_k"] = i32(x.cu_seqlens_k)
    return t


def bits_of(t) -> np.ndarray:
    """A torch bf16 tensor (any device) -> numpy uint16 bit patterns."""
    import torch
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
