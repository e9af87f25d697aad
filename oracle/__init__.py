"""CPU oracle for attention over a paged KV cache — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library's product path never does;
the two share no code, no constants and no helpers.

What it computes.  The pages (nano-vllm-rs README, "Run Inference" and "GGUF
Models": a paged KV cache whose block size is a knob; lunaryes/nano-vllm
diagram, "Components" and "Connections": a KV block manager that allocates
cached blocks and a model runner that sets an execution context; the
nano-vllm-sansho README, "Sansho Serving Roofline Anchors": q=1 decode and a
sliding-window-256 model, "Key Features": prefix caching) name the pieces but
never write the formula.  The plain reading is taken: textbook scaled-dot-
product softmax attention per (sequence, query head), over the key positions
that the causal and window rules admit, with each key/value row fetched by
walking the sequence's block table.  Everything is done in float64, so the
oracle's own rounding error (~1e-15) is negligible next to bf16 (~4e-3).

Readings taken where the pages are silent (each pinned by a test in
tests/test_oracle.py):
  * cache layout [num_blocks, block_size, num_kv_heads, head_dim]; a slot s is
    row s % block_size of block s // block_size;
  * logical position j of sequence b lives in slot
    block_tables[b, j // block_size] * block_size + j % block_size;
  * query head h reads KV head h // (num_q_heads // num_kv_heads);
  * decode: context_lens[b] counts the new token, which is the query, so the
    query sits at position L-1 and sees keys 0..L-1;
  * prefill with a cached prefix of P tokens: new query i sits at position
    P + i and sees keys 0..P+i (causal, aligned bottom-right);
  * sliding window W > 0: a query at position t sees keys j with t - j < W
    (W keys including itself); W = 0 means no window;
  * a slot of -1 in slot_mapping is a padding token and is not stored;
  * a sequence with no admitted keys yields a zero output row.

Parity status: every function here is pinned (see tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64", "kv_store", "gather_rows", "attention_rows", "paged_decode",
    "paged_prefill", "partial_attention", "merge_partials",
]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  A bf16 value is the upper half
    of a float32, so the conversion is exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def kv_store(k_cache: np.ndarray, v_cache: np.ndarray, key: np.ndarray,
             value: np.ndarray, slot_mapping: np.ndarray):
    """Store new K/V rows into the paged cache (a bit copy); returns new caches.

    For every token i with slot_mapping[i] >= 0, the [num_kv_heads, head_dim]
    rows key[i] / value[i] go to slot slot_mapping[i], i.e. block
    slot // block_size, row slot % block_size.  Slots must be distinct (two
    tokens in one slot would make the result depend on write order).
    """
    nb, bs, hkv, d = k_cache.shape
    slots = [int(s) for s in np.asarray(slot_mapping).ravel()]
    used = [s for s in slots if s >= 0]
    assert len(set(used)) == len(used), "slot_mapping entries must be distinct"
    kc = k_cache.copy()
    vc = v_cache.copy()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert s < nb * bs, "slot out of range"
        kc[s // bs, s % bs] = key[i]
        vc[s // bs, s % bs] = value[i]
    return kc, vc


def gather_rows(cache: np.ndarray, block_tables: np.ndarray, b: int,
                positions: np.ndarray, kv_head: int) -> np.ndarray:
    """Rows of one KV head for logical positions of sequence b, found by
    walking the block table: block = block_tables[b, j // block_size],
    row = j % block_size.  Returns float64 [len(positions), head_dim]."""
    bs = cache.shape[1]
    positions = np.asarray(positions, dtype=np.int64)
    blocks = block_tables[b, positions // bs].astype(np.int64)
    return bf16_to_f64(cache[blocks, positions % bs, kv_head, :])


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   allowed: np.ndarray) -> np.ndarray:
    """Softmax attention for query rows q [n, d] over keys k, v [m, d].

    ``allowed`` [n, m] says which keys each query sees.  out_i =
    sum_j p_ij v_j with p_ij = exp(s_ij - max_j s_ij) / sum_j exp(...) over
    allowed j, s_ij = scale * <q_i, k_j>.  Rows with no allowed key are 0.
    """
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    out = np.zeros((q.shape[0], v.shape[1]), dtype=np.float64)
    has_key = allowed.any(axis=1)
    if not has_key.any():
        return out
    s = s[has_key]
    p = np.exp(s - s.max(axis=1, keepdims=True))
    out[has_key] = (p @ v) / p.sum(axis=1, keepdims=True)
    return out


def paged_decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                 block_tables: np.ndarray, context_lens: np.ndarray, scale: float,
                 sliding_window: int = 0) -> np.ndarray:
    """Decode attention, one query token per sequence (the q=1 decode step).

    q: bf16 bits [B, Hq, d].  For sequence b with L = context_lens[b] the
    query is at position L-1 and attends keys lo..L-1, lo = max(0, L-W) when a
    window W > 0 is set.  Returns float64 [B, Hq, d].
    """
    nbs, hq, d = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    out = np.zeros((nbs, hq, d), dtype=np.float64)
    for b in range(nbs):
        L = int(context_lens[b])
        if L <= 0:
            continue
        lo = max(0, L - sliding_window) if sliding_window > 0 else 0
        pos = np.arange(lo, L)
        for g in range(hkv):
            k = gather_rows(k_cache, block_tables, b, pos, g)
            v = gather_rows(v_cache, block_tables, b, pos, g)
            heads = list(range(g * grp, (g + 1) * grp))
            qg = bf16_to_f64(q[b, heads, :])
            allowed = np.ones((grp, len(pos)), dtype=bool)
            out[b, heads, :] = attention_rows(qg, k, v, scale, allowed)
    return out


def paged_prefill(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                  block_tables: np.ndarray, cu_seqlens_q: np.ndarray,
                  cu_seqlens_k: np.ndarray, scale: float,
                  sliding_window: int = 0, seqs=None) -> np.ndarray:
    """Variable-length causal prefill over a partly cached prefix.

    q: bf16 bits [total_q, Hq, d], sequence b owning rows
    cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1.  Sequence b has Lk =
    cu_seqlens_k[b+1] - cu_seqlens_k[b] keys in the cache (its prefix and its
    new tokens, already stored), Lq new queries and prefix P = Lk - Lq.  New
    query i is at position P + i and attends keys j <= P + i (and P + i - j < W
    when a window W > 0 is set).  Returns float64 [total_q, Hq, d]; with
    ``seqs`` only those sequences' rows are filled.
    """
    total_q, hq, d = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    nseq = len(cu_seqlens_q) - 1
    for b in (range(nseq) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        lq = q1 - q0
        lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if lq <= 0:
            continue
        prefix = lk - lq
        assert prefix >= 0, "each sequence needs at least as many keys as queries"
        qpos = prefix + np.arange(lq)[:, None]
        kpos = np.arange(lk)[None, :]
        allowed = kpos <= qpos
        if sliding_window > 0:
            allowed &= (qpos - kpos) < sliding_window
        pos = np.arange(lk)
        for g in range(hkv):
            k = gather_rows(k_cache, block_tables, b, pos, g)
            v = gather_rows(v_cache, block_tables, b, pos, g)
            for h in range(g * grp, (g + 1) * grp):
                qh = bf16_to_f64(q[q0:q1, h, :])
                out[q0:q1, h, :] = attention_rows(qh, k, v, scale, allowed)
    return out


def partial_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Un-normalised attention state of one query q [d] over a subset of keys:
    (m, l, acc) with m = max_j s_j, l = sum_j exp(s_j - m),
    acc = sum_j exp(s_j - m) v_j.  An empty subset gives (-inf, 0, 0)."""
    d = v.shape[1]
    if k.shape[0] == 0:
        return -np.inf, 0.0, np.zeros(d, dtype=np.float64)
    s = scale * (k @ q)
    m = s.max()
    p = np.exp(s - m)
    return m, p.sum(), p @ v


def merge_partials(parts) -> np.ndarray:
    """Combine per-partition states (the split-K / flash-decoding merge).

    With M = max_p m_p, out = sum_p exp(m_p - M) acc_p / sum_p exp(m_p - M) l_p.
    Empty partitions (m = -inf, l = 0) contribute nothing; if every part is
    empty the result is 0.
    """
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    d = parts[0][2].shape[0]
    if not np.isfinite(ms).any():
        return np.zeros(d, dtype=np.float64)
    big = ms.max()
    w = np.where(np.isfinite(ms), np.exp(ms - big), 0.0)
    num = sum(wi * p[2] for wi, p in zip(w, parts))
    den = sum(wi * p[1] for wi, p in zip(w, parts))
    return num / den
