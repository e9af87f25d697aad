// paged_decode: attention of one query token per sequence over the paged KV
// cache (nano-vllm-sansho README, "Sansho Serving Roofline Anchors": the q=1
// decode step, and its sliding-window-256 model), split over the context
// (flash-decoding), the partitions merged in the same launch by the last of
// them to finish (or by a separate combine kernel).
//
// Work decomposition.  For (sequence b, KV head g) the admitted key positions
// [lo, L) are cut into partitions of PS tokens starting at lo.
// One workgroup of NW wavefronts reduces one partition; it serves all G query
// heads that share KV head g, so every K/V byte is read from HBM exactly once.
//
// Inside a wavefront each lane owns 16 bytes (8 dims) of a 256-byte head row,
// so one 128-bit load per lane covers 4 consecutive tokens (rows of 16 lanes).
// Tokens are taken in chunks of 16 (four such loads for K and four for V);
// a chunk never straddles a cache block because block_size is a multiple of 16,
// so one block-table entry serves the whole chunk.  Each 16-lane row keeps its
// own online-softmax state (running max m, sum l, fp32 accumulator), so the
// inner loop needs no cross-row traffic: q.k is reduced over the row's 16 lanes
// with DPP moves, everything else is lane-local.  Rows, then wavefronts, are
// merged only once at the end (shuffles, then LDS).  The next chunk's loads
// are issued before the current chunk is consumed.
//
// Scores are kept in the log2 domain: q is pre-multiplied by scale*log2(e) in
// fp32 and the hardware exp2 is used.
//
// A partition's result is either written as the final bf16 output (when the
// sequence has a single partition) or as the partial state (m, l, acc) that is
// merged: out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.  The merge is done
// by the sequence's last partition to finish (a device-scope arrival counter),
// or, without counters, by the combine kernel; both use the same code, so the
// results are bit-identical.
#pragma once

#include "device_common.h"
#include "launch.h"

// Tuning knobs (compile-time): wavefronts per workgroup, 128-bit loads per
// chunk for K (and as many for V; a chunk is 4 tokens per load), and whether
// K/V loads carry the non-temporal hint (the cache is streamed once).
#ifndef PK_DECODE_WAVES
#define PK_DECODE_WAVES 4
#endif
#ifndef PK_DECODE_LOADS
#define PK_DECODE_LOADS 4
#endif
#ifndef PK_DECODE_NT
#define PK_DECODE_NT 1
#endif
#ifndef PK_DECODE_DOT2
#define PK_DECODE_DOT2 1    // q.k with packed bf16 dot products (fp32 products and sums)
#endif

namespace pk {
namespace {

constexpr float kEmptyMax = -1.0e30f;   // running max before any key (finite: 2^(m-m) stays 1)

struct SeqRange {
  int L;        // admitted keys end (exclusive)
  int lo;       // admitted keys begin
  int nparts;   // partitions of the admitted keys (0 when L == 0)
  int row;      // q / out row of the sequence; -1: not computed (varlen form only)
};

// Context length of sequence b (with its new token).
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  return a.cu_seqlens_k ? a.cu_seqlens_k[b + 1] - a.cu_seqlens_k[b] : a.context_lens[b];
}

__device__ __forceinline__ SeqRange seq_range(const DecodeArgs& a, int b) {
  SeqRange r;
  const int cap = min(a.max_blocks_per_seq * a.block_size, a.max_context_len);
  r.L = min(max(seq_len(a, b), 0), cap);
  r.row = b;
  if (a.cu_seqlens_q) {
    r.row = a.cu_seqlens_q[b];
    if (a.cu_seqlens_q[b + 1] - r.row != 1 || r.row < 0 || r.row >= a.total_rows) r.row = -1;
  }
  r.lo = a.sliding_window > 0 ? max(0, r.L - a.sliding_window) : 0;
  // Partitions start at lo (not at multiples of the partition size), so a
  // window of W keys takes ceil(W / partition_size) of them.
  const int keys = r.L - r.lo;   // written so that nothing below can overflow int32
  r.nparts = r.L > 0 ? keys / a.partition_size + (keys % a.partition_size != 0) : 0;
  // The host plan sizes num_parts for the worst sequence; the clamp only keeps
  // workspace indexing in bounds should a caller break that contract.
  r.nparts = min(r.nparts, a.num_parts);
  return r;
}

template <int NL>
struct ChunkRegs {
  uint4 k[NL];
  uint4 v[NL];
  int64_t off;   // offset (16-byte units) of the chunk's first token in the caches
  bool ok;       // the chunk's block-table entry is a valid block
};

__device__ __forceinline__ uint4 load16(const uint4* p) {
#if PK_DECODE_NT
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

// The chunk at token `base`, whose cache block (logical block lb of the
// sequence) has table entry blk.
template <int NL>
__device__ __forceinline__ void load_chunk_at(ChunkRegs<NL>& c, const DecodeArgs& a, int blk, int lb,
                                              bool dummy, const uint4* kbase, const uint4* vbase,
                                              int64_t tok_stride, int64_t blk_stride, int base) {
  c.ok = !dummy && static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks);
  blk = c.ok ? blk : 0;
  c.off = dummy ? 0
                : static_cast<int64_t>(blk) * blk_stride +
                      static_cast<int64_t>(base - lb * a.block_size) * tok_stride;
#pragma unroll
  for (int k = 0; k < NL; ++k) c.k[k] = load16(kbase + c.off + 4 * k * tok_stride);
#pragma unroll
  for (int k = 0; k < NL; ++k) c.v[k] = load16(vbase + c.off + 4 * k * tok_stride);
}

// Chunk of 4*NL tokens starting at logical position `base` (a multiple of
// 4*NL that divides block_size, so the chunk lies in one cache block).  The
// table index is clamped into the row, and an entry outside the cache reads
// block 0 with `ok` false, so every address is in bounds whatever the table
// holds.  base < 0 asks for a dummy chunk (the prefetch past a wavefront's
// last chunk, never consumed): it reads the first tokens of cache block 0,
// which every workgroup shares, so it hits in L2 instead of fetching again
// from HBM (the K/V loads are non-temporal).
template <int NL>
__device__ __forceinline__ void load_chunk(ChunkRegs<NL>& c, const DecodeArgs& a,
                                           const int32_t* bt, const uint4* kbase,
                                           const uint4* vbase, int64_t tok_stride,
                                           int64_t blk_stride, int base) {
  const bool dummy = base < 0;
  const int lb = dummy ? 0 : min(base / a.block_size, a.max_blocks_per_seq - 1);
  load_chunk_at<NL>(c, a, bt[lb], lb, dummy, kbase, vbase, tok_stride, blk_stride, base);
}

// Work order by length.  Workgroups are dealt round-robin over the 8 XCDs and
// then over each XCD's 32 CUs, so workgroup w (one partition per sequence,
// grid (1, Hkv, B)) lands on CU slot q = w mod 256 in round r = w / 256.  Items
// (seq, KV head) are ranked by context length, longest first (all heads of a
// sequence in a row); round r takes ranks 256r .. 256r+255, in order on even
// rounds and mirrored on odd ones.  The CUs that got the longest items first
// get the shortest next, which evens out the bytes each CU streams, and the
// longest items start first.  Every wavefront ranks the <= 64 context lengths
// itself (one per lane, ties by index), so no wavefront waits on another.
__device__ __forceinline__ void length_ordered_item(const DecodeArgs& a, int by, int bz, int& b, int& g,
                                                    int& blk0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int B = a.num_seqs;
  const int w = by + a.num_kv_heads * bz;
  const int n = B * a.num_kv_heads;
  const int r = w / 256, q = w % 256;
  const int n_r = min(256, n - 256 * r);
  const int rank = 256 * r + ((r & 1) ? n_r - 1 - q : q);
  const int target = rank / a.num_kv_heads;   // rank of the sequence
  g = rank % a.num_kv_heads;
  const int cap = min(a.max_blocks_per_seq * a.block_size, a.max_context_len);
  // Unique keys, larger = earlier: length, then lower index first; 0 = no sequence.
  uint32_t key = 0;
  int e0 = 0;   // the sequence's first block-table entry, loaded with its length
  if (lane < B) {
    e0 = a.block_tables[static_cast<int64_t>(lane) * a.max_blocks_per_seq];
    const int L = min(max(seq_len(a, lane), 0), cap);
    key = ((static_cast<uint32_t>(L) << 6) | static_cast<uint32_t>(63 - lane)) + 1u;
  }
  // Radix select of the key with exactly `target` keys above it, from the top
  // bit down: among the remaining candidates, those with the bit set are all
  // above those without, so one ballot per bit decides which group holds it.
  uint64_t cand = __ballot(lane < B);
  int need = target;   // candidates above the wanted key not yet skipped
  const int nbits = 32 - __builtin_clz((static_cast<uint32_t>(cap) << 6) + 64u);
  for (int bit = nbits - 1; bit >= 0; --bit) {
    const uint64_t ones = __ballot((key >> bit) & 1u) & cand;
    const int c = __builtin_popcountll(ones);
    const bool in_ones = need < c;
    cand = in_ones ? ones : (cand & ~ones);
    need = in_ones ? need : need - c;
  }
  const uint64_t hit = cand;
  b = __builtin_amdgcn_readfirstlane(static_cast<int>(__builtin_ctzll(hit)));
  blk0 = __builtin_amdgcn_readlane(e0, b);
}

// One workgroup's work; (bx, by, bz) = (partition, KV head, sequence) in the
// kernel's own grid.  Also run by the mixed-batch kernel (mixed.hip).
// The output of (query head `head`, dim d) from the partials of its `nparts`
// partitions: one online pass in partition order, out = sum_p 2^(m_p-M) acc_p /
// sum_p 2^(m_p-M) l_p.  Each step's loads do not depend on the running state,
// so the unrolled loads are all in flight together.  COH: device-coherent loads
// (partials written by workgroups of the same launch).
template <bool COH>
__device__ __forceinline__ float merge_partials(const DecodeArgs& a, int64_t head, int d, int nparts) {
  const float* ml = a.ws_ml + head * a.num_parts * 2;
  const float* acc = a.ws_acc + head * a.num_parts * kHeadDim + d;
  auto ld = [](const float* p) __attribute__((always_inline)) {
    if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
  };
  float mx = kEmptyMax, ls = 0.f, av = 0.f;
#pragma unroll 4
  for (int p = 0; p < nparts; ++p) {
    const float mp = ld(ml + 2 * p);
    const float lp = ld(ml + 2 * p + 1);
    const float ap = ld(acc + p * kHeadDim);
    const float mn = fmaxf(mx, mp);
    const float fo = fast_exp2(mx - mn);
    const float fn = fast_exp2(mp - mn);
    ls = ls * fo + lp * fn;
    av = av * fo + ap * fn;
    mx = mn;
  }
  return ls > 0.f ? av / ls : 0.f;
}

// MERGE: a split sequence's partitions are merged in the same launch by the
// last of them to finish (a.merge_counters); else by the combine kernel.
template <int G, int NW, int NL, bool FUSE, bool MERGE = false>
__device__ __forceinline__ void decode_partition_body(const DecodeArgs& a, int bx, int by, int bz) {
  constexpr int CT = 4 * NL;   // tokens per chunk
  const int lane = threadIdx.x & (kWave - 1);
  // Wave-uniform by construction; readfirstlane lets the compiler keep the
  // chunk walk (and its block-table reads) in scalar registers, so a table
  // read never waits behind the vector loads already in flight.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int row = lane >> 4;   // which of the 4 tokens of a load
  const int col = lane & 15;   // which 16-byte column of the head row
  int b = bz, g = by, blk0 = 0;
  if (a.length_order) length_ordered_item(a, by, bz, b, g, blk0);
  const int pi = bx;
  const int hq = a.num_kv_heads * G;

  const int64_t tok_stride = static_cast<int64_t>(a.num_kv_heads) * 16;  // uint4 per slot
  const int64_t blk_stride = tok_stride * a.block_size;
  const uint4* kbase = static_cast<const uint4*>(a.k_cache) + g * 16 + col + row * tok_stride;
  const uint4* vbase = static_cast<const uint4*>(a.v_cache) + g * 16 + col + row * tok_stride;
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;

  // Without a window, partition pi starts at pi * partition_size whatever the
  // sequence length, so the first chunk's table read and K/V loads are issued
  // together with the context-length read instead of after it (one memory
  // round trip less before the first bytes arrive).  They are wasted if the
  // partition turns out to be empty.
  const bool spec = a.sliding_window == 0;
  ChunkRegs<NL> ca, cb;
  if (spec) {
    const int base0 = pi * a.partition_size + wave * CT;
    // With the ranked order the table entry of block 0 came with the ranking
    // (one round trip less before the first K/V loads).
    if (a.length_order && base0 < a.block_size)
      load_chunk_at<NL>(ca, a, blk0, 0, false, kbase, vbase, tok_stride, blk_stride, base0);
    else
      load_chunk<NL>(ca, a, bt, kbase, vbase, tok_stride, blk_stride, base0);
  }

  const SeqRange r = seq_range(a, b);
  if (r.row < 0) return;
  uint16_t* out = static_cast<uint16_t*>(a.out) + (static_cast<int64_t>(r.row) * hq + g * G) * kHeadDim;

  // Fused store: the new token sits at position L-1 of the sequence's own
  // length, whatever the clamp to max_context_len (or to the table) left for
  // attention.  It is written to that position's slot when the table has an
  // entry for it (as a store through slot_mapping would), and it replaces the
  // cached row only if attention admits that position (last < r.L).
  const int last = FUSE ? seq_len(a, b) - 1 : -1;
  uint4 kn = make_uint4(0, 0, 0, 0), vn = make_uint4(0, 0, 0, 0);
  if (FUSE) {
    const int64_t off = (static_cast<int64_t>(b) * a.num_kv_heads + g) * 16 + col;
    kn = static_cast<const uint4*>(a.k_new)[off];
    vn = static_cast<const uint4*>(a.v_new)[off];
  }
  // Head g's 256 bytes of the new K/V into the slot of position `last`.
  // Stores share the in-order vector-memory counter with loads, so a store
  // inside the streaming loop would make every later wait also wait for its
  // write to be acknowledged; it is issued after the loop, where no load
  // follows.
  auto store_new = [&]() {
    if (last < 0 || last / a.block_size >= a.max_blocks_per_seq) return;
    const int lb = last / a.block_size;
    const int blk = bt[lb];
    if (static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks)) {
      const int64_t off = static_cast<int64_t>(blk) * blk_stride +
                          static_cast<int64_t>(last - lb * a.block_size) * tok_stride;
      const_cast<uint4*>(kbase)[off] = kn;
      const_cast<uint4*>(vbase)[off] = vn;
    }
  };
  // The partition that stores (the one holding position L-1 when attention
  // admits it, else the first; wavefront 0, the first row of lanes).
  const bool storer = FUSE && wave == 0 && row == 0 &&
                      pi == (last < r.L ? r.nparts - 1 : 0);

  if (r.nparts == 0) {
    if (pi == 0)
      for (int o = threadIdx.x; o < G * kHeadDim; o += NW * kWave) out[o] = 0;
    if (storer) store_new();
    return;
  }
  if (pi >= r.nparts) return;
  const int t0 = r.lo + pi * a.partition_size;
  const int t1 = t0 + min(a.partition_size, r.L - t0);

#if PK_DECODE_DOT2
  // q kept as packed bf16 pairs; the scale is applied to the reduced score.
  uint4 qp[G];
  {
    const uint4* qv = static_cast<const uint4*>(a.q) + (static_cast<int64_t>(r.row) * hq + g * G) * 16 + col;
#pragma unroll
    for (int h = 0; h < G; ++h) qp[h] = qv[h * 16];
  }
#else
  float qf[G][8];
  {
    const uint4* qv = static_cast<const uint4*>(a.q) + (static_cast<int64_t>(r.row) * hq + g * G) * 16 + col;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      unpack8(qv[h * 16], qf[h]);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[h][e] *= a.scale_log2;
    }
  }
#endif

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kEmptyMax;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  // Consume one chunk held in registers (scores, online softmax, P.V).
  auto consume = [&](ChunkRegs<NL>& c, int base) {
    if (FUSE && last < r.L && static_cast<unsigned>(last - base) < static_cast<unsigned>(CT)) {
      // The chunk holding the new token (a wave-uniform test): its lanes take
      // the new K/V in place of what the cache holds at that position (the
      // slot itself is written after the streaming loop).
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        if (base + 4 * k + row == last) {
          c.k[k] = kn;
          c.v[k] = vn;
        }
      }
    }
    float s[NL][G];
    bool valid[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int t = base + 4 * k + row;
      valid[k] = c.ok && t >= t0 && t < t1;
#if PK_DECODE_DOT2
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = dot2_bf16(c.k[k].x, qp[h].x, 0.f);
        x = dot2_bf16(c.k[k].y, qp[h].y, x);
        x = dot2_bf16(c.k[k].z, qp[h].z, x);
        x = dot2_bf16(c.k[k].w, qp[h].w, x);
        x = row16_sum(x) * a.scale_log2;
        s[k][h] = valid[k] ? x : -INFINITY;
      }
#else
      float kf[8];
      unpack8(c.k[k], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) x = fmaf(qf[h][e], kf[e], x);
        x = row16_sum(x);
        s[k][h] = valid[k] ? x : -INFINITY;
      }
#endif
    }
    float pw[NL][G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[0][h];
#pragma unroll
      for (int k = 1; k < NL; ++k) cm = fmaxf(cm, s[k][h]);
      const float mn = fmaxf(m[h], cm);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      float sum = 0.f;
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        pw[k][h] = fast_exp2(s[k][h] - mn);
        sum += pw[k][h];
      }
      l[h] = fmaf(l[h], alpha, sum);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      // Masked tokens get weight 0; their V words are zeroed too so that
      // stale cache contents (possibly NaN patterns) cannot leak in.
      const uint4 vw = valid[k] ? c.v[k] : make_uint4(0, 0, 0, 0);
      float vf[8];
      unpack8(vw, vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw[k][h], vf[e], acc[h][e]);
    }
  };

  // Two register buffers in ping-pong: the loads of the next chunk are in
  // flight while the current one is consumed, with no register copies.  The
  // prefetch is unconditional (past the end it loads the shared dummy chunk):
  // a conditional load would make the wait counters assume the worst case at
  // the merge and stall on the prefetch itself.
  const int step = NW * CT;
  int b0 = (t0 / CT) * CT + wave * CT;   // == the speculative chunk when spec
  if (b0 < t1) {
    if (!spec) load_chunk<NL>(ca, a, bt, kbase, vbase, tok_stride, blk_stride, b0);
    while (true) {
      const int b1 = b0 + step;
      load_chunk<NL>(cb, a, bt, kbase, vbase, tok_stride, blk_stride, b1 < t1 ? b1 : -1);
      consume(ca, b0);
      if (b1 >= t1) break;
      const int b2 = b1 + step;
      load_chunk<NL>(ca, a, bt, kbase, vbase, tok_stride, blk_stride, b2 < t1 ? b2 : -1);
      consume(cb, b1);
      if (b2 >= t1) break;
      b0 = b2;
    }
  }

  // Once wavefront 0 has streamed its chunks; the merge below hides it.
  if (storer) store_new();
  // Merge the 4 rows of the wavefront (lanes l, l^16, l^32, l^48 share a column).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = fmaxf(m[h], shfl_xor(m[h], 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float f = fast_exp2(m[h] - mx);
    float lh = l[h] * f;
    lh += shfl_xor(lh, 16);
    lh += shfl_xor(lh, 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e] * f;
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      acc[h][e] = x;
    }
    m[h] = mx;
    l[h] = lh;
  }

  // Merge the wavefronts through LDS; one thread per (head, dim) output.
  __shared__ float s_acc[NW][G][kHeadDim];
  __shared__ float s_m[NW][G];
  __shared__ float s_l[NW][G];
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_acc[wave][h][col * 8 + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < G * kHeadDim; o += NW * kWave) {
    const int h = o / kHeadDim;
    const int d = o % kHeadDim;
    float mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, s_m[w][h]);
    float ls = 0.f, av = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = fast_exp2(s_m[w][h] - mx);
      ls = fmaf(s_l[w][h], f, ls);
      av = fmaf(s_acc[w][h][d], f, av);
    }
    if (r.nparts == 1) {
      out[o] = static_cast<uint16_t>(f32_to_bf16_bits(ls > 0.f ? av / ls : 0.f));
    } else {
      const int64_t slot = (static_cast<int64_t>(b) * hq + g * G + h) * a.num_parts + pi;
      if constexpr (MERGE) {
        // Device-coherent stores: the merging workgroup may run on another XCD,
        // whose L2 does not see this one's.
        __hip_atomic_store(a.ws_acc + slot * kHeadDim + d, av, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == 0) {
          __hip_atomic_store(a.ws_ml + slot * 2, mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(a.ws_ml + slot * 2 + 1, ls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        a.ws_acc[slot * kHeadDim + d] = av;
        if (d == 0) {
          a.ws_ml[slot * 2] = mx;
          a.ws_ml[slot * 2 + 1] = ls;
        }
      }
    }
  }
  if constexpr (MERGE) {
    if (r.nparts > 1) {
      // Once this workgroup's partial stores are complete (every wavefront
      // waits for its own, then the barrier), one arrival on the pair's
      // counter.  The partition that brings it to nparts merges all of them
      // and sets the counter back to zero; the others are done.  No workgroup
      // waits for another.  Device-coherent stores completed before the
      // arrival and device-coherent loads after it make the partials visible
      // without cache write-backs or invalidations.
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wavefront's stores acknowledged
      __syncthreads();
      __shared__ int s_merge;
      if (threadIdx.x == 0) {
        int32_t* t = a.merge_counters + static_cast<int64_t>(b) * a.num_kv_heads + g;
        const int arrived = __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = arrived == r.nparts - 1;
        if (last) __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_merge = last;
      }
      __syncthreads();
      if (!s_merge) return;
      for (int o = threadIdx.x; o < G * kHeadDim; o += NW * kWave) {
        const int64_t head = static_cast<int64_t>(b) * hq + g * G + o / kHeadDim;
        out[o] = static_cast<uint16_t>(f32_to_bf16_bits(merge_partials<true>(a, head, o % kHeadDim, r.nparts)));
      }
    }
  }
}

template <int G, int NW, int NL, bool FUSE>
__global__ void __launch_bounds__(NW * kWave)
decode_partition_kernel(DecodeArgs a) {
  decode_partition_body<G, NW, NL, FUSE>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// Split plans with the merge in the same launch: a 1D grid, partition fastest,
// then KV head, then sequence (the decode kernel's grid order, flattened).
template <int G, int NW, int NL, bool FUSE>
__global__ void __launch_bounds__(NW * kWave)
decode_partition_merged_kernel(DecodeArgs a) {
  const int w = static_cast<int>(blockIdx.x);
  const int pi = w % a.num_parts;
  const int pair = w / a.num_parts;
  decode_partition_body<G, NW, NL, FUSE, true>(a, pi, pair % a.num_kv_heads, pair / a.num_kv_heads);
}

// Merge the partitions of every sequence that has more than one (split plans
// without merge counters).
template <int G>
__global__ void __launch_bounds__(G * kHeadDim)
decode_combine_kernel(DecodeArgs a) {
  const int g = blockIdx.x;
  const int b = blockIdx.y;
  const SeqRange r = seq_range(a, b);
  if (r.nparts <= 1 || r.row < 0) return;   // written directly by the partition kernel
  const int hq = a.num_kv_heads * G;
  const int h = threadIdx.x / kHeadDim;
  const int d = threadIdx.x % kHeadDim;
  const int64_t head = static_cast<int64_t>(b) * hq + g * G + h;
  static_cast<uint16_t*>(a.out)[(static_cast<int64_t>(r.row) * hq + g * G + h) * kHeadDim + d] =
      static_cast<uint16_t>(f32_to_bf16_bits(merge_partials<false>(a, head, d, r.nparts)));
}

constexpr int kDecodeWaves = PK_DECODE_WAVES;
constexpr int kDecodeLoads = PK_DECODE_LOADS;

}  // namespace
}  // namespace pk
