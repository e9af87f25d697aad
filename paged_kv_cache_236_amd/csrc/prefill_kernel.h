// paged_prefill: variable-length causal attention for the new tokens of
// sequences whose prefix may already sit in the paged cache (prefix caching,
// nano-vllm-sansho README "Key Features"; prefill as its own phase, lunaryes/
// nano-vllm introduction).  New query i of sequence b is at position P_b + i
// (P_b = Lk_b - Lq_b cached tokens) and attends keys j <= P_b + i, and
// P_b + i - j < W with a sliding window W.
//
// This is a dense contraction, so it runs on the bf16 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Workgroup = (sequence b, KV head g, query tile t) with 4 wavefronts.  The
// workgroup's 128 "query columns" are the G query heads of KV head g times
// BM = 128 / G query rows, so each K/V tile read from HBM serves every head of
// the group.  Each wavefront owns 32 columns.
//
// Formulation.  Per 32-key tile the wavefront computes S^T = K . Q^T (keys x
// its 32 columns; A = K rows from LDS, B = Q^T held in registers for the whole
// kernel) and then O^T += V^T . P^T (head dims x columns).  In the 32x32 MFMA
// output layout a lane holds one column and 16 key rows, which are exactly the
// key slots the lane must supply as the B operand of the PV product, so the
// probabilities never leave registers; the online-softmax state (m, l) is per
// lane.  K and V sit in LDS in their natural row layout (one 256-byte row per
// key); the V^T operand is read with the transposing LDS read
// (ds_read_b64_tr_b16), which hands each lane four keys of one head dim.
// 16-byte chunks are XOR-swizzled within a row so that every operand read is
// bank-conflict free.
//
// Data movement.  K/V tiles (32 keys) go from HBM straight into LDS with the
// 16-byte global-to-LDS DMA loads (global_load_lds_dwordx4): no registers are
// spent on staging, and a ring of four LDS stages keeps three tiles in flight
// while one is consumed.  Each lane picks the global 16-byte chunk that the
// swizzle places at its LDS position.  The DMA is issued as inline assembly,
// so the compiler does not see it and does not drain every pending DMA before
// each (compiler-visible) operand read; the waits for the ring are explicit
// (s_waitcnt vmcnt for the wave's own DMAs, then a barrier for everyone's).
// Nothing else in the loop touches LDS: block-table entries are read with
// scalar loads (a 32-key tile spans at most two blocks) and the half-wave
// exchange uses v_permlane32_swap.
//
// Fused store (FUSE): the new tokens' K/V arrive as separate arrays; tiles
// read keys at positions >= P_b from those arrays instead of the cache, and
// each workgroup writes the rows of its own query positions into their cache
// slots at the end.  Key validity (a bad block-table entry) is decided from
// the table exactly as without fusion, so the result and the cache equal a
// store followed by the plain kernel, bit for bit.
//
// Softmax.  Scores are scaled inside the exp argument (one FMA per score), the
// bf16 probabilities are packed by the hardware converter, and the running max
// is only raised when a tile's max exceeds it by more than 2^8, so most tiles
// skip rescaling O (probabilities stay <= 256, far inside fp32 and bf16 range).
//
// Work order: heaviest items first.  With at most 128 (sequence, query tile)
// items every workgroup ranks them by their number of key tiles (cached prefix
// included) and takes the one of its rank, so the long chains start at once
// and a sequence's query tiles run together, sharing its K/V in L2.  With more
// items, latest query tiles (most keys of their sequence) first; then with
// num_seqs * num_kv_heads a multiple of 8 all tiles of one (b, g) pair land on
// the same XCD (workgroups are dealt round-robin over the 8 XCDs) and share
// its L2.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBN = 32;                   // keys per tile
constexpr int kCols = 128;                // query columns (head x row) per workgroup
constexpr int kThreads = 256;             // 4 wavefronts x 32 columns
constexpr int kRow = 256;                 // bytes of one K or V row (128 bf16)
constexpr int kTile = kBN * kRow;         // bytes of one K or V tile (8 KiB)
constexpr int kStages = 4;                // LDS ring depth (tiles in flight + 1)
constexpr int kDmaPerTile = 4;            // DMA instructions per wave per tile (2 K + 2 V)
constexpr float kRescaleSlack = 8.0f;     // log2 units the running max may lag

// The ring: one array per stage for K and for V.  Separate arrays let the
// compiler tell that a read of one stage does not alias a global-to-LDS load
// into another, so it places the operand reads' waits itself and inserts no
// wait for the loads in flight into other stages.
__shared__ __attribute__((aligned(1024))) char s_k0[kTile], s_k1[kTile], s_k2[kTile], s_k3[kTile];
__shared__ __attribute__((aligned(1024))) char s_v0[kTile], s_v1[kTile], s_v2[kTile], s_v3[kTile];

template <int ST>
__device__ __forceinline__ char* k_stage() {
  static_assert(ST >= 0 && ST < kStages, "ring stage");
  return ST == 0 ? s_k0 : ST == 1 ? s_k1 : ST == 2 ? s_k2 : s_k3;
}
template <int ST>
__device__ __forceinline__ char* v_stage() {
  static_assert(ST >= 0 && ST < kStages, "ring stage");
  return ST == 0 ? s_v0 : ST == 1 ? s_v1 : ST == 2 ? s_v2 : s_v3;
}


// Position of 16-byte chunk c (0..15) of key row r in LDS.
//  K: c ^ (r % 16): the A operand of S^T reads one chunk of rows 0..15 per 16 lanes.
//  V: c ^ 4 (r % 4): a transposed read covers 4 consecutive rows x 4 chunks per 32 lanes.
__device__ __forceinline__ int k_pos(int r, int c) { return c ^ (r & 15); }
__device__ __forceinline__ int v_pos(int r, int c) { return c ^ ((r & 3) << 2); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8), issued through the builtin so that the compiler's
// own wait insertion knows which loads they already cover.
constexpr int waitcnt_vm(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }
constexpr int waitcnt_lgkm(int n) { return 0xf | (0x3 << 14) | (0x7 << 4) | ((n & 0xf) << 8); }

// Combine lane l with lane l ^ 32 (v_permlane32_swap hands each lane both
// values of the pair, in an order that differs between the halves, so only
// symmetric combinations are taken).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One block-table entry through the scalar cache.  Written out because with
// LDS DMA in the loop the compiler can no longer prove the table unmodified and
// would use a vector load, whose use waits for every pending DMA as well.  The
// table is only read during the kernel.
__device__ __forceinline__ int32_t table_entry(const int32_t* row, int idx) {
  int32_t v;
  // The address is wave-uniform; both halves go through readfirstlane so it
  // sits in scalar registers whatever the compiler's uniformity analysis
  // concluded (each half widened as unsigned: no sign extension).
  const uint64_t pv = reinterpret_cast<uint64_t>(row + idx);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(pv))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(pv >> 32))));
  const int32_t* p = reinterpret_cast<const int32_t*>((static_cast<uint64_t>(hi) << 32) | lo);
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
  return v;
}

// The (at most two) cache blocks holding keys kb .. kb+31 of the sequence,
// worked out once per tile in scalar registers.
struct TileMap {
  int startA, startB;     // first key of each block
  int endA;               // first key past block A
  int64_t baseA, baseB;   // byte offset of each block's row 0, KV head g (slot 0 if bad)
  bool okA, okB;          // the entries are inside the table and the cache
};

// How the kernel finds a key's cache block.
constexpr int kDivBlocks = 0;    // any block size: index by division, a tile may span two blocks
constexpr int kShiftBlocks = 1;  // power of two below a tile: index by shift, up to two blocks
constexpr int kTileInBlock = 2;  // power of two >= a tile: every tile lies inside one block

template <bool POW2>
__device__ __forceinline__ int div_block(const PrefillArgs& a, int x) {
  return POW2 ? (x >> a.block_shift) : x / a.block_size;
}

template <bool POW2>
__device__ __forceinline__ TileMap tile_map(const PrefillArgs& a, const int32_t* bt, int kb, int g,
                                            int64_t slot_bytes) {
  TileMap m;
  const int lbA = div_block<POW2>(a, kb);
  const int lbB = div_block<POW2>(a, kb + kBN - 1);
  m.startA = lbA * a.block_size;
  m.startB = lbB * a.block_size;
  m.endA = m.startA + a.block_size;
  const int blkA = table_entry(bt, min(lbA, a.max_blocks_per_seq - 1));
  const int blkB = lbB == lbA ? blkA : table_entry(bt, min(lbB, a.max_blocks_per_seq - 1));
  m.okA = lbA < a.max_blocks_per_seq && static_cast<unsigned>(blkA) < static_cast<unsigned>(a.num_blocks);
  m.okB = lbB < a.max_blocks_per_seq && static_cast<unsigned>(blkB) < static_cast<unsigned>(a.num_blocks);
  const int64_t head = static_cast<int64_t>(g) * kRow;
  m.baseA = (m.okA ? static_cast<int64_t>(blkA) * a.block_size * slot_bytes : 0) + head;
  m.baseB = (m.okB ? static_cast<int64_t>(blkB) * a.block_size * slot_bytes : 0) + head;
  return m;
}

// 32-bit mask of the keys kb .. kb+31 that exist and have a valid block.
__device__ __forceinline__ uint32_t valid_mask(const TileMap& m, int kb, int Lk) {
  const int n = min(max(Lk - kb, 0), kBN);                 // keys before the end
  const int na = min(max(m.endA - kb, 0), kBN);            // keys in block A
  const uint32_t upto_n = n >= kBN ? 0xffffffffu : (1u << n) - 1u;
  const uint32_t in_a = na >= kBN ? 0xffffffffu : (1u << na) - 1u;
  return upto_n & ((m.okA ? in_a : 0u) | (m.okB ? ~in_a : 0u));
}

// 16-byte global-to-LDS loads (global_load_lds_dwordx4): each lane's 16
// bytes land at M0 + 16 * lane.  Issued as assembly on purpose: the compiler
// then does not know that these instructions write LDS, so it inserts no wait
// for them before the kernel's (compiler-visible) LDS operand reads; the
// kernel orders them itself (its own wait for its loads, then a barrier).
// Compiler-generated waits for its own memory loads stay correct: loads
// complete in order, so unseen older loads only make those waits stricter.
// `base` is wave-uniform (scalar base + 32-bit lane offset form).
__device__ __forceinline__ void dma16_saddr(const char* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}
// A wave-uniform pointer as a scalar value (both 32-bit halves read from the
// first lane; each half widened as unsigned so the low word is not sign
// extended).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(v >> 32))));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}
// Per-lane 64-bit address form.
__device__ __forceinline__ void dma16_vaddr(const char* addr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               ::"v"(addr), "s"(lds) : "memory", "m0");
}

// Zero 16 bytes of LDS.  Written out so the compiler does not wait for the
// pending global-to-LDS loads (it cannot tell which bytes they write).
__device__ __forceinline__ void zero_lds16(char* p) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  asm volatile("ds_write_b128 %0, %1" ::"v"(lds_addr(p)), "v"(z) : "memory");
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));

// One transposing LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i supplies the address of key (base + i/4), dims 4*(i%4)..+3,
// and receives dim i of the four keys.
__device__ __forceinline__ u32x2_t read_tr16(const char* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(u32x2_t, v);
}

// Work order by true work.  A query tile's cost is its number of 32-key tiles,
// which depends on its sequence's cached prefix as well as on its index, so
// "latest query tile first" can leave heavy tiles of long-prefix sequences to
// the end.  Instead every workgroup ranks all (sequence, query tile) items by
// key-tile count (most first, counts above 63 alike; ties by item index; empty
// items last) and takes the item of rank bx / num_kv_heads, KV head
// bx % num_kv_heads: longest processing time first.  Up to 128 items, two per
// lane: a ballot radix select over the 6 count bits finds the count, then a
// prefix count of the remaining candidates finds the item; the candidate sets
// are wave-wide masks, so the select runs on the scalar unit, and item k
// splits into (sequence, tile) with a multiply by the host's reciprocal of the
// tile count.  The lengths and first block-table entry of every item's
// sequence are loaded in one round trip, and the chosen item's come from the
// lane that loaded them.
template <int BM>
__device__ __forceinline__ void ranked_item(const PrefillArgs& a, int ntiles, int rank, int& b,
                                            int& t, int& q0, int& q1, int& k0, int& k1,
                                            int& blk0) {
  static_assert(kPrefillRankMax == 2 * kWave, "two items per lane");
  const int lane = threadIdx.x & (kWave - 1);
  const int S = a.num_seqs * ntiles;
  // Item k = lane + 64 j is query tile k % ntiles of sequence k / ntiles.
  auto seq_of = [&](int k) __attribute__((always_inline)) {
    return ntiles > 1 ? static_cast<int>(__umulhi(static_cast<uint32_t>(k), a.tiles_recip)) : k;
  };
  int vq0[2], vq1[2], vk0[2], vk1[2], vbt[2];
  uint32_t cnt[2];
  uint64_t cand[2];   // candidate items, one bit per lane
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int bb = seq_of(min(lane + kWave * j, S - 1));
    vq0[j] = a.cu_seqlens_q[bb];
    vq1[j] = a.cu_seqlens_q[bb + 1];
    vk0[j] = a.cu_seqlens_k[bb];
    vk1[j] = a.cu_seqlens_k[bb + 1];
    vbt[j] = a.block_tables[static_cast<int64_t>(bb) * a.max_blocks_per_seq];
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int k = lane + kWave * j;
    const int tt = k - seq_of(k) * ntiles;
    const int Lq = vq1[j] - vq0[j], Lk = vk1[j] - vk0[j], P = Lk - Lq, qa = tt * BM;
    int n = 0;
    if (!(Lq <= 0 || P < 0 || qa >= Lq || vq0[j] < 0 || vq0[j] + Lq > a.total_q)) {
      const int pos_lo = P + qa, pos_hi = P + min(qa + BM, Lq) - 1;
      const int kstart = a.sliding_window > 0 ? max(0, pos_lo - a.sliding_window + 1) : 0;
      n = pos_hi / kBN - kstart / kBN + 1;
    }
    cnt[j] = static_cast<uint32_t>(min(n, 63));
    cand[j] = __ballot(k < S);
  }
  // The count bucket holding rank `rank`, from the top bit down: among the
  // remaining candidates those with the bit set rank above those without.
  // The candidate sets are wave-wide masks, so this runs on the scalar unit.
  int need = rank;
#pragma unroll
  for (int bit = 5; bit >= 0; --bit) {
    const uint64_t ones0 = __ballot((cnt[0] >> bit) & 1u) & cand[0];
    const uint64_t ones1 = __ballot((cnt[1] >> bit) & 1u) & cand[1];
    const int c = __builtin_popcountll(ones0) + __builtin_popcountll(ones1);
    const bool in_ones = need < c;
    cand[0] = in_ones ? ones0 : cand[0] & ~ones0;
    cand[1] = in_ones ? ones1 : cand[1] & ~ones1;
    need = in_ones ? need : need - c;
  }
  // Within the bucket, items in index order (k = lane + 64 j): the `need`-th
  // remaining candidate, found by each candidate's count of candidates below it.
  const int c0 = __builtin_popcountll(cand[0]);
  const int j = need < c0 ? 0 : 1;
  const uint64_t m = j == 0 ? cand[0] : cand[1];
  need = j == 0 ? need : need - c0;
  const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
  const bool mine = ((m >> lane) & 1u) && below == need;
  const uint64_t hit = __ballot(mine);   // one lane: the rank is below the item count
  const int src = hit ? static_cast<int>(__builtin_ctzll(hit)) : 0;
  const int k = src + kWave * j;
  b = seq_of(k);
  t = k - b * ntiles;
  q0 = __builtin_amdgcn_readlane(j == 0 ? vq0[0] : vq0[1], src);
  q1 = __builtin_amdgcn_readlane(j == 0 ? vq1[0] : vq1[1], src);
  k0 = __builtin_amdgcn_readlane(j == 0 ? vk0[0] : vk0[1], src);
  k1 = __builtin_amdgcn_readlane(j == 0 ? vk1[0] : vk1[1], src);
  blk0 = __builtin_amdgcn_readlane(j == 0 ? vbt[0] : vbt[1], src);
}

// POS: the softmax scale is positive, so the max of the raw scores gives the
// max of the scaled ones and each probability is exp2(fma(s, c, -m)).
// MODE: block addressing (kDivBlocks, kShiftBlocks or kTileInBlock).
// FUSE: store the new tokens (a.k_new / a.v_new) and read them from there.
template <int G, bool POS, int MODE, bool FUSE>
__device__ __forceinline__ void paged_prefill_body(const PrefillArgs& a, int bx) {
  constexpr int BM = kCols / G;   // query rows per workgroup
  constexpr bool POW2 = MODE != kDivBlocks;
  constexpr bool ONE = MODE == kTileInBlock;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hgrp = lane >> 5;   // which 8-element k group of the MFMA operands
  const int c32 = lane & 31;
  const int i16 = lane & 15;
  const int half = (lane >> 4) & 1;   // which 16 rows of a 32-row MFMA A operand
  const int hq = a.num_kv_heads * G;
  const float c = a.scale_log2;

  // ---- work item: most key tiles first, or latest query tiles first --------
  const int npairs = a.num_seqs * a.num_kv_heads;
  const int ntiles = (a.max_seqlen_q + BM - 1) / BM;
  int t, b, g, q0, q1, k0, k1, blk_first;
  if (a.lpt_order) {
    // rank bx / Hkv, KV head bx % Hkv (shifts for a power-of-two Hkv)
    const int hkv = a.num_kv_heads;
    const bool pow2 = (hkv & (hkv - 1)) == 0;
    const int rank = pow2 ? bx >> __builtin_ctz(hkv) : bx / hkv;
    g = pow2 ? bx & (hkv - 1) : bx - rank * hkv;
    ranked_item<BM>(a, ntiles, rank, b, t, q0, q1, k0, k1, blk_first);
  } else {
    t = ntiles - 1 - bx / npairs;
    const int pr = bx % npairs;
    b = pr / a.num_kv_heads;
    g = pr % a.num_kv_heads;
    // The sequence's lengths and its first block-table entry, fetched in one
    // memory round trip: the empty asm needs all five values at once, so the
    // compiler issues the five loads before a single wait (left alone it
    // waits after each).  Without a window the first tile lies in block 0, so
    // its DMAs need no further table lookup (the entry is judged like any
    // other).
    q0 = a.cu_seqlens_q[b];
    q1 = a.cu_seqlens_q[b + 1];
    k0 = a.cu_seqlens_k[b];
    k1 = a.cu_seqlens_k[b + 1];
    blk_first = a.block_tables[static_cast<int64_t>(b) * a.max_blocks_per_seq];
  }
  const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;
  q0 = __builtin_amdgcn_readfirstlane(q0);
  q1 = __builtin_amdgcn_readfirstlane(q1);
  k0 = __builtin_amdgcn_readfirstlane(k0);
  k1 = __builtin_amdgcn_readfirstlane(k1);
  blk_first = __builtin_amdgcn_readfirstlane(blk_first);
  asm volatile("" : "+s"(q0), "+s"(q1), "+s"(k0), "+s"(k1), "+s"(blk_first));
  const int Lq = q1 - q0;
  const int Lk = k1 - k0;
  const int P = Lk - Lq;
  const int qa = t * BM;
  if (Lq <= 0 || P < 0 || qa >= Lq || q0 < 0 || q0 + Lq > a.total_q) return;
  const int qb = min(qa + BM, Lq);
  const int W = a.sliding_window;
  const int pos_lo = P + qa, pos_hi = P + qb - 1;
  const int kstart = W > 0 ? max(0, pos_lo - W + 1) : 0;
  const int tile0 = kstart / kBN, tile1 = pos_hi / kBN;
  const char* kcache = static_cast<const char*>(a.k_cache);
  const char* vcache = static_cast<const char*>(a.v_cache);
  const int64_t slot_bytes = static_cast<int64_t>(a.num_kv_heads) * kRow;
  // New key j >= P lives in row q0 + j - P of the new-token arrays (the same
  // row stride as the cache), KV head g.
  const int64_t new_base = (static_cast<int64_t>(q0) - P) * slot_bytes + static_cast<int64_t>(g) * kRow;
  const char* knew = FUSE ? static_cast<const char*>(a.k_new) + new_base : nullptr;
  const char* vnew = FUSE ? static_cast<const char*>(a.v_new) + new_base : nullptr;

  // This lane's two DMA rows of a tile (4 rows per DMA instruction, 2 per wave
  // for K and 2 for V) and the chunks it fetches for them.
  int dma_row[2], dma_kchunk[2], dma_vchunk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    dma_row[j] = 8 * wave + 4 * j + (lane >> 4);
    dma_kchunk[j] = k_pos(dma_row[j], i16) * 16;
    dma_vchunk[j] = v_pos(dma_row[j], i16) * 16;
  }
  // Tile-relative byte offsets of those chunks when the tile lies in one block.
  uint32_t dma_koff[2], dma_voff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    dma_koff[j] = static_cast<uint32_t>(dma_row[j] * slot_bytes + dma_kchunk[j]);
    dma_voff[j] = static_cast<uint32_t>(dma_row[j] * slot_bytes + dma_vchunk[j]);
  }
  // Last block looked up (tiles inside one block): its logical index, byte
  // offset of row 0 for KV head g, and whether the entry is valid.
  int cur_lb = -1;
  int64_t cur_base = 0;
  bool cur_ok = false;
  if constexpr (ONE) {
    cur_lb = 0;
    cur_ok = static_cast<unsigned>(blk_first) < static_cast<unsigned>(a.num_blocks);
    cur_base = (cur_ok ? static_cast<int64_t>(blk_first) * a.block_size * slot_bytes : 0) +
               static_cast<int64_t>(g) * kRow;
  }

  // ---- DMA of one tile into ring stage ST (this wave's 8 K rows and 8 V rows)
  // Returns whether some row of the tile has a bad block entry (for a tile in
  // one block: the whole tile, same answer in every wave; otherwise: one of
  // this wave's rows).  Rows of a bad block read slot 0 of the cache instead.
  // Spanning tiles read the sequence's last key for keys past its end; a tile
  // inside one block reads the block's rows past the end (in bounds), and
  // those V rows are zeroed in LDS before use.
  auto issue_tile = [&](int kt, auto st) -> bool {
    constexpr int ST = decltype(st)::value;
    const int kb = kt * kBN;
    if constexpr (ONE) {
      const int lb = kb >> a.block_shift;
      if (lb != cur_lb) {
        const int blk = table_entry(bt, min(lb, a.max_blocks_per_seq - 1));
        cur_ok = lb < a.max_blocks_per_seq && static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks);
        cur_base = (cur_ok ? static_cast<int64_t>(blk) * a.block_size * slot_bytes : 0) +
                   static_cast<int64_t>(g) * kRow;
        cur_lb = lb;
      }
      // (kb mod block_size) * slot_bytes < 2^31: the host picks this mode only then
      const int64_t tb = cur_base + static_cast<uint32_t>((kb & (a.block_size - 1)) *
                                                          static_cast<uint32_t>(slot_bytes));
      if (FUSE && kb >= P && kb + kBN <= Lk) {
        // All 32 keys new: consecutive rows of the new-token arrays, with the
        // cache's row stride, so the same lane offsets apply.
        const char* ks = uniform_ptr(knew + static_cast<int64_t>(kb) * slot_bytes);
        const char* vs = uniform_ptr(vnew + static_cast<int64_t>(kb) * slot_bytes);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          dma16_saddr(ks, dma_koff[j], lds_addr(&k_stage<ST>()[(8 * wave + 4 * j) * kRow]));
          dma16_saddr(vs, dma_voff[j], lds_addr(&v_stage<ST>()[(8 * wave + 4 * j) * kRow]));
        }
        return !cur_ok;
      }
      if (FUSE && kb + kBN > P) {
        // Keys >= P from the new-token arrays (past the end: the last key),
        // earlier ones from the cache block.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int key = min(kb + dma_row[j], Lk - 1);
          const int64_t crow = tb + static_cast<int64_t>(dma_row[j]) * slot_bytes;
          const char* ks = key >= P ? knew + static_cast<int64_t>(key) * slot_bytes : kcache + crow;
          const char* vs = key >= P ? vnew + static_cast<int64_t>(key) * slot_bytes : vcache + crow;
          dma16_vaddr(ks + dma_kchunk[j], lds_addr(&k_stage<ST>()[(8 * wave + 4 * j) * kRow]));
          dma16_vaddr(vs + dma_vchunk[j], lds_addr(&v_stage<ST>()[(8 * wave + 4 * j) * kRow]));
        }
        return !cur_ok;
      }
      const char* ksrc = uniform_ptr(kcache + tb);
      const char* vsrc = uniform_ptr(vcache + tb);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        dma16_saddr(ksrc, dma_koff[j], lds_addr(&k_stage<ST>()[(8 * wave + 4 * j) * kRow]));
        dma16_saddr(vsrc, dma_voff[j], lds_addr(&v_stage<ST>()[(8 * wave + 4 * j) * kRow]));
      }
      return !cur_ok;
    } else {
      const TileMap m = tile_map<POW2>(a, bt, kb, g, slot_bytes);
      bool any_bad = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int key = kb + dma_row[j];
        const int kk = min(key, Lk - 1);
        const bool inA = kk < m.endA;
        any_bad |= !(inA ? m.okA : m.okB) && key < Lk;
        const int64_t row = (inA ? m.baseA : m.baseB) +
                            static_cast<int64_t>(kk - (inA ? m.startA : m.startB)) * slot_bytes;
        const bool fresh = FUSE && kk >= P;
        const char* ks = fresh ? knew + static_cast<int64_t>(kk) * slot_bytes : kcache + row;
        const char* vs = fresh ? vnew + static_cast<int64_t>(kk) * slot_bytes : vcache + row;
        dma16_vaddr(ks + dma_kchunk[j], lds_addr(&k_stage<ST>()[(8 * wave + 4 * j) * kRow]));
        dma16_vaddr(vs + dma_vchunk[j], lds_addr(&v_stage<ST>()[(8 * wave + 4 * j) * kRow]));
      }
      return __ballot(any_bad) != 0;
    }
  };

  // ---- this lane's query column -------------------------------------------
  const int col = wave * 32 + c32;
  const int hl = col / BM;
  const int qi = qa + col % BM;
  const bool qvalid = qi < Lq;
  const int qpos = P + qi;
  const int head = g * G + hl;
  // positions spanned by this wavefront's columns (for skipping masked tiles)
  const int wq_lo = qa + (wave * 32) % BM;
  const int wq_hi = min(wq_lo + min(32, BM) - 1, Lq - 1);
  const int wpos_lo = P + wq_lo, wpos_hi = P + wq_hi;
  // Per-wavefront tile thresholds (keys kb .. kb+31 of tile kt = kb/32):
  //  active:    some key is admitted for some row: act_lo <= kt <= act_hi
  //             (a wavefront without valid rows has act_hi = -1);
  //  need_mask: some key lies past the earliest row (kt >= diag_tile) or below
  //             the latest row's window (kt < win_to), or the tile has keys
  //             without data (past the end: implied by kt >= diag_tile; a bad
  //             block entry: checked separately).
  const int last_tile = (Lk - 1) / kBN;
  const int act_lo = W > 0 ? max(0, wpos_lo - W + 1) / kBN : 0;
  const int act_hi = wq_lo < Lq ? min(wpos_hi, Lk - 1) / kBN : -1;
  const int diag_tile = (wpos_lo + 1) / kBN;
  const int win_to = (W > 0 && wpos_hi - W + 1 > 0) ? (wpos_hi - W + 1 + kBN - 1) / kBN : 0;

  // Ring prologue: tiles tile0 .. tile0+2 (clamped to tile1; every DMA is
  // issued unconditionally so the wait counts below are exact).
  // Bad block entries: per stage for spanning tiles (bit s: this wave wrote a
  // row with a bad entry into stage s); for tiles inside one block a sticky
  // flag (once a bad entry was seen, every later tile looks its block up again).
  uint32_t badbits = 0;
  bool bad_seen = false;
  auto note_bad = [&](bool bad, auto st) __attribute__((always_inline)) {
    constexpr int ST = decltype(st)::value;
    if constexpr (ONE) bad_seen |= bad;
    else badbits = (badbits & ~(1u << ST)) | ((bad ? 1u : 0u) << ST);
  };
  note_bad(issue_tile(tile0, std::integral_constant<int, 0>{}), std::integral_constant<int, 0>{});
  note_bad(issue_tile(min(tile0 + 1, tile1), std::integral_constant<int, 1>{}), std::integral_constant<int, 1>{});
  note_bad(issue_tile(min(tile0 + 2, tile1), std::integral_constant<int, 2>{}), std::integral_constant<int, 2>{});

  // This lane's Q^T operand (kept in registers for the whole kernel), loaded
  // after the ring prologue's DMAs are on their way.  One wait for everything
  // then tells the compiler that Q is resident, so it puts no wait for it in
  // the loop (a compiler wait there would also drain the ring's DMAs, which it
  // does not see).  Tile0's DMAs were issued with the next two, so waiting
  // for all three costs about nothing.
  bf16x8_t qreg[8];
  {
    const uint4* qp = static_cast<const uint4*>(a.q) +
                      (static_cast<int64_t>(q0 + (qvalid ? qi : qa)) * hq + head) * 16 + hgrp;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = __builtin_bit_cast(bf16x8_t, qp[2 * kk]);
  }

  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // Byte offsets of this lane's operand reads inside a stage's K and V tiles.
  int kofs[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kofs[kk] = c32 * kRow + k_pos(c32, 2 * kk + hgrp) * 16;
  int vofs[4];   // key (4*hgrp + i16/4) of PV step 0, dims of m-tile mt
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int keyA = hgrp * 4 + (i16 >> 2);
    const int ch = mt * 4 + half * 2 + ((i16 & 3) >> 1);
    vofs[mt] = keyA * kRow + v_pos(keyA, ch) * 16 + (i16 & 1) * 8;
  }

  f32x16_t o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.f;
  float m = -1.0e30f, lsum = 0.f;

  // One tile: wait for its stage, refill the stage read one step earlier, and
  // consume it.
  auto step = [&](int kt, auto st) {
    constexpr int ST = decltype(st)::value;
    constexpr int NXT = (ST + kStages - 1) % kStages;
    // This wave's DMAs for the stage are done once at most the two newer
    // tiles' DMAs are pending; the barrier extends that to every wave (and
    // tells everyone that stage NXT, refilled next, was fully read).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm((kStages - 2) * kDmaPerTile));
    const int kb = kt * kBN;
    bool bad_tile = false;
    if constexpr (ONE) {
      if (kt == last_tile || bad_seen) {
        // Zero this wave's V rows without data (all of them for a bad block,
        // else those past the sequence end) so they cannot reach P.V.
        if (bad_seen) {
          const int lb = kb >> a.block_shift;
          const int blk = table_entry(bt, min(lb, a.max_blocks_per_seq - 1));
          bad_tile = !(lb < a.max_blocks_per_seq &&
                       static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks));
        }
        const int first = bad_tile ? 0 : Lk - kb;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (dma_row[j] >= first) zero_lds16(&v_stage<ST>()[dma_row[j] * kRow + i16 * 16]);
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      }
    } else if ((bad_tile = (badbits >> ST) & 1u)) {
      // Rare path (a block-table entry outside the cache): zero this wave's V
      // rows whose key has no valid block, so stale data cannot reach P.V.
      const uint32_t vm = valid_mask(tile_map<POW2>(a, bt, kb, g, slot_bytes), kb, Lk);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (kb + dma_row[j] < Lk && !((vm >> dma_row[j]) & 1u))
          zero_lds16(&v_stage<ST>()[dma_row[j] * kRow + i16 * 16]);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    }
    __builtin_amdgcn_s_barrier();
    {
      note_bad(issue_tile(min(kt + kStages - 1, tile1), std::integral_constant<int, NXT>{}),
               std::integral_constant<int, NXT>{});
    }

    if (kt < act_lo || kt > act_hi) return;
    bool need_mask = kt >= diag_tile || kt < win_to;
    uint32_t vmask = 0xffffffffu;
    if constexpr (ONE) {
      if (bad_tile) vmask = 0u;
      else if (kt == last_tile && Lk - kb < kBN) vmask = (1u << (Lk - kb)) - 1u;
      need_mask |= bad_tile;
    } else {
      vmask = valid_mask(tile_map<POW2>(a, bt, kb, g, slot_bytes), kb, Lk);
      need_mask |= vmask != 0xffffffffu;
    }

    // Issue priority: two workgroups share each SIMD, one wavefront each.  A
    // wavefront takes the lowest priority while it issues its operand reads
    // and S products (a dependent chain of matrix products with idle issue
    // slots between them), the highest for its softmax (the serial part of
    // the tile), a middle one for P.V, the ring bookkeeping and the next
    // barrier, and the highest again for the epilogue.  The S products then
    // fill the gaps of the other wavefront's softmax.  Prefix workload 32.1
    // against 34.3 us with no priority changes.
    __builtin_amdgcn_s_setprio(0);

    // ---- operand reads (compiler-visible: it waits for each just before its
    // use): K for S^T, then V^T for both PV steps, whose latency hides behind
    // the S product and the softmax.
    u32x4_t kop[8];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) kop[kk] = *reinterpret_cast<const u32x4_t*>(k_stage<ST>() + kofs[kk]);
    u32x2_t va[2][4], vbb[2][4];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        va[ks2][mt] = read_tr16(v_stage<ST>() + vofs[mt] + ks2 * 16 * kRow);
        vbb[ks2][mt] = read_tr16(v_stage<ST>() + vofs[mt] + ks2 * 16 * kRow + 8 * kRow);
      }
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kop[kk]), qreg[kk],
                                                  s, 0, 0, 0);
    // All eight K reads first (left to itself the compiler issues them two at
    // a time, each pair waiting out an LDS round trip before its products),
    // then each S product followed by two of the V^T reads.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }

    __builtin_amdgcn_s_setprio(2);

    // ---- online softmax over this lane's column ------------------------------
    // (16 keys of the tile in this lane, the other 16 in lane ^ 32)
    float mx = -INFINITY;
    if (need_mask) {
      // Keys of the tile this lane's query may see: valid block, causal
      // (key <= qpos) and inside the window (qpos - key < W), as a bit mask
      // over the tile's 32 keys, shifted to this lane's key group.
      const int hi = qpos - kb;                            // last allowed tile key
      const int lo = W > 0 ? qpos - W + 1 - kb : 0;        // first allowed tile key
      uint32_t allow = hi < 0 ? 0u : (hi >= 31 ? 0xffffffffu : (2u << hi) - 1u);
      allow &= lo <= 0 ? 0xffffffffu : (lo > 31 ? 0u : ~((1u << lo) - 1u));
      allow = ((allow & vmask) >> (hgrp * 4));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = POS ? s[r] : s[r] * c;
        s[r] = (allow >> ((r >> 2) * 8 + (r & 3))) & 1u ? x : -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (!POS) s[r] *= c;
        mx = fmaxf(mx, s[r]);
      }
    }
    mx = max_xor32(mx);
    const float mcand = POS ? mx * c : mx;   // candidate running max, scaled (log2) units
    const bool grow = mcand > m + kRescaleSlack;
    if (__ballot(grow) != 0) {
      const float mn = grow ? mcand : m;
      const float alpha = fast_exp2(m - mn);
      m = mn;
      lsum *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;
    }

    __builtin_amdgcn_s_setprio(1);

    // ---- O^T += V^T . P^T ------------------------------------------------------
    // In step ks2 the lane's 8 key slots are keys 16*ks2 + 4*hgrp + {0..3} and
    // 16*ks2 + 8 + 4*hgrp + {0..3} of the tile: accumulator registers
    // 8*ks2 .. 8*ks2+7.  The A operand (V^T: 32 dims x those keys) comes from
    // two transposed reads; for one of them, lane group i16 supplies the
    // address of key (base + i16/4), dims (16*half + 4*(i16%4)) .. +4, and
    // receives dim 16*half + i16 of the four keys.
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      uint32_t pw[4];
#pragma unroll
      for (int r = 0; r < 8; r += 2) {
        const float x0 = s[8 * ks2 + r], x1 = s[8 * ks2 + r + 1];
        const float p0 = fast_exp2(POS ? fmaf(x0, c, -m) : x0 - m);
        const float p1 = fast_exp2(POS ? fmaf(x1, c, -m) : x1 - m);
        pw[r >> 1] = pack_bf16x2(p0, p1);
        lsum = dot2_bf16(pw[r >> 1], 0x3f803f80u, lsum);   // + the two rounded probabilities
      }
      const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x4_t w = {va[ks2][mt].x, va[ks2][mt].y, vbb[ks2][mt].x, vbb[ks2][mt].y};
        const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, w);
        o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, o[mt], 0, 0, 0);
      }
    }
  };

  for (int kt = tile0;;) {
    step(kt, std::integral_constant<int, 0>{});
    if (++kt > tile1) break;
    step(kt, std::integral_constant<int, 1>{});
    if (++kt > tile1) break;
    step(kt, std::integral_constant<int, 2>{});
    if (++kt > tile1) break;
    step(kt, std::integral_constant<int, 3>{});
    if (++kt > tile1) break;
  }
  __builtin_amdgcn_s_setprio(2);
  // Drain this wave's remaining (clamped, unused) DMAs before the wave ends.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- fused store: this workgroup's new tokens into their cache slots -------
  // Rows P+qa .. P+qb-1 of KV head g, 16 lanes per 256-byte row, four rows per
  // thread per round.  The first round's rows and block-table entries are
  // loaded here and stored after the output rows are written, so the loads'
  // latency overlaps that write; more rounds (one query head per KV head)
  // follow.  Done last: a store inside or before the loop would hold up the
  // loop's DMA waits (stores and loads share the in-order vector-memory
  // counter) until its write is acknowledged.  A position whose block-table
  // entry is outside the table or the cache is not stored.
  const int st_rows = qb - qa;
  const int64_t st_src0 = (static_cast<int64_t>(q0) + qa) * slot_bytes + static_cast<int64_t>(g) * kRow +
                          (tid & 15) * 16;
  constexpr int kStride = kThreads / 16;   // rows covered by one pass of the workgroup
  struct StoreRound {
    int r[4], lb[4], blk[4];
    uint4 k[4], v[4];
  };
  auto st_load = [&](StoreRound& R, int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      R.r[i] = r0 + i * kStride;
      const int rr = min(R.r[i], st_rows - 1);
      R.lb[i] = div_block<POW2>(a, P + qa + rr);
      R.blk[i] = bt[min(R.lb[i], a.max_blocks_per_seq - 1)];   // read in bounds, judged at the store
      R.k[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + st_src0 +
                                               static_cast<int64_t>(rr) * slot_bytes);
      R.v[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + st_src0 +
                                               static_cast<int64_t>(rr) * slot_bytes);
    }
    // Keep the table reads unconditional, so all twelve loads are in flight together.
    asm volatile("" : "+v"(R.blk[0]), "+v"(R.blk[1]), "+v"(R.blk[2]), "+v"(R.blk[3]));
  };
  auto st_store = [&](const StoreRound& R) __attribute__((always_inline)) {
    char* kdst = static_cast<char*>(const_cast<void*>(a.k_cache)) + static_cast<int64_t>(g) * kRow + (tid & 15) * 16;
    char* vdst = static_cast<char*>(const_cast<void*>(a.v_cache)) + static_cast<int64_t>(g) * kRow + (tid & 15) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = R.r[i] < st_rows && R.lb[i] < a.max_blocks_per_seq &&
                      static_cast<unsigned>(R.blk[i]) < static_cast<unsigned>(a.num_blocks);
      if (ok) {
        const int pos = P + qa + R.r[i];
        const int64_t dst = (static_cast<int64_t>(R.blk[i]) * a.block_size + pos % a.block_size) * slot_bytes;
        *reinterpret_cast<uint4*>(kdst + dst) = R.k[i];
        *reinterpret_cast<uint4*>(vdst + dst) = R.v[i];
      }
    }
  };
  StoreRound st_first;
  if constexpr (FUSE) st_load(st_first, tid >> 4);

  // ---- normalise and write ---------------------------------------------------
  // The MFMA layout gives each lane one query row (column of O^T), so storing
  // from registers would scatter 8-byte pieces over 32 output rows per
  // instruction.  Instead each wavefront transposes its 32 rows x 256 bytes
  // through LDS (one ring stage per wavefront, free once every wavefront has
  // drained its DMAs and passed the barrier) and writes whole rows with
  // 16-byte coalesced stores.  In LDS, 16-byte chunk c of row r sits at
  // position c ^ (r % 16): the row-wise reads are conflict free and the
  // column-wise writes at most 2-way.
  const float ltot = sum_xor32(lsum);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  __syncthreads();
  char* const ot = wave == 0 ? s_k0 : wave == 1 ? s_k1 : wave == 2 ? s_k2 : s_k3;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int ch = mt * 4 + rg;   // dims 8 ch .. 8 ch + 7; this lane holds half hgrp
      const uint2 v = make_uint2(pack_bf16x2(o[mt][rg * 4] * inv, o[mt][rg * 4 + 1] * inv),
                                 pack_bf16x2(o[mt][rg * 4 + 2] * inv, o[mt][rg * 4 + 3] * inv));
      *reinterpret_cast<uint2*>(ot + c32 * kRow + (ch ^ (c32 & 15)) * 16 + hgrp * 8) = v;
    }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);      // row = this wavefront's column r
    const uint4 v = *reinterpret_cast<const uint4*>(ot + r * kRow + (i16 ^ (r & 15)) * 16);
    const int rcol = wave * 32 + r;
    const int rqi = qa + rcol % BM;
    if (rqi < Lq) {
      uint16_t* orow = static_cast<uint16_t*>(a.out) +
                       (static_cast<int64_t>(q0 + rqi) * hq + g * G + rcol / BM) * kHeadDim;
      *reinterpret_cast<uint4*>(orow + i16 * 8) = v;
    }
  }

  if constexpr (FUSE) {
    st_store(st_first);
    for (int r0 = (tid >> 4) + 4 * kStride; r0 < st_rows; r0 += 4 * kStride) {
      StoreRound R;
      st_load(R, r0);
      st_store(R);
    }
  }
}

// One workgroup per (query tile, sequence, KV head), heaviest tiles first.
template <int G, bool POS, int MODE, bool FUSE>
__global__ void __launch_bounds__(kThreads, 2)
paged_prefill_kernel(PrefillArgs a) {
  paged_prefill_body<G, POS, MODE, FUSE>(a, static_cast<int>(blockIdx.x));
}

}  // namespace
}  // namespace pk
