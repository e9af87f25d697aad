// Host-side launchers of the kernels; called by the C ABI layer (api.hip)
// after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pk {

// Longest block-table row paged_prefill accepts (its entries are staged in LDS).
constexpr int kPrefillMaxBlocksPerSeq = 2048;

struct StoreArgs {
  const void* key;
  const void* value;
  const int32_t* slot_mapping;
  void* k_cache;
  void* v_cache;
  int32_t num_tokens;
  int32_t row_vecs;        // 16-byte vectors per token row (num_kv_heads * head_dim / 8)
  int64_t num_slots;       // num_blocks * block_size
};
hipError_t launch_kv_store(const StoreArgs& a, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const void* k_new;       // bf16 [num_seqs, num_kv_heads, 128]: the token at position L-1, or
  const void* v_new;       // nullptr (then position L-1 is read from the cache like any other)
  float* ws_acc;           // [num_seqs, num_q_heads, num_parts, 128] fp32 (split only)
  float* ws_ml;            // [num_seqs, num_q_heads, num_parts, 2] fp32 (split only)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t group;           // q heads per kv head
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_blocks_per_seq;
  int32_t max_context_len;
  int32_t sliding_window;
  int32_t partition_size;
  int32_t num_parts;       // partition slots per sequence
  int32_t length_order;    // 1: workgroups take (seq, head) items longest-first, paired long/short
  int32_t* merge_counters; // split plans: one arrival counter per (seq, KV head), zero between
                           // launches; nullptr: a combine launch merges the partitions
  float scale_log2;        // softmax scale * log2(e)
  // Varlen form (decode rows of a mixed batch), or nullptr: sequence b's
  // length is cu_seqlens_k[b+1] - cu_seqlens_k[b] (context_lens unused) and its
  // q / out row is cu_seqlens_q[b] (< total_rows); a sequence without exactly
  // one new token is not computed.
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t total_rows;
};
hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream);

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;         // written too when k_new is set
  const void* v_cache;
  const void* k_new;           // bf16 [total_q, num_kv_heads, 128]: the new tokens' K/V, stored
  const void* v_new;           // by the kernel and read from here; nullptr: already in the cache
  const int32_t* block_tables;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_seqlen_q;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t block_size;
  int32_t block_shift;     // log2(block_size) when it is a power of two, else -1
  int32_t max_blocks_per_seq;
  int32_t sliding_window;
  float scale_log2;
  int32_t lpt_order;       // 1: workgroups take (sequence, query tile) items by key-tile count, most first
  uint32_t tiles_recip;    // lpt_order: floor(2^32 / query tiles per sequence) + 1 (0 for one tile),
                           // so item k splits as k / tiles = mulhi(k, tiles_recip), exact while
                           // k * tiles < 2^32 (items are < kPrefillRankMax here)
};
hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream);

// Most (sequence, query tile) items a prefill workgroup ranks by work itself.
constexpr int kPrefillRankMax = 128;

// A mixed batch in one launch: prefill work items of `p` first, then the
// decode items of `d` (one partition per sequence).  hipErrorNotSupported
// (nothing launched) when the configuration is not the one the combined
// kernel covers; the caller then launches the two kinds separately.
hipError_t launch_mixed_batch(const PrefillArgs& p, const DecodeArgs& d, hipStream_t stream);

// Checked mode (index validation).
constexpr int kCheckCounts = 4;
inline int64_t check_bitmap_words(int32_t num_blocks, int32_t block_size) {
  return (static_cast<int64_t>(num_blocks) * block_size + 31) / 32;
}
struct CheckArgs {
  const int32_t* slot_mapping;   // [num_tokens] or nullptr
  const int32_t* block_tables;   // [num_seqs, max_blocks_per_seq] or nullptr
  const int32_t* context_lens;   // [num_seqs], used when cu_seqlens_k is nullptr
  const int32_t* cu_seqlens_q;   // [num_seqs + 1] or nullptr
  const int32_t* cu_seqlens_k;   // [num_seqs + 1] or nullptr
  int32_t num_tokens;
  int32_t num_seqs;
  int32_t max_blocks_per_seq;
  int32_t num_blocks;
  int32_t block_size;
  int32_t* counts;               // [kCheckCounts]
  uint32_t* bitmap;              // [check_bitmap_words] one bit per cache slot
};
hipError_t launch_check_indices(const CheckArgs& a, hipStream_t stream);

}  // namespace pk
