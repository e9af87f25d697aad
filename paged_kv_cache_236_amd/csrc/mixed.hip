// A mixed batch (chunked prefill: decode sequences and prefill chunks in one
// step, "How lunaryes/nano-vllm works", introduction; nano-vllm-rs README,
// "Run Inference", token budget per step) in one launch whose workgroups are
// of two kinds.  The first ones are prefill work items (query tile, sequence,
// KV head) of the chunks, heaviest first; the rest are decode items (sequence,
// KV head) of the one-token sequences.  The chunks' prefill is bound by the
// chain of key tiles of its longest query tile and the decode rows by HBM, so
// running them side by side in one grid lets the decode rows' K/V stream
// while the long chains compute.  Two launches, or two streams, run them one
// after the other.  Each workgroup runs the same code as the separate kernel
// of its kind (prefill_kernel.h, decode_kernel.h), so the results are
// bit-identical to those launches.
#include "decode_kernel.h"
#include "prefill_kernel.h"

namespace pk {
namespace {

static_assert(kThreads == kDecodeWaves * kWave, "both kinds of workgroup have the same size");

// Grid order: the prefill's heaviest `heavy` workgroups (the first half of its
// work order: items ranked by key-tile count, or latest query tiles first),
// then every decode item, then the rest of the prefill.  The long chains start
// at once; the decode rows then stream on most of the GPU while those chains
// compute, and the short prefill items fill the tail.  Measured on 48 decode
// rows + 4 chunks with latest tiles first: prefill first 95.6 us, the first
// 1 / 2 / 4 / 6 / 8 / 11 of 16 query-tile ranks first 82.2 / 81.5 / 79.8 /
// 80.0 / 78.8 / 83.0 us, two launches 92 us; with the ranked order and the
// first half first, 71.5 us.
template <int G, bool POS>
__global__ void __launch_bounds__(kThreads, 2)
mixed_batch_kernel(PrefillArgs p, DecodeArgs d, int heavy, int decode_groups) {
  const int bx = static_cast<int>(blockIdx.x);
  if (bx < heavy) {
    paged_prefill_body<G, POS, kTileInBlock, false>(p, bx);
    return;
  }
  if (bx >= heavy + decode_groups) {
    paged_prefill_body<G, POS, kTileInBlock, false>(p, bx - decode_groups);
    return;
  }
  // Decode items in the decode kernel's grid order (partition fastest, then
  // KV head, then sequence); one partition per sequence here.
  const int w = bx - heavy;
  decode_partition_body<G, kDecodeWaves, 4, false>(d, 0, w % d.num_kv_heads, w / d.num_kv_heads);
}

template <int G>
hipError_t launch_group(const PrefillArgs& p, const DecodeArgs& d, int64_t prefill_groups,
                        int64_t decode_groups, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(prefill_groups + decode_groups)), block(kThreads);
  const int64_t pairs = static_cast<int64_t>(p.num_seqs) * p.num_kv_heads;
  const int64_t ntiles = prefill_groups / pairs;
  const int heavy = static_cast<int>(pairs * ((ntiles + 1) / 2));
  if (p.scale_log2 > 0.f)
    hipLaunchKernelGGL((mixed_batch_kernel<G, true>), grid, block, 0, stream, p, d, heavy,
                       static_cast<int>(decode_groups));
  else
    hipLaunchKernelGGL((mixed_batch_kernel<G, false>), grid, block, 0, stream, p, d, heavy,
                       static_cast<int>(decode_groups));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mixed_batch(const PrefillArgs& p, const DecodeArgs& d, hipStream_t stream) {
  // The combined kernel covers the common case: tiles inside one cache block
  // (power-of-two block of >= 32 keys), no fused store, the decode rows in one
  // partition each with 16-token chunks, and the same head grouping.  Eight
  // query heads per KV head are left to two launches: the decode body then
  // needs 336 registers and 82 KiB of LDS, one workgroup per CU.
  const int BM = kCols / (p.group > 0 ? p.group : 1);
  const int64_t ntiles = (p.max_seqlen_q + BM - 1) / BM;
  const int64_t prefill_groups = ntiles * p.num_seqs * p.num_kv_heads;
  const int64_t decode_groups = static_cast<int64_t>(d.num_seqs) * d.num_kv_heads;
  const bool in_block = p.block_shift >= 0 && p.block_size >= kBN &&
                        static_cast<int64_t>(p.block_size) * p.num_kv_heads * kRow < (int64_t{1} << 31);
  if (!in_block || p.k_new || d.k_new || d.num_parts != 1 || p.group != d.group || p.group > 4 ||
      kDecodeLoads != 4 || d.block_size % 16 != 0 || prefill_groups <= 0 || decode_groups <= 0 ||
      prefill_groups + decode_groups > 0x7fffffff)
    return hipErrorNotSupported;
  switch (p.group) {
    case 1: return launch_group<1>(p, d, prefill_groups, decode_groups, stream);
    case 2: return launch_group<2>(p, d, prefill_groups, decode_groups, stream);
    case 4: return launch_group<4>(p, d, prefill_groups, decode_groups, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pk
