// paged_prefill launcher: picks the kernel instantiation for the head group,
// the sign of the scale, the block addressing mode and the fused store.  The
// kernel is in prefill_kernel.h.
#include "prefill_kernel.h"

namespace pk {
namespace {

template <int G>
hipError_t launch_group(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BM = kCols / G;
  const int64_t ntiles = (a.max_seqlen_q + BM - 1) / BM;
  const int64_t grid = ntiles * a.num_seqs * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 gr(static_cast<unsigned>(grid)), bl(kThreads);
  const bool pos = a.scale_log2 > 0.f;
  // Tiles inside one block need a power-of-two block of >= 32 keys and a block
  // of one KV head's rows under 2 GiB (32-bit offsets inside a block).
  const bool in_block = a.block_shift >= 0 && a.block_size >= kBN &&
                        static_cast<int64_t>(a.block_size) * a.num_kv_heads * kRow < (int64_t{1} << 31);
  const int mode = a.block_shift < 0 ? kDivBlocks : (in_block ? kTileInBlock : kShiftBlocks);
  auto go = [&](auto kernel) { hipLaunchKernelGGL(kernel, gr, bl, 0, stream, a); };
  auto pick = [&](auto fuse) {
    constexpr bool F = decltype(fuse)::value;
    if (pos) {
      if (mode == kTileInBlock) go(paged_prefill_kernel<G, true, kTileInBlock, F>);
      else if (mode == kShiftBlocks) go(paged_prefill_kernel<G, true, kShiftBlocks, F>);
      else go(paged_prefill_kernel<G, true, kDivBlocks, F>);
    } else {
      if (mode == kTileInBlock) go(paged_prefill_kernel<G, false, kTileInBlock, F>);
      else if (mode == kShiftBlocks) go(paged_prefill_kernel<G, false, kShiftBlocks, F>);
      else go(paged_prefill_kernel<G, false, kDivBlocks, F>);
    }
  };
  if (a.k_new) pick(std::true_type{});
  else pick(std::false_type{});
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_prefill(const PrefillArgs& a, hipStream_t stream) {
  switch (a.group) {
    case 1: return launch_group<1>(a, stream);
    case 2: return launch_group<2>(a, stream);
    case 4: return launch_group<4>(a, stream);
    case 8: return launch_group<8>(a, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace pk
