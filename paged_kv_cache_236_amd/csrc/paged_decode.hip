// paged_decode launcher: picks the kernel instantiation for the head group
// and the chunk width.  Split plans run as one launch that merges its own
// partitions when merge counters are given, else with the combine kernel
// after the partition kernel.  The kernels are in decode_kernel.h.
#include "decode_kernel.h"

namespace pk {
namespace {

template <int G>
hipError_t launch_group(const DecodeArgs& a, hipStream_t stream) {
  const int64_t merged_groups = static_cast<int64_t>(a.num_parts) * a.num_seqs * a.num_kv_heads;
  if (a.num_parts > 1 && a.merge_counters && merged_groups <= 0x7fffffff) {
    // Split plan, merged in the same launch (chunk width as below).
    const dim3 grid(static_cast<unsigned>(merged_groups)), block(kDecodeWaves * kWave);
    const bool wide = kDecodeLoads > 4 && a.block_size % (4 * kDecodeLoads) == 0;
    if (wide && a.k_new)
      hipLaunchKernelGGL((decode_partition_merged_kernel<G, kDecodeWaves, kDecodeLoads, true>), grid, block, 0, stream, a);
    else if (wide)
      hipLaunchKernelGGL((decode_partition_merged_kernel<G, kDecodeWaves, kDecodeLoads, false>), grid, block, 0, stream, a);
    else if (a.k_new)
      hipLaunchKernelGGL((decode_partition_merged_kernel<G, kDecodeWaves, 4, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partition_merged_kernel<G, kDecodeWaves, 4, false>), grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid(a.num_parts, a.num_kv_heads, a.num_seqs);
  // Chunks must not straddle a cache block: fall back to 16-token chunks when
  // block_size is not a multiple of the wider chunk.
  const bool fuse = a.k_new != nullptr;
  if (kDecodeLoads > 4 && a.block_size % (4 * kDecodeLoads) == 0) {
    if (fuse)
      hipLaunchKernelGGL((decode_partition_kernel<G, kDecodeWaves, kDecodeLoads, true>), grid,
                         dim3(kDecodeWaves * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partition_kernel<G, kDecodeWaves, kDecodeLoads, false>), grid,
                         dim3(kDecodeWaves * kWave), 0, stream, a);
  } else {
    if (fuse)
      hipLaunchKernelGGL((decode_partition_kernel<G, kDecodeWaves, 4, true>), grid,
                         dim3(kDecodeWaves * kWave), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_partition_kernel<G, kDecodeWaves, 4, false>), grid,
                         dim3(kDecodeWaves * kWave), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_parts <= 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<G>), dim3(a.num_kv_heads, a.num_seqs),
                     dim3(G * kHeadDim), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_paged_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (a.group) {
    case 1: return launch_group<1>(a, stream);
    case 2: return launch_group<2>(a, stream);
    case 4: return launch_group<4>(a, stream);
    case 8: return launch_group<8>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pk
