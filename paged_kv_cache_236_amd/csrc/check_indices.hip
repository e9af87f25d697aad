// Checked mode: device-side validation of the index arrays that the fast
// paths trust (they bounds-check every access, so a bad index never reads or
// writes out of bounds, but it silently changes the answer).  Each kernel
// counts violations into a caller-owned int32 array; nothing is allocated.
//
//   counts[0]  slot_mapping entries outside [-1, num_blocks * block_size)
//   counts[1]  repeated slots: every occurrence of a slot >= 0 after its first
//   counts[2]  block-table entries outside [0, num_blocks) within a sequence's
//              used range (entries past it are never read and not checked)
//   counts[3]  sequences with inconsistent lengths: a context length below 0
//              or beyond the table's capacity, and with cu_seqlens a
//              decreasing prefix sum or fewer keys than new queries
//
// Slot uniqueness uses a bitmap of one bit per cache slot (the workspace),
// set with atomic OR; the clear kernel zeroes it and the counts first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace pk {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) clear_kernel(uint32_t* bitmap, int64_t words, int32_t* counts) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < words) bitmap[i] = 0u;
  if (i < kCheckCounts) counts[i] = 0;
}

__global__ void __launch_bounds__(kThreads) slots_kernel(CheckArgs a) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i >= a.num_tokens) return;
  const int64_t s = a.slot_mapping[i];
  const int64_t nslots = static_cast<int64_t>(a.num_blocks) * a.block_size;
  if (s < -1 || s >= nslots) {
    atomicAdd(&a.counts[0], 1);
  } else if (s >= 0) {
    const uint32_t bit = 1u << (s & 31);
    if (atomicOr(&a.bitmap[s >> 5], bit) & bit) atomicAdd(&a.counts[1], 1);
  }
}

// One workgroup per sequence: its lengths, then its used table entries.
__global__ void __launch_bounds__(kThreads) tables_kernel(CheckArgs a) {
  const int b = blockIdx.x;
  const int64_t cap = static_cast<int64_t>(a.max_blocks_per_seq) * a.block_size;
  int64_t L;
  bool bad = false;
  if (a.cu_seqlens_k) {
    L = static_cast<int64_t>(a.cu_seqlens_k[b + 1]) - a.cu_seqlens_k[b];
    if (a.cu_seqlens_q) {
      const int64_t lq = static_cast<int64_t>(a.cu_seqlens_q[b + 1]) - a.cu_seqlens_q[b];
      bad |= lq < 0 || lq > L;
    }
  } else {
    L = a.context_lens[b];
  }
  bad |= L < 0 || L > cap;
  if (threadIdx.x == 0 && bad) atomicAdd(&a.counts[3], 1);
  if (L <= 0) return;
  const int64_t used = (min(L, cap) + a.block_size - 1) / a.block_size;
  const int32_t* row = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;
  int n = 0;
  for (int64_t j = threadIdx.x; j < used; j += kThreads)
    n += static_cast<unsigned>(row[j]) >= static_cast<unsigned>(a.num_blocks);
  if (n) atomicAdd(&a.counts[2], n);
}

}  // namespace

hipError_t launch_check_indices(const CheckArgs& a, hipStream_t stream) {
  const int64_t words = check_bitmap_words(a.num_blocks, a.block_size);
  const int64_t clear_n = words > kCheckCounts ? words : kCheckCounts;
  hipLaunchKernelGGL(clear_kernel, dim3(static_cast<unsigned>((clear_n + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, a.bitmap, words, a.counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.num_tokens > 0 && a.slot_mapping) {
    hipLaunchKernelGGL(slots_kernel, dim3(static_cast<unsigned>((a.num_tokens + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.num_seqs > 0 && a.block_tables) {
    hipLaunchKernelGGL(tables_kernel, dim3(static_cast<unsigned>(a.num_seqs)), dim3(kThreads), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pk
