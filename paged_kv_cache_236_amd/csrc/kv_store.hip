// kv_store: the slot-mapping scatter of new K/V rows into paged cache blocks
// (nano-vllm-rs README, "GGUF Models": the KV cache is paged; lunaryes/nano-vllm
// diagram, "Connections": the block manager allocates the cached blocks whose
// slots the new tokens are written to).
//
// One workgroup per token.  A token's K row and V row are each
// num_kv_heads * head_dim bf16 (2 KiB at 8 x 128), contiguous in the input and
// contiguous in the cache slot, so the copy is two runs of 128-bit vector
// loads/stores: every lane moves 16 bytes, fully coalesced.  It is a bit copy.
#include "device_common.h"
#include "launch.h"

namespace pk {
namespace {

constexpr int kStoreThreads = 256;

__global__ void __launch_bounds__(kStoreThreads)
kv_store_kernel(const uint4* __restrict__ key, const uint4* __restrict__ value,
                const int32_t* __restrict__ slot_mapping,
                uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                int32_t row_vecs, int64_t num_slots) {
  const int64_t token = blockIdx.x;
  const int64_t slot = slot_mapping[token];
  // -1 marks a padding token; anything outside the cache is not stored either.
  if (slot < 0 || slot >= num_slots) return;
  const uint4* ksrc = key + token * row_vecs;
  const uint4* vsrc = value + token * row_vecs;
  uint4* kdst = k_cache + slot * row_vecs;
  uint4* vdst = v_cache + slot * row_vecs;
  // Lanes [0, row_vecs) copy the K row, the next row_vecs lanes the V row.
  for (int i = threadIdx.x; i < 2 * row_vecs; i += kStoreThreads) {
    if (i < row_vecs) {
      kdst[i] = ksrc[i];
    } else {
      vdst[i - row_vecs] = vsrc[i - row_vecs];
    }
  }
}

}  // namespace

hipError_t launch_kv_store(const StoreArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_store_kernel, dim3(a.num_tokens), dim3(kStoreThreads), 0, stream,
                     static_cast<const uint4*>(a.key), static_cast<const uint4*>(a.value),
                     a.slot_mapping, static_cast<uint4*>(a.k_cache),
                     static_cast<uint4*>(a.v_cache), a.row_vecs, a.num_slots);
  return hipGetLastError();
}

}  // namespace pk
