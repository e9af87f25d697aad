// The C ABI (include/pagedkv.h): argument validation, decode split planning,
// workspace sizing and status reporting.  Validation reads only host values,
// never device memory, so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "launch.h"
#include "pagedkv.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace pk {
pk_status record_status(pk_status s, const char* message) {
  if (s == PK_OK) g_last_error.clear();
  else g_last_error = message;
  return s;
}
}  // namespace pk

namespace {

pk_status fail(pk_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  return pk::record_status(s, buf);
}

pk_status ok() { return pk::record_status(PK_OK, ""); }

constexpr double kLog2e = 1.4426950408889634;
constexpr int32_t kHeadDim = 128;
constexpr int64_t kPartitionQuantum = 64;   // 4 wavefronts x 16-token chunks
constexpr int64_t kNumCUs = 256;            // MI355X: 8 XCDs x 32 CUs
constexpr int32_t kOrderMaxSeqs = 64;       // sequences one wavefront can rank
constexpr int64_t kNoSplitKeys = 256;       // with few pairs, contexts this short are not split
constexpr int64_t kMaxPartition = int64_t{1} << 30;   // partition sizes stay far inside int32
constexpr int64_t kMaxSlots = 65535;         // partition slots per sequence
constexpr int32_t kMaxDecodeSeqs = 65535;    // sequences per decode call (a grid dimension)

bool supported_group(int32_t g) { return g == 1 || g == 2 || g == 4 || g == 8; }

pk_status check_cache_shape(int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                            int32_t head_dim) {
  if (num_blocks <= 0) return fail(PK_ERR_INVALID_ARG, "num_blocks must be > 0 (got %d)", num_blocks);
  if (num_kv_heads <= 0) return fail(PK_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", num_kv_heads);
  if (head_dim != kHeadDim)
    return fail(PK_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", head_dim);
  if (block_size < 16 || block_size > 1024 || block_size % 16 != 0)
    return fail(PK_ERR_UNSUPPORTED,
                "block_size %d is not supported (a multiple of 16 in [16, 1024])", block_size);
  const int64_t elems = static_cast<int64_t>(num_blocks) * block_size * num_kv_heads * head_dim;
  if (elems / head_dim / num_kv_heads / block_size != num_blocks)
    return fail(PK_ERR_INVALID_ARG, "cache size overflows");
  return PK_OK;
}

pk_status check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0) return fail(PK_ERR_INVALID_ARG, "num_q_heads must be > 0 (got %d)", num_q_heads);
  if (num_q_heads % num_kv_heads != 0)
    return fail(PK_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (!supported_group(num_q_heads / num_kv_heads))
    return fail(PK_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads = %d is not in {1, 2, 4, 8}",
                num_q_heads / num_kv_heads);
  return PK_OK;
}

struct Plan {
  int32_t partition_size;
  int32_t num_parts;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partition slots one sequence needs: partitions start at its first admitted
// key, so its min(L, W) admitted keys (L without a window) take ceil(./PS).
int64_t slots_for(int64_t max_ctx, int64_t window, int64_t ps) {
  const int64_t keys = window > 0 ? std::min(max_ctx, window) : max_ctx;
  const int64_t n = ceil_div(keys, ps);
  return std::max<int64_t>(n, 1);
}

pk_status plan_decode(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                      int32_t sliding_window, int32_t request, Plan* plan) {
  if (num_seqs < 0) return fail(PK_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_kv_heads <= 0) return fail(PK_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", num_kv_heads);
  if (max_context_len < 0)
    return fail(PK_ERR_INVALID_ARG, "max_context_len must be >= 0 (got %d)", max_context_len);
  if (sliding_window < 0)
    return fail(PK_ERR_INVALID_ARG, "sliding_window must be >= 0 (got %d)", sliding_window);
  if (request < 0 || request % kPartitionQuantum != 0 || request > kMaxPartition)
    return fail(PK_ERR_INVALID_ARG,
                "partition_size_request %d must be 0 or a positive multiple of 64 up to 2^30", request);
  const int64_t ctx = std::max<int32_t>(max_context_len, 1);
  int64_t ps = request;
  if (ps == 0) {
    // Keys one (sequence, KV head) can attend.
    const int64_t eff = sliding_window > 0 ? std::min<int64_t>(ctx, sliding_window) : ctx;
    const int64_t pairs = static_cast<int64_t>(std::max(num_seqs, 1)) * num_kv_heads;
    if (pairs >= kNumCUs) {
      // The grid already covers every CU: one partition per pair, whatever the
      // length (no merge, and the length-ordered pairing applies).  Splitting
      // costs more than it balances: the c = 64 layer in two partitions 43.8
      // against 35.6 us; 64 sequences of 4096..8192 keys in 2048-key
      // partitions 286 against 245 us.
      ps = 64;
      while (ps < eff && ps < kMaxPartition) ps *= 2;
    } else if (eff <= kNoSplitKeys) {
      // Few pairs and short contexts: the whole batch is a few microseconds of
      // latency, and the merge costs more than splitting saves (8 sequences of
      // <= 128 keys: 5.2 us in one partition, 6.6 us in two).
      ps = 64;
      while (ps < eff) ps *= 2;
    } else {
      // Few pairs: split until the grid has a workgroup per CU, 64 keys at
      // least.  Larger partitions on fewer CUs beat more, smaller ones (each
      // split partition pays its merge arrival): c = 8 at 512 keys 7.9 us in
      // 128-key partitions against 9.3 us in 64-key ones, c = 2 at 4096 keys
      // 12.4 against 15.9 us, c = 4 at 1024 keys 8.4 against 11.6 us; one
      // workgroup per two CUs is slower again (c = 8 at 512 keys: 9.5 us).
      ps = 2048;
      while (ps > kPartitionQuantum && pairs * slots_for(ctx, sliding_window, ps) < kNumCUs) ps /= 2;
      // Beyond kMaxSlots partitions of 2048 keys: larger partitions.
      while (slots_for(ctx, sliding_window, ps) > kMaxSlots && ps < kMaxPartition) ps *= 2;
    }
  }
  const int64_t slots = slots_for(ctx, sliding_window, ps);
  if (slots > kMaxSlots) return fail(PK_ERR_UNSUPPORTED, "too many partitions (%lld)", (long long)slots);
  plan->partition_size = static_cast<int32_t>(ps);
  plan->num_parts = static_cast<int32_t>(slots);
  return PK_OK;
}

size_t workspace_bytes_for(int32_t num_seqs, int32_t num_q_heads, const Plan& p) {
  if (p.num_parts <= 1) return 0;
  const size_t heads = static_cast<size_t>(num_seqs) * num_q_heads * p.num_parts;
  const size_t acc = heads * kHeadDim * sizeof(float);
  const size_t acc_aligned = (acc + 255) / 256 * 256;
  return acc_aligned + heads * 2 * sizeof(float);
}

}  // namespace

// ---------------------------------------------------------------------------
// Merge counters for split decode, one per (sequence, KV head) of a call: a
// static pool on every GPU the library runs on, zero when the module loads;
// the partition that merges a pair sets its counter back to zero.  Each call
// takes the next num_seqs * num_kv_heads counters of its device's pool,
// wrapping at the end, so calls in flight at the same time use different
// counters unless more than kMergeCounters pairs are in flight together.  In
// host code `merge_counters` names a host-side stand-in: the device address is
// looked up once per device, with that device current.
namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMergeCounters = int64_t{1} << 20;
static __device__ __align__(256) int32_t merge_counters[kMergeCounters];
std::mutex g_counter_mu;
int32_t* g_counter_ptr[kMaxDevices] = {};
int64_t g_counter_next[kMaxDevices] = {};

// Counters for `pairs` pairs on the device that runs `stream`, or nullptr when
// none can be had (the stream's device is not the current one, the lookup
// failed, or the call has more pairs than the pool): a combine launch then
// merges the partitions.
int32_t* take_merge_counters(void* stream, int64_t pairs) {
  if (pairs <= 0 || pairs > kMergeCounters) return nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  if (stream && hipGetStreamDeviceId(static_cast<hipStream_t>(stream)) != dev) return nullptr;
  std::lock_guard<std::mutex> lock(g_counter_mu);
  if (!g_counter_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(merge_counters)) != hipSuccess || !p) {
      (void)hipGetLastError();   // leave no error for the launch check to find
      return nullptr;
    }
    g_counter_ptr[dev] = static_cast<int32_t*>(p);
  }
  if (g_counter_next[dev] + pairs > kMergeCounters) g_counter_next[dev] = 0;
  int32_t* t = g_counter_ptr[dev] + g_counter_next[dev];
  g_counter_next[dev] += pairs;
  return t;
}

}  // namespace

static pk_status paged_decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                          int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                          float scale, int32_t sliding_window, int32_t partition_size_request,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const void* k_new, const void* v_new,
                          const int32_t* cu_seqlens_q = nullptr,
                          const int32_t* cu_seqlens_k = nullptr, int32_t total_rows = 0,
                          pk::DecodeArgs* capture = nullptr) {
  pk_status s = check_cache_shape(num_blocks, block_size, num_kv_heads, head_dim);
  if (s != PK_OK) return s;
  if ((s = check_heads(num_q_heads, num_kv_heads)) != PK_OK) return s;
  if (max_blocks_per_seq <= 0)
    return fail(PK_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0 (got %d)", max_blocks_per_seq);
  if (num_seqs > kMaxDecodeSeqs)
    return fail(PK_ERR_UNSUPPORTED, "at most %d sequences per decode call (got %d)", kMaxDecodeSeqs,
                num_seqs);
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PK_ERR_UNSUPPORTED,
                "max_blocks_per_seq * block_size = %lld tokens per table row exceeds 2^31 - 1",
                static_cast<long long>(max_blocks_per_seq) * block_size);
  if (!std::isfinite(scale)) return fail(PK_ERR_INVALID_ARG, "scale must be finite");
  Plan p;
  if ((s = plan_decode(num_seqs, num_kv_heads, max_context_len, sliding_window,
                       partition_size_request, &p)) != PK_OK)
    return s;
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables ||
      !(context_lens || (cu_seqlens_q && cu_seqlens_k)))
    return fail(PK_ERR_INVALID_ARG, "null pointer argument");
  const size_t need = workspace_bytes_for(num_seqs, num_q_heads, p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(PK_ERR_WORKSPACE, "workspace must be 16-byte aligned");
  pk::DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.k_new = k_new;
  a.v_new = v_new;
  const size_t heads = static_cast<size_t>(num_seqs) * num_q_heads * p.num_parts;
  a.ws_acc = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            (heads * kHeadDim * sizeof(float) + 255) / 256 * 256)
                 : nullptr;
  a.num_seqs = num_seqs;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_context_len = max_context_len;
  a.sliding_window = sliding_window;
  a.partition_size = p.partition_size;
  a.num_parts = p.num_parts;
  // Length ordering pays when each (seq, KV head) item is one workgroup and
  // there are more items than CUs (several items share a CU); the in-kernel
  // ranking handles up to one wavefront of sequences.  With a window the
  // context length no longer measures an item's work (every long sequence
  // admits W keys), so the ranking is skipped (measured 2 % faster on 64
  // sequences of 4096-8192 keys with a 256-key window).
  a.length_order = p.num_parts == 1 && num_seqs <= kOrderMaxSeqs &&
                   num_seqs * num_kv_heads > kNumCUs && sliding_window == 0;
  a.merge_counters = p.num_parts > 1
                         ? take_merge_counters(stream, static_cast<int64_t>(num_seqs) * num_kv_heads)
                         : nullptr;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * kLog2e);
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.total_rows = total_rows;
  if (capture) {   // checked and built, launched by the caller
    *capture = a;
    return ok();
  }
  const hipError_t e = pk::launch_paged_decode(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PK_ERR_LAUNCH, "paged_decode launch failed: %s", hipGetErrorString(e));
  return ok();
}


extern "C" {

const char* pk_version(void) { return "pagedkv 0.1.0 gfx950"; }

const char* pk_status_string(pk_status s) {
  switch (s) {
    case PK_OK: return "PK_OK";
    case PK_ERR_INVALID_ARG: return "PK_ERR_INVALID_ARG";
    case PK_ERR_UNSUPPORTED: return "PK_ERR_UNSUPPORTED";
    case PK_ERR_WORKSPACE: return "PK_ERR_WORKSPACE";
    case PK_ERR_LAUNCH: return "PK_ERR_LAUNCH";
    case PK_ERR_INDEX: return "PK_ERR_INDEX";
  }
  return "PK_ERR_UNKNOWN";
}

const char* pk_last_error_message(void) { return g_last_error.c_str(); }

pk_status pk_kv_store(const void* key, const void* value, const int32_t* slot_mapping,
                      int32_t num_tokens, void* k_cache, void* v_cache, int32_t num_blocks,
                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim, void* stream) {
  if (num_tokens < 0) return fail(PK_ERR_INVALID_ARG, "num_tokens must be >= 0 (got %d)", num_tokens);
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PK_ERR_INVALID_ARG, "cache dimensions must be > 0");
  if ((static_cast<int64_t>(num_kv_heads) * head_dim) % 8 != 0)
    return fail(PK_ERR_UNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 8");
  if (num_tokens == 0) return ok();
  if (!key || !value || !slot_mapping || !k_cache || !v_cache)
    return fail(PK_ERR_INVALID_ARG, "null pointer argument");
  pk::StoreArgs a;
  a.key = key;
  a.value = value;
  a.slot_mapping = slot_mapping;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_tokens = num_tokens;
  a.row_vecs = static_cast<int32_t>(static_cast<int64_t>(num_kv_heads) * head_dim / 8);
  a.num_slots = static_cast<int64_t>(num_blocks) * block_size;
  const hipError_t e = pk::launch_kv_store(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PK_ERR_LAUNCH, "kv_store launch failed: %s", hipGetErrorString(e));
  return ok();
}

pk_status pk_paged_decode_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len,
                               int32_t sliding_window, int32_t partition_size_request,
                               int32_t* partition_size_out, int32_t* num_partitions_out) {
  Plan p;
  const pk_status s = plan_decode(num_seqs, num_kv_heads, max_context_len, sliding_window,
                                  partition_size_request, &p);
  if (s != PK_OK) return s;
  if (partition_size_out) *partition_size_out = p.partition_size;
  if (num_partitions_out) *num_partitions_out = p.num_parts;
  return ok();
}

size_t pk_paged_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len,
                                      int32_t sliding_window, int32_t partition_size_request) {
  if (head_dim != kHeadDim) {
    fail(PK_ERR_UNSUPPORTED, "head_dim %d is not supported (only 128)", head_dim);
    return 0;
  }
  if (num_kv_heads <= 0 || check_heads(num_q_heads, num_kv_heads) != PK_OK) {
    if (num_kv_heads <= 0) fail(PK_ERR_INVALID_ARG, "num_kv_heads must be > 0");
    return 0;
  }
  Plan p;
  if (plan_decode(num_seqs, num_kv_heads, max_context_len, sliding_window, partition_size_request,
                  &p) != PK_OK)
    return 0;
  ok();
  return workspace_bytes_for(num_seqs, num_q_heads, p);
}

pk_status pk_paged_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                          int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                          int32_t head_dim, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                          float scale, int32_t sliding_window, int32_t partition_size_request,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return paged_decode_impl(out, q, k_cache, v_cache, num_blocks, block_size, num_kv_heads, head_dim,
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                           max_context_len, scale, sliding_window, partition_size_request,
                           workspace, workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode without a caller workspace (pk_paged_decode_noalloc): the split-K
// partials live in `scratch`, a static device array of every GPU the library
// runs on.  In host code `scratch` names a host-side stand-in, not the device
// array: the device address is looked up once per device, with that device
// current, and only that address is passed to kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[PK_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the device that is current and owns
// `stream` (set-up on the first call for a device).
pk_status scratch_address(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PK_ERR_LAUNCH, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PK_ERR_UNSUPPORTED, "device %d is beyond the %d devices supported", dev, kMaxDevices);
  if (stream) {
    const int sdev = hipGetStreamDeviceId(static_cast<hipStream_t>(stream));
    if (sdev != dev)
      return fail(PK_ERR_INVALID_ARG, "the stream belongs to device %d but device %d is current",
                  sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PK_ERR_LAUNCH, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PK_OK;
}

}  // namespace

extern "C" {

pk_status pk_paged_decode_noalloc(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, int32_t num_blocks, int32_t block_size,
                                  int32_t num_kv_heads, int32_t head_dim,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, int32_t max_context_len, float scale,
                                  int32_t sliding_window, int32_t partition_size_request,
                                  void* stream) {
  pk_status s = check_cache_shape(num_blocks, block_size, num_kv_heads, head_dim);
  if (s != PK_OK) return s;
  if ((s = check_heads(num_q_heads, num_kv_heads)) != PK_OK) return s;
  Plan p;
  if ((s = plan_decode(num_seqs, num_kv_heads, max_context_len, sliding_window,
                       partition_size_request, &p)) != PK_OK)
    return s;
  const size_t need = workspace_bytes_for(num_seqs, num_q_heads, p);
  if (need > PK_NOALLOC_SCRATCH_BYTES)
    return fail(PK_ERR_WORKSPACE,
                "pk_paged_decode_noalloc: the split-K partials need %zu bytes, more than the "
                "%zu-byte static scratch (use pk_paged_decode with a workspace, or a larger "
                "partition_size_request)",
                need, static_cast<size_t>(PK_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0 && (s = scratch_address(stream, &ws)) != PK_OK) return s;
  return paged_decode_impl(out, q, k_cache, v_cache, num_blocks, block_size, num_kv_heads, head_dim,
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                           max_context_len, scale, sliding_window, partition_size_request,
                           ws, need > 0 ? static_cast<size_t>(PK_NOALLOC_SCRATCH_BYTES) : 0,
                           stream, nullptr, nullptr);
}

pk_status pk_paged_decode_store(void* out, const void* q, const void* k_new, const void* v_new,
                                void* k_cache, void* v_cache, int32_t num_blocks,
                                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, int32_t max_context_len, float scale,
                                int32_t sliding_window, int32_t partition_size_request,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new))
    return fail(PK_ERR_INVALID_ARG, "null pointer argument (k_new / v_new)");
  return paged_decode_impl(out, q, k_cache, v_cache, num_blocks, block_size, num_kv_heads, head_dim,
                           block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads,
                           max_context_len, scale, sliding_window, partition_size_request,
                           workspace, workspace_bytes, stream, k_new, v_new);
}

namespace {

pk_status prefill_common(void* out, const void* q, const void* k_new, const void* v_new,
                         const void* k_cache, const void* v_cache, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                         int32_t num_q_heads, float scale, int32_t sliding_window, bool fused,
                         void* stream, pk::PrefillArgs* capture = nullptr) {
  pk_status s = check_cache_shape(num_blocks, block_size, num_kv_heads, head_dim);
  if (s != PK_OK) return s;
  if ((s = check_heads(num_q_heads, num_kv_heads)) != PK_OK) return s;
  if (max_blocks_per_seq <= 0)
    return fail(PK_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0 (got %d)", max_blocks_per_seq);
  if (max_blocks_per_seq > pk::kPrefillMaxBlocksPerSeq)
    return fail(PK_ERR_UNSUPPORTED, "paged_prefill supports max_blocks_per_seq <= %d (got %d)",
                pk::kPrefillMaxBlocksPerSeq, max_blocks_per_seq);
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0)
    return fail(PK_ERR_INVALID_ARG, "num_seqs, total_q and max_seqlen_q must be >= 0");
  if (sliding_window < 0)
    return fail(PK_ERR_INVALID_ARG, "sliding_window must be >= 0 (got %d)", sliding_window);
  if (!std::isfinite(scale)) return fail(PK_ERR_INVALID_ARG, "scale must be finite");
  if (num_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !cu_seqlens_k)
    return fail(PK_ERR_INVALID_ARG, "null pointer argument");
  if (fused && (!k_new || !v_new)) return fail(PK_ERR_INVALID_ARG, "null key or value");
  pk::PrefillArgs a;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = fused ? k_new : nullptr;
  a.v_new = fused ? v_new : nullptr;
  a.block_tables = block_tables;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.max_seqlen_q = max_seqlen_q;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.block_shift = -1;
  for (int s = 0; s < 31; ++s)
    if ((1 << s) == block_size) a.block_shift = s;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.sliding_window = sliding_window;
  a.scale_log2 = static_cast<float>(static_cast<double>(scale) * kLog2e);
  {
    // Items ranked by their key-tile count in each workgroup (longest first)
    // when there are few enough of them; else latest query tile first.
    const int64_t bm = 128 / a.group;
    const int64_t tiles = (max_seqlen_q + bm - 1) / bm;
    const int64_t items = static_cast<int64_t>(num_seqs) * tiles;
    a.lpt_order = items <= pk::kPrefillRankMax ? 1 : 0;
    a.tiles_recip = tiles > 1 ? static_cast<uint32_t>((int64_t{1} << 32) / tiles + 1) : 0u;
  }
  if (capture) {   // checked and built, launched by the caller
    *capture = a;
    return ok();
  }
  const hipError_t e = pk::launch_paged_prefill(a, static_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported)
    return fail(PK_ERR_UNSUPPORTED, "paged_prefill: this configuration is not implemented");
  if (e != hipSuccess) return fail(PK_ERR_LAUNCH, "paged_prefill launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

pk_status pk_paged_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                           int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                           int32_t head_dim, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t total_q,
                           int32_t max_seqlen_q, int32_t num_q_heads, float scale,
                           int32_t sliding_window, void* stream) {
  return prefill_common(out, q, nullptr, nullptr, k_cache, v_cache, num_blocks, block_size,
                        num_kv_heads, head_dim, block_tables, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_k, num_seqs, total_q, max_seqlen_q, num_q_heads, scale,
                        sliding_window, false, stream);
}

size_t pk_check_indices_workspace_size(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PK_ERR_INVALID_ARG, "num_blocks and block_size must be > 0");
    return 0;
  }
  ok();
  return static_cast<size_t>(pk::check_bitmap_words(num_blocks, block_size)) * sizeof(uint32_t);
}

pk_status pk_check_indices(const int32_t* slot_mapping, int32_t num_tokens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           int32_t num_seqs, const int32_t* context_lens,
                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                           int32_t num_blocks, int32_t block_size, int32_t* counts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PK_ERR_INVALID_ARG, "num_blocks and block_size must be > 0");
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0)
    return fail(PK_ERR_INVALID_ARG, "num_tokens, num_seqs and max_blocks_per_seq must be >= 0");
  if (!counts) return fail(PK_ERR_INVALID_ARG, "counts must not be NULL");
  if (num_tokens > 0 && !slot_mapping) return fail(PK_ERR_INVALID_ARG, "null slot_mapping");
  if (num_seqs > 0 && (!block_tables || max_blocks_per_seq <= 0 || !(context_lens || cu_seqlens_k)))
    return fail(PK_ERR_INVALID_ARG, "sequences need block_tables, max_blocks_per_seq > 0 and "
                                    "context_lens or cu_seqlens_k");
  const size_t need = static_cast<size_t>(pk::check_bitmap_words(num_blocks, block_size)) * sizeof(uint32_t);
  if (!workspace || workspace_bytes < need)
    return fail(PK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (reinterpret_cast<uintptr_t>(workspace) % 4 != 0 || reinterpret_cast<uintptr_t>(counts) % 4 != 0)
    return fail(PK_ERR_INVALID_ARG, "workspace and counts must be 4-byte aligned");
  pk::CheckArgs a;
  a.slot_mapping = num_tokens > 0 ? slot_mapping : nullptr;
  a.block_tables = num_seqs > 0 ? block_tables : nullptr;
  a.context_lens = context_lens;
  a.cu_seqlens_q = cu_seqlens_q;
  a.cu_seqlens_k = cu_seqlens_k;
  a.num_tokens = num_tokens;
  a.num_seqs = num_seqs;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.counts = counts;
  a.bitmap = static_cast<uint32_t*>(workspace);
  const hipError_t e = pk::launch_check_indices(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PK_ERR_LAUNCH, "check_indices launch failed: %s", hipGetErrorString(e));
  return ok();
}

pk_status pk_paged_prefill_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                  int32_t head_dim, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, int32_t num_seqs,
                                  int32_t num_decode_seqs, int32_t total_q, int32_t max_seqlen_q,
                                  int32_t max_decode_context_len, int32_t num_q_heads, float scale,
                                  int32_t sliding_window, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  if (num_seqs < 0 || num_decode_seqs < 0 || num_decode_seqs > num_seqs)
    return fail(PK_ERR_INVALID_ARG, "need 0 <= num_decode_seqs <= num_seqs (got %d of %d)",
                num_decode_seqs, num_seqs);
  if (total_q < 0) return fail(PK_ERR_INVALID_ARG, "total_q must be >= 0 (got %d)", total_q);
  if (max_decode_context_len < 0)
    return fail(PK_ERR_INVALID_ARG, "max_decode_context_len must be >= 0 (got %d)",
                max_decode_context_len);
  if (num_seqs > 0 && (!cu_seqlens_q || !cu_seqlens_k || !block_tables))
    return fail(PK_ERR_INVALID_ARG, "null pointer argument");
  // Check both parts before launching either.
  pk_status s = check_cache_shape(num_blocks, block_size, num_kv_heads, head_dim);
  if (s != PK_OK) return s;
  if ((s = check_heads(num_q_heads, num_kv_heads)) != PK_OK) return s;
  if (max_blocks_per_seq <= 0 || max_blocks_per_seq > pk::kPrefillMaxBlocksPerSeq)
    return fail(max_blocks_per_seq <= 0 ? PK_ERR_INVALID_ARG : PK_ERR_UNSUPPORTED,
                "max_blocks_per_seq must be in [1, %d] (got %d)", pk::kPrefillMaxBlocksPerSeq,
                max_blocks_per_seq);
  Plan p;
  if ((s = plan_decode(num_decode_seqs, num_kv_heads, max_decode_context_len, sliding_window, 0,
                       &p)) != PK_OK)
    return s;
  const size_t need = workspace_bytes_for(num_decode_seqs, num_q_heads, p);
  if (num_decode_seqs > 0 && need > 0 && (!workspace || workspace_bytes < need))
    return fail(PK_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  const int32_t rest = num_seqs - num_decode_seqs;
  auto decode_part = [&](void* st, pk::DecodeArgs* capture) {
    return paged_decode_impl(out, q, k_cache, v_cache, num_blocks, block_size, num_kv_heads,
                             head_dim, block_tables, max_blocks_per_seq, nullptr, num_decode_seqs,
                             num_q_heads, max_decode_context_len, scale, sliding_window, 0,
                             workspace, workspace_bytes, st, nullptr, nullptr, cu_seqlens_q,
                             cu_seqlens_k, total_q, capture);
  };
  auto prefill_part = [&](void* st, pk::PrefillArgs* capture) {
    return prefill_common(out, q, nullptr, nullptr, k_cache, v_cache, num_blocks, block_size,
                          num_kv_heads, head_dim,
                          block_tables + static_cast<int64_t>(num_decode_seqs) * max_blocks_per_seq,
                          max_blocks_per_seq, cu_seqlens_q + num_decode_seqs,
                          cu_seqlens_k + num_decode_seqs, rest, total_q, max_seqlen_q, num_q_heads,
                          scale, sliding_window, false, st, capture);
  };
  // Both kinds in one launch when the combined kernel covers the shapes (the
  // prefill's long chains and the decode rows' streaming then overlap),
  // else the decode rows and then the prefill on the caller's stream.
  // (Two streams measured no faster: the two kernels did not overlap.)
  if (num_decode_seqs > 0 && rest > 0 && total_q > 0 && max_seqlen_q > 0) {
    pk::DecodeArgs da;
    pk::PrefillArgs pa;
    if ((s = decode_part(stream, &da)) != PK_OK) return s;
    if ((s = prefill_part(stream, &pa)) != PK_OK) return s;
    const hipError_t e = pk::launch_mixed_batch(pa, da, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) return ok();
    if (e != hipErrorNotSupported)
      return fail(PK_ERR_LAUNCH, "mixed batch launch failed: %s", hipGetErrorString(e));
  }
  if (num_decode_seqs > 0 && (s = decode_part(stream, nullptr)) != PK_OK) return s;
  if (rest > 0 && (s = prefill_part(stream, nullptr)) != PK_OK) return s;
  return ok();
}

pk_status pk_paged_prefill_store(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, int32_t num_blocks,
                                 int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t num_seqs, int32_t total_q, int32_t max_seqlen_q,
                                 int32_t num_q_heads, float scale, int32_t sliding_window,
                                 void* stream) {
  return prefill_common(out, q, key, value, k_cache, v_cache, num_blocks, block_size,
                        num_kv_heads, head_dim, block_tables, max_blocks_per_seq, cu_seqlens_q,
                        cu_seqlens_k, num_seqs, total_q, max_seqlen_q, num_q_heads, scale,
                        sliding_window, true, stream);
}

}  // extern "C"
