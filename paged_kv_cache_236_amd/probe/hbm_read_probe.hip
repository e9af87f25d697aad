// HBM measurement probe (not part of the library).
//
//   hbm_read_probe        streaming-read ceiling: grid-stride 16-byte loads over a
//                         4 GiB buffer (well beyond the 256 MB MALL), U loads in
//                         flight per thread, with and without the non-temporal hint;
//                         then a 1 GiB copy.
//   hbm_read_probe copy   only the 1 GiB copy: a plain copy kernel of known size,
//                         used to calibrate the FETCH_SIZE / WRITE_SIZE counters.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ void __launch_bounds__(256) read_stream(const u32x4* __restrict__ p, size_t n, unsigned* out) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = NT ? __builtin_nontemporal_load(p + i + u * stride) : p[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x12345678u) out[0] = acc;
}

// copy for counter calibration: n 16-byte vectors
__global__ void __launch_bounds__(256) copy_kernel(const u32x4* __restrict__ a, u32x4* __restrict__ b, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) b[i] = a[i];
}

#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("err %s line %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)

template <int U, bool NT>
float run(const u32x4* p, size_t n, unsigned* out, int blocks) {
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  read_stream<U, NT><<<blocks, 256>>>(p, n, out);
  hipEventRecord(a);
  const int reps = 5;
  for (int r = 0; r < reps; ++r) read_stream<U, NT><<<blocks, 256>>>(p, n, out);
  hipEventRecord(b); hipEventSynchronize(b);
  float ms; hipEventElapsedTime(&ms, a, b);
  return (double)n * 16 * reps / (ms * 1e-3) / 1e9;
}

int main(int argc, char** argv) {
  const bool copy_only = argc > 1;
  const size_t bytes = 4ull << 30;
  const size_t n = bytes / 16;
  u32x4* p; unsigned* out; u32x4* q;
  CK(hipMalloc(&p, bytes)); CK(hipMalloc(&out, 64)); CK(hipMalloc(&q, 1ull << 30));
  CK(hipMemset(p, 1, bytes));
  int blocks_list[] = {1024, 2048, 4096, 8192, 16384};
  for (int blocks : blocks_list) {
    if (copy_only) break;
    printf("blocks %5d: U1 %.0f  U4 %.0f  U8 %.0f  U16 %.0f | NT U4 %.0f  U8 %.0f  U16 %.0f GB/s\n", blocks,
           run<1, false>(p, n, out, blocks), run<4, false>(p, n, out, blocks), run<8, false>(p, n, out, blocks),
           run<16, false>(p, n, out, blocks), run<4, true>(p, n, out, blocks), run<8, true>(p, n, out, blocks),
           run<16, true>(p, n, out, blocks));
  }
  // copy kernel, 1 GiB -> 1 GiB region (for counter calibration): 64M vectors
  const size_t nc = (1ull << 30) / 16;
  hipEvent_t a, b; hipEventCreate(&a); hipEventCreate(&b);
  copy_kernel<<<8192, 256>>>(p, q, nc);
  hipEventRecord(a);
  copy_kernel<<<8192, 256>>>(p, q, nc);
  hipEventRecord(b); hipEventSynchronize(b);
  float ms; hipEventElapsedTime(&ms, a, b);
  printf("copy 1 GiB: %.3f ms, %.0f GB/s (read+write)\n", ms, 2.0 * (1ull << 30) / (ms * 1e-3) / 1e9);
  CK(hipDeviceSynchronize());
  hipFree(p); hipFree(q); hipFree(out);
  return 0;
}
