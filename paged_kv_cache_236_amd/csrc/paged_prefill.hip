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
// Formulation.  Per 64-key tile the wavefront computes S^T = K . Q^T (keys x
// its 32 columns; A = K rows from LDS, B = Q^T held in registers for the whole
// kernel) and then O^T += V^T . P^T (head dims x columns).  In the 32x32 MFMA
// output layout a lane holds one column and 16 key rows, which are exactly the
// key slots the lane must supply as the B operand of the PV product, so the
// probabilities never leave registers; the online-softmax state (m, l) is
// per lane.  V is written to LDS transposed (V^T[dim][key]) so that the A
// operand of PV is two contiguous 8-byte LDS reads per lane.  Both LDS tiles
// are padded so that the MFMA operand reads are bank-conflict free.
//
// K/V tiles are fetched through the block table into registers one tile
// ahead, then written to the other of two LDS buffers: one barrier per tile.
//
// Work order: query tiles are issued heaviest (latest, most keys) first, and
// with num_seqs * num_kv_heads a multiple of 8 all tiles of one (b, g) pair land
// on the same XCD (workgroups are dealt round-robin over the 8 XCDs), so the
// pair's K/V is reused from that XCD's L2.
#include "device_common.h"
#include "launch.h"

namespace pk {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 64;                 // keys per tile
constexpr int kCols = 128;              // query columns (head x row) per workgroup
constexpr int kThreads = 256;           // 4 wavefronts x 32 columns
constexpr int kKRow = kHeadDim + 8;     // bf16 per K row in LDS (16-byte pad)
constexpr int kVRow = kBN + 4;          // bf16 per V^T row in LDS (8-byte pad)
constexpr int kKTile = kBN * kKRow;     // bf16
constexpr int kVTile = kHeadDim * kVRow;

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// One K/V tile (64 keys) in flight in registers: four 16-byte K chunks and
// four 16-byte V chunks per thread, plus a validity bit per K chunk's key.
struct TileRegs {
  uint4 k0, k1, k2, k3;
  uint4 v0, v1, v2, v3;
  uint32_t kvalid;   // bit it: key of K chunk `it` is a valid cache slot
};

// Block-table entries of the keys a workgroup touches are staged in LDS once;
// the host rejects max_blocks_per_seq > kPrefillMaxBlocksPerSeq.
__shared__ int32_t s_bt[kPrefillMaxBlocksPerSeq];   // entries lb0 .. lb1 of the row

struct Walk {
  int lb0;
  int Lk;
  int block_size;
  float inv_block_size;
  int max_blocks;
  int num_blocks;
};

// j / block_size for 0 <= j < 2^24 without an integer divide: a float
// estimate corrected by one step.
__device__ __forceinline__ int div_bs(int j, const Walk& w) {
  int q = static_cast<int>(static_cast<float>(j) * w.inv_block_size);
  q += ((q + 1) * w.block_size <= j) ? 1 : 0;
  q -= (q * w.block_size > j) ? 1 : 0;
  return q;
}

// Cache slot of key j of the sequence; *valid is false (and the slot 0, a
// harmless address) when j is past the sequence or its block is outside the
// table or the cache.  Branch-free.
__device__ __forceinline__ int64_t key_slot(const Walk& w, int j, bool* valid) {
  const int lb = div_bs(j, w);
  bool ok = j < w.Lk && lb < w.max_blocks;
  const int lbc = ok ? lb : w.lb0;
  const int blk = s_bt[lbc - w.lb0];
  ok = ok && static_cast<unsigned>(blk) < static_cast<unsigned>(w.num_blocks);
  *valid = ok;
  return ok ? static_cast<int64_t>(blk) * w.block_size + (j - lb * w.block_size) : 0;
}

// K chunk `it` of thread tid: key (it*256 + tid) / 16, 16-byte column tid % 16;
// 16 consecutive threads read one 256-byte row.
__device__ __forceinline__ uint4 load_k_chunk(const PrefillArgs& a, const Walk& w, int kbase,
                                              int g, int tid, int it, uint32_t& valid) {
  const int idx = it * kThreads + tid;
  bool ok;
  const int64_t s = key_slot(w, kbase + (idx >> 4), &ok);
  valid |= (ok ? 1u : 0u) << it;
  const int64_t row_vecs = static_cast<int64_t>(a.num_kv_heads) * 16;
  return static_cast<const uint4*>(a.k_cache)[s * row_vecs + g * 16 + (idx & 15)];
}

__device__ __forceinline__ TileRegs load_tile(const PrefillArgs& a, const Walk& w, int kbase,
                                              int g, int tid) {
  TileRegs r;
  r.kvalid = 0;
  r.k0 = load_k_chunk(a, w, kbase, g, tid, 0, r.kvalid);
  r.k1 = load_k_chunk(a, w, kbase, g, tid, 1, r.kvalid);
  r.k2 = load_k_chunk(a, w, kbase, g, tid, 2, r.kvalid);
  r.k3 = load_k_chunk(a, w, kbase, g, tid, 3, r.kvalid);
  // V: keys 2p, 2p+1 (p = tid % 32), 16-byte columns tid/32 and tid/32 + 8.
  // Rows of invalid keys are zeroed: their probability is 0, and a zero row
  // keeps stale cache contents (possibly NaN patterns) out of P.V.
  const uint4* vc = static_cast<const uint4*>(a.v_cache);
  const int64_t row_vecs = static_cast<int64_t>(a.num_kv_heads) * 16;
  const int p = tid & 31;
  bool ok0, ok1;
  const int64_t s0 = key_slot(w, kbase + 2 * p, &ok0);
  const int64_t s1 = key_slot(w, kbase + 2 * p + 1, &ok1);
  const uint4* r0 = vc + s0 * row_vecs + g * 16 + (tid >> 5);
  const uint4* r1 = vc + s1 * row_vecs + g * 16 + (tid >> 5);
  const uint4 zero = make_uint4(0, 0, 0, 0);
  r.v0 = ok0 ? r0[0] : zero;
  r.v1 = ok1 ? r1[0] : zero;
  r.v2 = ok0 ? r0[8] : zero;
  r.v3 = ok1 ? r1[8] : zero;
  return r;
}

__device__ __forceinline__ uint32_t pick_pair(uint32_t a, uint32_t b, int hi) {
  // (half `hi` of a) | (half `hi` of b) << 16
  return hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// Write the two keys' 8 dims of one 16-byte column into V^T (8 rows, 2 keys each).
__device__ __forceinline__ void store_vt_pair(uint16_t* vt_lds, int ch, int p, const uint4& a,
                                              const uint4& b) {
  uint16_t* base = vt_lds + ch * 8 * kVRow + 2 * p;
  *reinterpret_cast<uint32_t*>(base + 0 * kVRow) = pick_pair(a.x, b.x, 0);
  *reinterpret_cast<uint32_t*>(base + 1 * kVRow) = pick_pair(a.x, b.x, 1);
  *reinterpret_cast<uint32_t*>(base + 2 * kVRow) = pick_pair(a.y, b.y, 0);
  *reinterpret_cast<uint32_t*>(base + 3 * kVRow) = pick_pair(a.y, b.y, 1);
  *reinterpret_cast<uint32_t*>(base + 4 * kVRow) = pick_pair(a.z, b.z, 0);
  *reinterpret_cast<uint32_t*>(base + 5 * kVRow) = pick_pair(a.z, b.z, 1);
  *reinterpret_cast<uint32_t*>(base + 6 * kVRow) = pick_pair(a.w, b.w, 0);
  *reinterpret_cast<uint32_t*>(base + 7 * kVRow) = pick_pair(a.w, b.w, 1);
}

__device__ __forceinline__ void store_tile(const TileRegs& r, uint16_t* k_lds, uint16_t* vt_lds,
                                           uint8_t* valid_lds, int tid) {
  const int key = tid >> 4, ch = tid & 15;
  *reinterpret_cast<uint4*>(k_lds + (key + 0) * kKRow + ch * 8) = r.k0;
  *reinterpret_cast<uint4*>(k_lds + (key + 16) * kKRow + ch * 8) = r.k1;
  *reinterpret_cast<uint4*>(k_lds + (key + 32) * kKRow + ch * 8) = r.k2;
  *reinterpret_cast<uint4*>(k_lds + (key + 48) * kKRow + ch * 8) = r.k3;
  if (ch == 0) {
    valid_lds[key + 0] = r.kvalid & 1u;
    valid_lds[key + 16] = (r.kvalid >> 1) & 1u;
    valid_lds[key + 32] = (r.kvalid >> 2) & 1u;
    valid_lds[key + 48] = (r.kvalid >> 3) & 1u;
  }
  const int p = tid & 31;
  store_vt_pair(vt_lds, tid >> 5, p, r.v0, r.v1);
  store_vt_pair(vt_lds, (tid >> 5) + 8, p, r.v2, r.v3);
}

template <int G>
__global__ void __launch_bounds__(kThreads, 2)
paged_prefill_kernel(PrefillArgs a) {
  constexpr int BM = kCols / G;   // query rows per workgroup
  __shared__ __attribute__((aligned(16))) uint16_t s_k[2][kKTile];
  __shared__ __attribute__((aligned(16))) uint16_t s_vt[2][kVTile];
  __shared__ uint8_t s_valid[2][kBN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hgrp = lane >> 5;   // which 8-element k group of the MFMA operands
  const int c32 = lane & 31;
  const int hq = a.num_kv_heads * G;

  // ---- work item: heaviest query tiles first ------------------------------
  const int npairs = a.num_seqs * a.num_kv_heads;
  const int ntiles = (a.max_seqlen_q + BM - 1) / BM;
  const int t = ntiles - 1 - static_cast<int>(blockIdx.x) / npairs;
  const int pr = static_cast<int>(blockIdx.x) % npairs;
  const int b = pr / a.num_kv_heads;
  const int g = pr % a.num_kv_heads;
  const int q0 = a.cu_seqlens_q[b];
  const int Lq = a.cu_seqlens_q[b + 1] - q0;
  const int Lk = a.cu_seqlens_k[b + 1] - a.cu_seqlens_k[b];
  const int P = Lk - Lq;
  const int qa = t * BM;
  if (Lq <= 0 || P < 0 || qa >= Lq || q0 < 0 || q0 + Lq > a.total_q) return;
  const int qb = min(qa + BM, Lq);
  const int W = a.sliding_window;
  const int pos_lo = P + qa, pos_hi = P + qb - 1;
  const int kstart = W > 0 ? max(0, pos_lo - W + 1) : 0;
  const int tile0 = kstart / kBN, tile1 = pos_hi / kBN;

  Walk w;
  w.Lk = Lk;
  w.block_size = a.block_size;
  w.inv_block_size = 1.0f / static_cast<float>(a.block_size);
  w.max_blocks = a.max_blocks_per_seq;
  w.num_blocks = a.num_blocks;
  w.lb0 = min(tile0 * kBN / a.block_size, a.max_blocks_per_seq - 1);
  {
    const int lb1 = min((tile1 * kBN + kBN - 1) / a.block_size, a.max_blocks_per_seq - 1);
    const int32_t* bt = a.block_tables + static_cast<int64_t>(b) * a.max_blocks_per_seq;
    for (int i = w.lb0 + tid; i <= lb1; i += kThreads) s_bt[i - w.lb0] = bt[i];
    __syncthreads();
  }

  // ---- this lane's query column -------------------------------------------
  const int col = wave * 32 + c32;
  const int hl = col / BM;
  const int qi = qa + col % BM;
  const bool qvalid = qi < Lq;
  const int qpos = P + qi;
  const int head = g * G + hl;
  // positions spanned by this wavefront's columns (for skipping masked sub-tiles)
  const int wq_lo = qa + (wave * 32) % BM;
  const int wq_hi = min(wq_lo + min(32, BM) - 1, Lq - 1);
  const int wpos_lo = P + wq_lo, wpos_hi = P + wq_hi;

  bf16x8_t qreg[8];
  {
    const uint4* qp = static_cast<const uint4*>(a.q) +
                      (static_cast<int64_t>(q0 + (qvalid ? qi : qa)) * hq + head) * 16 + hgrp;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) qreg[kk] = as_bf16x8(qp[2 * kk]);
  }

  f32x16_t o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mt][r] = 0.f;
  float m = -1.0e30f, lsum = 0.f;

  TileRegs regs = load_tile(a, w, tile0 * kBN, g, tid);
  store_tile(regs, s_k[0], s_vt[0], s_valid[0], tid);
  __syncthreads();

  for (int kt = tile0; kt <= tile1; ++kt) {
    const int buf = (kt - tile0) & 1;
    const bool more = kt < tile1;
    if (more) regs = load_tile(a, w, (kt + 1) * kBN, g, tid);

    const int kb = kt * kBN;
    const uint64_t vmask = __ballot(s_valid[buf][lane] != 0);
    const bool need_mask = (vmask != ~0ull) || (kb + kBN - 1 > pos_lo) ||
                           (W > 0 && kb < pos_hi - W + 1);
    const uint16_t* kl = s_k[buf];
    const uint16_t* vl = s_vt[buf];

    f32x16_t s[2];
    bool active[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int k0 = kb + sub * 32;
      active[sub] = k0 <= wpos_hi && k0 < Lk && !(W > 0 && k0 + 31 < wpos_lo - W + 1);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[sub][r] = 0.f;
      if (active[sub]) {
        const uint16_t* krow = kl + (sub * 32 + c32) * kKRow + hgrp * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const bf16x8_t kop = as_bf16x8(*reinterpret_cast<const uint4*>(krow + kk * 16));
          s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kk], s[sub], 0, 0, 0);
        }
      }
    }

    // online softmax over this lane's column (keys of the tile: 16 per sub-tile
    // in this lane, the other 16 in lane ^ 32)
    float mx = -INFINITY;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[sub][r] * a.scale_log2;
        if (!active[sub]) {
          x = -INFINITY;
        } else if (need_mask) {
          const int klocal = sub * 32 + (r >> 2) * 8 + hgrp * 4 + (r & 3);
          const int key = kb + klocal;
          const bool ok = ((vmask >> klocal) & 1ull) && key <= qpos && (W == 0 || qpos - key < W);
          x = ok ? x : -INFINITY;
        }
        s[sub][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    lsum *= alpha;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mt][r] *= alpha;

    // O^T += V^T . P^T, one 32-key sub-tile at a time.  In step ks2 the lane's
    // 8 key slots are keys 16*ks2 + 4*hgrp + {0..3} and 16*ks2 + 8 + 4*hgrp +
    // {0..3} of the sub-tile: accumulator registers 8*ks2 .. 8*ks2+7.
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      if (!active[sub]) continue;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        uint32_t w[4];
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          const float p0 = fast_exp2(s[sub][8 * ks2 + r] - mn);
          const float p1 = fast_exp2(s[sub][8 * ks2 + r + 1] - mn);
          lsum += p0 + p1;
          w[r >> 1] = pack_bf16x2(p0, p1);
        }
        const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        const int koff = sub * 32 + ks2 * 16 + hgrp * 4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint16_t* vrow = vl + (mt * 32 + c32) * kVRow + koff;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, o[mt], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(regs, s_k[buf ^ 1], s_vt[buf ^ 1], s_valid[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- normalise and write ---------------------------------------------------
  const float ltot = lsum + __shfl_xor(lsum, 32, kWave);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (qvalid) {
    uint16_t* orow = static_cast<uint16_t*>(a.out) +
                     (static_cast<int64_t>(q0 + qi) * hq + head) * kHeadDim;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int dim = mt * 32 + rg * 8 + hgrp * 4;
        const uint2 v = make_uint2(pack_bf16x2(o[mt][rg * 4] * inv, o[mt][rg * 4 + 1] * inv),
                                   pack_bf16x2(o[mt][rg * 4 + 2] * inv, o[mt][rg * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(orow + dim) = v;
      }
  }
}

template <int G>
hipError_t launch_group(const PrefillArgs& a, hipStream_t stream) {
  constexpr int BM = kCols / G;
  const int64_t ntiles = (a.max_seqlen_q + BM - 1) / BM;
  const int64_t grid = ntiles * a.num_seqs * a.num_kv_heads;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((paged_prefill_kernel<G>), dim3(static_cast<unsigned>(grid)), dim3(kThreads),
                     0, stream, a);
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
