// A1: block representatives = mean of the present keys of every block.
// Page "稀疏注意力的Trade-offs" section 2.1 (block-pooled token representations) and page
// "开源大模型注意力机制演进" section 4, pseudo-code step 1 (keys aggregated per block).
//
// HBM-streaming reduction: one workgroup per (block, KV head, sequence).  The incremental form
// (decode: only the blocks from a given one on, normally the block the new tokens landed in)
// runs the same workgroups on fewer blocks, so its results equal a full pass bit for bit.  The workgroup's
// 256 lanes read the block's blk x d slab with 16-byte loads (a key row is covered by
// d/VEC consecutive lanes, so every load instruction reads whole rows), all loads of the
// block are issued before the first add, partial row sums are folded through LDS, and the
// d fp32 means are written once.
#include "common.h"

namespace sas {

// First block computed per sequence (grid x counts blocks from it); current: the one block that holds
// position L_b - 1, found on the device (lengths in device memory).
struct BlockStart {
  int32_t j[SAS_MAX_BATCH];
  int32_t current;
};

template <typename T, int D, int BLK>
__global__ __launch_bounds__(256) void reps_kernel(SeqTable st, BlockStart start, const T *__restrict__ K, int64_t kb,
                                                   int64_t kh, int64_t kt, float *__restrict__ reps,
                                                   int64_t rb, int64_t rh, int64_t rj,
                                                   const int32_t *__restrict__ table, int64_t tld) {
  constexpr int VEC = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int TPR = D / VEC;             // lanes per key row
  constexpr int RPP = 256 / TPR;           // rows per pass
  constexpr int PASSES = BLK / RPP;
  static_assert(BLK % RPP == 0, "block must be a multiple of rows per pass");
  __shared__ float part[RPP][D + 1];

  const int g = blockIdx.y, b = blockIdx.z;
  const int L = seq_len(st, b);
  // current-block mode (lengths in device memory): the block that holds position L - 1
  const int j = (start.current ? (L - 1) / BLK : start.j[b]) + (int)blockIdx.x;
  const int t0 = j * BLK;
  if (t0 >= L) return;
  const int n = min(BLK, L - t0);
  const int tid = threadIdx.x;
  const int c = tid % TPR, r = tid / TPR;
  // paged K (table != nullptr): block j is page table[b * tld + j], kb its stride
  const T *base = table ? K + (int64_t)table[b * tld + j] * kb + g * kh + c * VEC
                        : K + b * kb + g * kh + (int64_t)t0 * kt + c * VEC;

  u32x4 raw[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    int row = r + ps * RPP;
    if (row < n) raw[ps] = *reinterpret_cast<const u32x4 *>(base + (int64_t)row * kt);
    else raw[ps] = u32x4{0u, 0u, 0u, 0u};
  }
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += bf16_lo(raw[ps][w]);
        acc[2 * w + 1] += bf16_hi(raw[ps][w]);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[ps][w]);
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[r][c * VEC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < RPP; ++q) s += part[q][tid];
    reps[b * rb + g * rh + (int64_t)j * rj + tid] = s / (float)n;
  }
}

template <typename T, int D>
static hipError_t reps_dispatch_blk(const sas_problem &p, const SeqTable &st, const void *K,
                                    const int64_t *ks, float *reps, const int64_t *rs, const int32_t *first,
                                    hipStream_t s, const int32_t *table, int64_t tld, bool current) {
  BlockStart start{};
  int nbmax = 0;
  if (current) {
    start.current = 1;
    nbmax = 1;
  } else {
    for (int b = 0; b < p.batch; ++b) {
      start.j[b] = first ? first[b] : 0;
      nbmax = max(nbmax, cdiv(st.len[b], p.block) - start.j[b]);
    }
  }
  if (nbmax <= 0) return hipSuccess;  // nothing to compute
  dim3 grid(nbmax, p.hkv, p.batch);
  if (p.block == 64)
    hipLaunchKernelGGL((reps_kernel<T, D, 64>), grid, dim3(256), 0, s, st, start, (const T *)K, ks[0], ks[1],
                       ks[2], reps, rs[0], rs[1], rs[2], table, tld);
  else
    hipLaunchKernelGGL((reps_kernel<T, D, 128>), grid, dim3(256), 0, s, st, start, (const T *)K, ks[0], ks[1],
                       ks[2], reps, rs[0], rs[1], rs[2], table, tld);
  return hipGetLastError();
}

hipError_t launch_reps(const sas_problem &p, const SeqTable &st, const void *K, const int64_t *ks,
                       float *reps, const int64_t *rs, const int32_t *first, hipStream_t s, const int32_t *table,
                       int64_t tld, bool current) {
  if (p.dtype == SAS_BF16) {
    if (p.head_dim == 128)
      return reps_dispatch_blk<uint16_t, 128>(p, st, K, ks, reps, rs, first, s, table, tld, current);
    return reps_dispatch_blk<uint16_t, 64>(p, st, K, ks, reps, rs, first, s, table, tld, current);
  }
  if (p.head_dim == 128) return reps_dispatch_blk<float, 128>(p, st, K, ks, reps, rs, first, s, table, tld, current);
  return reps_dispatch_blk<float, 64>(p, st, K, ks, reps, rs, first, s, table, tld, current);
}

}  // namespace sas
