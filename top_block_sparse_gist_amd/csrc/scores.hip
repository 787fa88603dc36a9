// A2: block scores.  For a selection unit u (its query rows times its query heads) and a
// block j with representative r_j:  s[u, j] = scale * mean_q (q . r_j) = scale * qbar_u . r_j.
// Page "开源大模型注意力机制演进" section 4, pseudo-code step 1 (coarse block importance);
// page "通过Gist Token的简化稀疏注意力", method, item 1 (the query scored against every
// historical gist token).
//
// Prefill: (1) pool_kernel streams Q once and writes qbar per unit (fp32);
//          (2) score_gemm_kernel forms qbar x R^T per (sequence, KV head) as a 64x64-tiled
//              fp32 product; tiles wholly after every unit's current block are skipped.
// Decode : score_decode_kernel pools the (<= 16) query vectors of each unit in LDS and
//          streams one 64-block tile of representatives per workgroup (HBM-bound GEMV).
// Only entries j <= c(u) are written.
#include "common.h"

namespace sas {

// ------------------------------------------------------------------------------------------
// query pooling (prefill)
// ------------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(SeqTable st, const T *__restrict__ Q, int64_t qb,
                                                   int64_t qh, int64_t qt, int tq, int blk, int S,
                                                   int QB, int G, int per_head,
                                                   float *__restrict__ qbar) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int TPR = D / VEC;
  constexpr int RPP = 256 / TPR;
  __shared__ float part[RPP][D + 1];
  const int i = blockIdx.x, s = blockIdx.y, b = blockIdx.z;
  const int q0 = st.q0[b];
  const int c = q0 / blk + i;
  const int t_lo = max(0, c * blk - q0);
  const int t_hi = min(tq, (c + 1) * blk - q0);
  if (t_lo >= t_hi) return;
  const int rows = t_hi - t_lo;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : s * G;
  const int nvec = rows * nh;
  const int tid = threadIdx.x;
  const int cc = tid % TPR, r = tid / TPR;
  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  for (int v0 = 0; v0 < nvec; v0 += 4 * RPP) {
    u32x4 raw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int v = v0 + w * RPP + r;
      if (v < nvec) {
        int h = h0 + v / rows, t = t_lo + v % rows;
        raw[w] = *reinterpret_cast<const u32x4 *>(Q + b * qb + h * qh + (int64_t)t * qt + cc * VEC);
      } else {
        raw[w] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          acc[2 * x] += bf16_lo(raw[w][x]);
          acc[2 * x + 1] += bf16_hi(raw[w][x]);
        }
      } else {
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[x] += __uint_as_float(raw[w][x]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[r][cc * VEC + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < RPP; ++q) sum += part[q][tid];
    const int64_t u = ((int64_t)b * S + s) * QB + i;
    qbar[u * D + tid] = sum / (float)nvec;
  }
}

// ------------------------------------------------------------------------------------------
// qbar x R^T, 64 units x 64 blocks per workgroup, fp32 FMA (4x4 outputs per lane)
// ------------------------------------------------------------------------------------------
template <typename R, int D>
__global__ __launch_bounds__(256) void score_gemm_kernel(SeqTable st, const float *__restrict__ qbar,
                                                         const R *__restrict__ reps, int64_t rb,
                                                         int64_t rh, int64_t rj, int gist, int tq,
                                                         int blk, int S, int QB, int G, int per_head,
                                                         int hkv, float scale,
                                                         float *__restrict__ scores, int64_t ld) {
  constexpr int KC = 32;  // d chunk
  __shared__ float As[KC][64 + 4];
  __shared__ float Bs[KC][64 + 4];
  const int b = blockIdx.z / hkv, g = blockIdx.z % hkv;
  const int L = st.len[b];
  const int q0 = st.q0[b];
  const int c0 = q0 / blk;
  const int nqb = (q0 + tq - 1) / blk - c0 + 1;
  const int nU = per_head ? G : 1;
  const int M = nU * nqb;
  const int m0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  if (m0 >= M) return;
  // largest current block among this tile's units
  int cmax = 0;
  {
    int mlast = min(M, m0 + 64) - 1;
    int ilo = m0 % nqb, ihi = mlast % nqb;
    cmax = (mlast / nqb != m0 / nqb) ? c0 + nqb - 1 : c0 + max(ilo, ihi);
  }
  if (j0 > cmax) return;
  const int nrep = gist ? L / blk : cdiv(L, blk);
  const int tid = threadIdx.x;
  // wave w owns the 32 x 32 output block (units mw.., blocks nw..) of the 64 x 64 tile, formed with
  // v_mfma_f32_32x32x2_f32: lane l supplies A[unit mw + l % 32][dim k + l / 32] and
  // B[dim k + l / 32][block nw + l % 32]; register r of its result is unit mw + 8 (r / 4) + 4 (l / 32)
  // + r % 4, block nw + l % 32.  A wave whose units all lie past M skips the products.
  const int wave = tid >> 6, lane = tid & 63;
  const int mw = 32 * (wave >> 1), nw = 32 * (wave & 1);
  const bool wave_live = m0 + mw < M;

  auto unit_row = [&](int m) -> int64_t {
    int sl = m / nqb, i = m % nqb;
    int s = per_head ? g * G + sl : g;
    return ((int64_t)b * S + s) * QB + i;
  };

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  // the next d chunk's global loads are issued into registers before this chunk's products, so
  // they fly during them (each product still sums its d terms in order 0..D-1)
  const R *rbase = reps + b * rb + g * rh;
  auto load_a = [&](int k0, f32x4 (&ra)[2]) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int e = tid + w * 256;  // 64 units x 8 float4
      const int m = m0 + e / 8, kq = (e % 8) * 4;
      ra[w] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (m < M) ra[w] = *reinterpret_cast<const f32x4 *>(qbar + unit_row(m) * D + k0 + kq);
    }
  };
  auto load_b = [&](int k0, u32x4 (&rv)[2]) {
    if constexpr (sizeof(R) == 4) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int e = tid + w * 256;  // 64 reps x 8 float4
        const int j = j0 + e / 8, kq = (e % 8) * 4;
        rv[w] = u32x4{0u, 0u, 0u, 0u};
        if (j < nrep) rv[w] = *reinterpret_cast<const u32x4 *>(rbase + (int64_t)j * rj + k0 + kq);
      }
    } else {
      const int j = j0 + tid / 4, kq = (tid % 4) * 8;  // 64 reps x 4 chunks of 8 bf16
      rv[0] = u32x4{0u, 0u, 0u, 0u};
      if (j < nrep) rv[0] = *reinterpret_cast<const u32x4 *>(rbase + (int64_t)j * rj + k0 + kq);
    }
  };
  f32x4 ra[2];
  u32x4 rv[2];
  load_a(0, ra);
  load_b(0, rv);
  for (int k0 = 0; k0 < D; k0 += KC) {
    // A tile: 64 units x 32 dims; B tile: 64 reps x 32 dims (transposed into LDS)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int e = tid + w * 256;
      const int mm = e / 8, kq = (e % 8) * 4;
#pragma unroll
      for (int x = 0; x < 4; ++x) As[kq + x][mm] = ra[w][x];
    }
    if constexpr (sizeof(R) == 4) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int e = tid + w * 256;
        const int jj = e / 8, kq = (e % 8) * 4;
#pragma unroll
        for (int x = 0; x < 4; ++x) Bs[kq + x][jj] = __uint_as_float(rv[w][x]);
      }
    } else {
      const int jj = tid / 4, kq = (tid % 4) * 8;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        Bs[kq + 2 * x][jj] = bf16_lo(rv[0][x]);
        Bs[kq + 2 * x + 1][jj] = bf16_hi(rv[0][x]);
      }
    }
    __syncthreads();
    if (k0 + KC < D) {
      load_a(k0 + KC, ra);
      load_b(k0 + KC, rv);
    }
    if (wave_live) {
#pragma unroll
      for (int k = 0; k < KC; k += 2) {
        const float a = As[k + (lane >> 5)][mw + (lane & 31)];
        const float bb = Bs[k + (lane >> 5)][nw + (lane & 31)];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bb, acc, 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!wave_live) return;
  const int j = j0 + nw + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + mw + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (m >= M) continue;
    const int c = c0 + m % nqb;
    // gist keys exist for the complete chunks before the current one only
    const int have = gist ? min(nrep, c) : nrep;
    if (j <= c) scores[unit_row(m) * ld + j] = (j < have) ? acc[r] * scale : -INFINITY;
  }
}

// ------------------------------------------------------------------------------------------
// decode: one 64-block tile of representatives per workgroup, all units of one KV head
// ------------------------------------------------------------------------------------------
template <typename T, typename R, int D>
__global__ __launch_bounds__(256) void score_decode_kernel(SeqTable st, const T *__restrict__ Q,
                                                           int64_t qb, int64_t qh,
                                                           const R *__restrict__ reps, int64_t rb,
                                                           int64_t rh, int64_t rj, int gist, int blk,
                                                           int S, int G, int per_head, float scale,
                                                           float *__restrict__ scores, int64_t ld) {
  constexpr int VEC = 16 / sizeof(R);  // rep elements per 16-byte load
  constexpr int TPR = D / VEC;         // lanes per rep row (16 or 32: within one wave)
  constexpr int RPP = 256 / TPR;
  constexpr int PASSES = 64 / RPP;
  __shared__ float qs[16][D];
  const int j0 = blockIdx.x * 64, g = blockIdx.y, b = blockIdx.z;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  if (j0 > c) return;
  // gist keys exist for the complete chunks before the current one only
  const int nrep = gist ? min(L / blk, c) : cdiv(L, blk);
  const int nU = per_head ? G : 1;
  const int tid = threadIdx.x;
  // pooled query per unit
  for (int e = tid; e < nU * D; e += 256) {
    int u = e / D, k = e % D;
    float v;
    if (per_head) {
      const T *q = Q + b * qb + (int64_t)(g * G + u) * qh + k;
      v = sizeof(T) == 2 ? bf16_to_f32(*(const uint16_t *)q) : *(const float *)q;
    } else {
      float sum = 0.f;
      for (int h = 0; h < G; ++h) {
        const T *q = Q + b * qb + (int64_t)(g * G + h) * qh + k;
        sum += sizeof(T) == 2 ? bf16_to_f32(*(const uint16_t *)q) : *(const float *)q;
      }
      v = sum / (float)G;
    }
    qs[u][k] = v;
  }
  __syncthreads();
  const int cc = tid % TPR, r = tid / TPR;
  const R *rbase = reps + b * rb + g * rh + cc * VEC;
  u32x4 raw[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    int j = j0 + r + ps * RPP;
    if (j <= c && j < nrep) raw[ps] = *reinterpret_cast<const u32x4 *>(rbase + (int64_t)j * rj);
    else raw[ps] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = j0 + r + ps * RPP;
    float rv[VEC];
    if constexpr (sizeof(R) == 2) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        rv[2 * x] = bf16_lo(raw[ps][x]);
        rv[2 * x + 1] = bf16_hi(raw[ps][x]);
      }
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x) rv[x] = __uint_as_float(raw[ps][x]);
    }
    for (int u = 0; u < nU; ++u) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) part = fmaf(qs[u][cc * VEC + e], rv[e], part);
      part = group_sum<TPR>(part);
      if (cc == 0 && j <= c) {
        int s = per_head ? g * G + u : g;
        scores[((int64_t)b * S + s) * ld + j] = (j < nrep) ? part * scale : -INFINITY;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------------
template <typename T, int D>
static hipError_t pool_dispatch(const sas_problem &p, const SeqTable &st, const void *Q,
                                const int64_t *qs, int32_t tq, int32_t sel_mode, float *qbar,
                                hipStream_t s) {
  const int QB = num_qblocks(tq, p.block);
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  dim3 grid(QB, S, p.batch);
  hipLaunchKernelGGL((pool_kernel<T, D>), grid, dim3(256), 0, s, st, (const T *)Q, qs[0], qs[1], qs[2],
                     tq, p.block, S, QB, p.hq / p.hkv, per_head, qbar);
  return hipGetLastError();
}

hipError_t launch_pool_queries(const sas_problem &p, const SeqTable &st, const void *Q,
                               const int64_t *qs, int32_t tq, int32_t sel_mode, float *qbar,
                               hipStream_t s) {
  if (p.dtype == SAS_BF16)
    return p.head_dim == 128 ? pool_dispatch<uint16_t, 128>(p, st, Q, qs, tq, sel_mode, qbar, s)
                             : pool_dispatch<uint16_t, 64>(p, st, Q, qs, tq, sel_mode, qbar, s);
  return p.head_dim == 128 ? pool_dispatch<float, 128>(p, st, Q, qs, tq, sel_mode, qbar, s)
                           : pool_dispatch<float, 64>(p, st, Q, qs, tq, sel_mode, qbar, s);
}

template <typename R, int D>
static hipError_t gemm_dispatch(const sas_problem &p, const SeqTable &st, const float *qbar,
                                int32_t tq, const void *reps, int gist, const int64_t *rs,
                                int32_t sel_mode, float scale, float *scores, int64_t ld,
                                hipStream_t s) {
  const int QB = num_qblocks(tq, p.block);
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  const int G = p.hq / p.hkv;
  int nbmax = 0;
  for (int b = 0; b < p.batch; ++b) nbmax = max(nbmax, cdiv(st.len[b], p.block));
  const int M = (per_head ? G : 1) * QB;
  dim3 grid(cdiv(nbmax, 64), cdiv(M, 64), p.batch * p.hkv);
  hipLaunchKernelGGL((score_gemm_kernel<R, D>), grid, dim3(256), 0, s, st, qbar, (const R *)reps, rs[0],
                     rs[1], rs[2], gist, tq, p.block, S, QB, G, per_head, p.hkv, scale, scores, ld);
  return hipGetLastError();
}

hipError_t launch_scores_prefill(const sas_problem &p, const SeqTable &st, const float *qbar,
                                 int32_t tq, const void *reps, int32_t reps_kind, const int64_t *rs,
                                 int32_t sel_mode, float scale, float *scores, int64_t ld,
                                 hipStream_t s) {
  const int gist = reps_kind == SAS_REPS_GIST;
  const bool rbf16 = gist && p.dtype == SAS_BF16;
  if (rbf16)
    return p.head_dim == 128
               ? gemm_dispatch<uint16_t, 128>(p, st, qbar, tq, reps, gist, rs, sel_mode, scale, scores, ld, s)
               : gemm_dispatch<uint16_t, 64>(p, st, qbar, tq, reps, gist, rs, sel_mode, scale, scores, ld, s);
  return p.head_dim == 128
             ? gemm_dispatch<float, 128>(p, st, qbar, tq, reps, gist, rs, sel_mode, scale, scores, ld, s)
             : gemm_dispatch<float, 64>(p, st, qbar, tq, reps, gist, rs, sel_mode, scale, scores, ld, s);
}

template <typename T, typename R, int D>
static hipError_t dec_dispatch(const sas_problem &p, const SeqTable &st, const void *Q,
                               const int64_t *qs, const void *reps, int gist, const int64_t *rs,
                               int32_t sel_mode, float scale, float *scores, int64_t ld,
                               hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  int nbmax = 0;
  for (int b = 0; b < p.batch; ++b) nbmax = max(nbmax, cdiv(st.len[b], p.block));
  dim3 grid(cdiv(nbmax, 64), p.hkv, p.batch);
  hipLaunchKernelGGL((score_decode_kernel<T, R, D>), grid, dim3(256), 0, s, st, (const T *)Q, qs[0], qs[1],
                     (const R *)reps, rs[0], rs[1], rs[2], gist, p.block, S, p.hq / p.hkv, per_head,
                     scale, scores, ld);
  return hipGetLastError();
}

hipError_t launch_scores_decode(const sas_problem &p, const SeqTable &st, const void *Q,
                                const int64_t *qs, const void *reps, int32_t reps_kind,
                                const int64_t *rs, int32_t sel_mode, float scale, float *scores,
                                int64_t ld, hipStream_t s) {
  const int gist = reps_kind == SAS_REPS_GIST;
  if (p.dtype == SAS_BF16) {
    if (gist)
      return p.head_dim == 128
                 ? dec_dispatch<uint16_t, uint16_t, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s)
                 : dec_dispatch<uint16_t, uint16_t, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s);
    return p.head_dim == 128
               ? dec_dispatch<uint16_t, float, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s)
               : dec_dispatch<uint16_t, float, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s);
  }
  return p.head_dim == 128
             ? dec_dispatch<float, float, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s)
             : dec_dispatch<float, float, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, s);
}

}  // namespace sas
