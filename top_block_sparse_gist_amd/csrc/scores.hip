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
#include <algorithm>

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
// qbar x R^T per (sequence, KV head), fp32 on v_mfma_f32_32x32x2_f32.
// Work items are (sequence, KV head, range of 128 blocks, chunk of 32 units), in that order.  The
// grid is one workgroup per resident slot, and workgroup k takes an equal contiguous run of the
// items (XCD x holds the x-th eighth of them, so a pair's units stay in one L2).  A workgroup has
// four waves; wave w keeps the representatives of blocks 32w.. of the current range in registers
// (the B operand, reloaded when the run moves to the next range) and forms their scores against
// the chunk's units.  The units' qbar rows stream through LDS: the next item's chunk is copied
// HBM -> LDS by the buffer unit while this one is multiplied (two buffers, one barrier per item),
// and an item's scores are stored during the next item, so no wait covers a store.  The d index of
// each MFMA is permuted so that a lane reads 4 consecutive elements with one 16-byte load (B from
// global memory, A from LDS): MFMA 4a + e takes, in k-slot s = lane / 32, element 8a + 4s + e of
// both operands.  A score is a sum of d products in an order fixed by that permutation; the
// oracle's bound (1e-5 relative to the largest score) holds for any order.  LDS rows are stored
// unpadded with their 16-byte chunks XOR-swizzled by (row & 7), so the A reads of 8 consecutive
// rows at one logical chunk fall on distinct banks.
// ------------------------------------------------------------------------------------------
constexpr int SCORE_UNITS = 32;                  // units per chunk
constexpr int SCORE_WAVES = 4;                   // waves per workgroup, 32 blocks each
constexpr int SCORE_RANGE = 32 * SCORE_WAVES;    // blocks per range

// first item of each sequence (over its KV heads, ranges and chunks); off[batch] = all items
struct ScoreItems {
  int32_t off[SAS_MAX_BATCH + 1];
};

template <typename R, int D>
__global__ __launch_bounds__(64 * SCORE_WAVES, 3) void score_gemm_kernel(SeqTable st, ScoreItems items, const float *__restrict__ qbar,
                                                            uint32_t qbar_bytes, const R *__restrict__ reps,
                                                            int64_t rb, int64_t rh, int64_t rj, int gist,
                                                            int tq, int blk, int S, int QB, int G, int per_head,
                                                            int hkv, int batch, float scale,
                                                            float *__restrict__ scores, int64_t ld) {
  constexpr int CPR = D / 4;                             // 16-byte chunks per qbar row
  constexpr int NCP = SCORE_UNITS * D * 4 / 1024 / SCORE_WAVES;  // 1 KiB copies per wave per chunk
  static_assert(NCP >= 1, "each wave copies whole KiB");
  __shared__ __attribute__((aligned(16))) float abuf[2][SCORE_UNITS * D];
  __shared__ int64_t trow[3][SCORE_UNITS];  // score row of each unit of an item's chunk (three slots)
  __shared__ int32_t tcur[3][SCORE_UNITS];  // its current block (-1: no unit)
  // this workgroup's run of items: XCD x = n % 8 takes the x-th eighth
  const int per = gridDim.x >> 3;
  const int run = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int T = items.off[batch];
  const int it1 = (int)((int64_t)(run + 1) * T / gridDim.x);
  int it = (int)((int64_t)run * T / gridDim.x);
  const int nU = per_head ? G : 1;

  struct Item {
    int it, b, g, r, ch, c0, nqb, M, nrep, j0, cmax;
  };
  // item geometry; cmax: the largest current block among the chunk's units (the item is dead when
  // it is below the range's first block)
  auto geo = [&](int x) {
    Item a;
    a.it = x;
    int b = 0;
    while (items.off[b + 1] <= x) ++b;
    const int q0 = st.q0[b];
    a.b = b;
    a.c0 = q0 / blk;
    a.nqb = (q0 + tq - 1) / blk - a.c0 + 1;
    a.M = nU * a.nqb;
    a.nrep = gist ? st.len[b] / blk : cdiv(st.len[b], blk);
    const int nr = (a.c0 + a.nqb - 1) / SCORE_RANGE + 1, nch = cdiv(a.M, SCORE_UNITS);
    int rem = x - items.off[b];
    a.g = rem / (nr * nch);
    rem -= a.g * nr * nch;
    a.r = rem / nch;
    a.ch = rem - a.r * nch;
    a.j0 = a.r * SCORE_RANGE;
    const int lo = a.ch * SCORE_UNITS, last = min(a.M, lo + SCORE_UNITS) - 1;
    a.cmax = (last / a.nqb != lo / a.nqb) ? a.c0 + a.nqb - 1 : a.c0 + max(lo % a.nqb, last % a.nqb);
    return a;
  };
  auto next_live = [&](int x) {
    Item a;
    a.it = -1;
    for (; x < it1; ++x) {
      a = geo(x);
      if (a.cmax >= a.j0) return a;
    }
    a.it = -1;
    return a;
  };
  Item cur = next_live(it);
  if (cur.it < 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = lane >> 5, l32 = lane & 31;
  // qbar through a range-checked buffer resource: a unit past M reads zeros
  const i32x4 qrs = lds_rsrc(qbar, qbar_bytes);
  // table slot `slot` and LDS buffer `buf` take item a's chunk: lane l32 forms unit 32 ch + l32's
  // row; the copy lanes fetch their rows' chunks from it (the LDS chunk (row, cl) holds qbar
  // chunk cl ^ (row & 7))
  auto prep = [&](const Item &a, int slot, int buf) {
    const int m = a.ch * SCORE_UNITS + l32;
    const bool ok = m < a.M;
    int64_t ur = 0;
    if (ok) {
      const int sl = m / a.nqb, i = m - sl * a.nqb;
      const int sh = per_head ? a.g * G + sl : a.g;
      ur = ((int64_t)a.b * S + sh) * QB + i;
    }
    if (wave == 0 && ks == 0) {
      trow[slot][l32] = ur;
      tcur[slot][l32] = ok ? a.c0 + m % a.nqb : -1;
    }
    // a unit past M reads at the end of qbar: out of range, zeros
    const uint32_t boff = ok ? (uint32_t)(ur * (D * 4)) : qbar_bytes;
#pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int e = (wave * NCP + i) * 64 + lane;
      const int row = e / CPR, cl = e % CPR;
      const uint32_t voff = (uint32_t)__shfl((int)boff, row, 64) + 16u * (cl ^ (row & 7));
      buf_load_lds<16>(qrs, lds_base(abuf) + 4u * (buf * SCORE_UNITS * D + (wave * NCP + i) * 256), voff, 0u);
    }
  };
  // B operand of item a's range: bf[4a + e] = rep[j0 + 32 wave + l32][8a + 4 ks + e] (0 past the
  // representatives)
  float bf[D / 2];
  auto load_b = [&](const Item &a) {
    const int j = a.j0 + 32 * wave + l32;
    const bool ok = j < a.nrep;
    const R *rrow = reps + a.b * rb + a.g * rh + (ok ? (int64_t)j * rj : 0) + 4 * ks;
#pragma unroll
    for (int x = 0; x < D / 8; ++x) {
      if constexpr (sizeof(R) == 4) {
        const f32x4 v = ok ? *reinterpret_cast<const f32x4 *>(rrow + 8 * x) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) bf[4 * x + e] = v[e];
      } else {
        const u32x2 v = ok ? *reinterpret_cast<const u32x2 *>(rrow + 8 * x) : u32x2{0u, 0u};
        bf[4 * x + 0] = bf16_lo(v[0]);
        bf[4 * x + 1] = bf16_hi(v[0]);
        bf[4 * x + 2] = bf16_lo(v[1]);
        bf[4 * x + 3] = bf16_hi(v[1]);
      }
    }
  };
  prep(cur, 0, 0);
  load_b(cur);

  // scores of the item whose chunk is in table slot `slot` (lane: block j, units 8 (r / 4) + 4 ks +
  // r % 4 of the chunk)
  auto store = [&](const f32x16 &acc, int slot, int j, int nrep) {
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int ml = 8 * (rr >> 2) + 4 * ks + (rr & 3);
      const int c = tcur[slot][ml];
      // gist keys exist for the complete chunks before the current one only
      const int have = gist ? min(nrep, c) : nrep;
      if (j <= c) scores[trow[slot][ml] * ld + j] = (j < have) ? acc[rr] * scale : -INFINITY;
    }
  };
  f32x16 pacc;
  int pslot = -1, pj = 0, pnrep = 0;
  for (int k = 0; cur.it >= 0; ++k) {
    const int buf = k & 1, slot = k % 3;
    wait_vmcnt<0>();
    __syncthreads();  // the item's chunk and B are in place; the other buffer and the oldest slot are free
    const Item nx = next_live(cur.it + 1);
    if (nx.it >= 0) prep(nx, (k + 1) % 3, buf ^ 1);
    if (pslot >= 0) store(pacc, pslot, pj, pnrep);
    pslot = -1;
    const int js = cur.j0 + 32 * wave;
    if (js <= cur.cmax) {  // some unit of the chunk reaches this wave's blocks
      f32x16 acc;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) acc[rr] = 0.f;
      const float *arow = &abuf[buf][l32 * D];
      const int sw = l32 & 7;
#pragma unroll
      for (int x = 0; x < D / 8; ++x) {
        const f32x4 av = *reinterpret_cast<const f32x4 *>(arow + 4 * ((2 * x + ks) ^ sw));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], bf[4 * x + e], acc, 0, 0, 0);
      }
      pacc = acc;
      pslot = slot;
      pj = js + l32;
      pnrep = cur.nrep;
    }
    // the next item's range: its representatives replace these (in flight until the next barrier)
    if (nx.it >= 0 && (nx.b != cur.b || nx.g != cur.g || nx.r != cur.r)) load_b(nx);
    cur = nx;
  }
  if (pslot >= 0) store(pacc, pslot, pj, pnrep);
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

// resident workgroup slots of the score product on the current device (four per CU: 34 KB of LDS and
// 128 VGPRs each)
static int score_slots() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = 4 * cus;
  }
  return cached[dev];
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
  const int nU = per_head ? G : 1;
  // items per sequence: KV heads x ranges of 128 blocks (up to the last unit's current block) x
  // chunks of 32 units
  ScoreItems items{};
  int64_t T = 0;
  for (int b = 0; b < p.batch; ++b) {
    const int q0 = st.q0[b], c0 = q0 / p.block;
    const int nqb = (q0 + tq - 1) / p.block - c0 + 1;
    const int nr = (c0 + nqb - 1) / SCORE_RANGE + 1;
    items.off[b] = (int32_t)T;
    T += (int64_t)p.hkv * nr * cdiv(nU * nqb, SCORE_UNITS);
  }
  if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
  items.off[p.batch] = (int32_t)T;
  // one workgroup per slot (a multiple of 8: the eighths of the item list go to the 8 XCDs)
  const int64_t nwg = std::min<int64_t>(8 * cdiv64(T, 8), 8 * (score_slots() / 8));
  const uint32_t qbar_bytes = (uint32_t)((int64_t)p.batch * S * QB * D * 4);
  hipLaunchKernelGGL((score_gemm_kernel<R, D>), dim3((unsigned)nwg), dim3(64 * SCORE_WAVES), 0, s, st, items, qbar, qbar_bytes,
                     (const R *)reps, rs[0], rs[1], rs[2], gist, tq, p.block, S, QB, G, per_head, p.hkv, p.batch,
                     scale, scores, ld);
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
