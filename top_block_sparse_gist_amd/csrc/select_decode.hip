// A2 + A3 fused for decode: block scores and the per-unit top-k (+ forced blocks, + gate) in
// one launch.  Same results as sas_block_scores followed by sas_topk_select.
// Page "开源大模型注意力机制演进" section 4 pseudo-code steps 1-2 (coarse block scores, then
// top-k over them); page "SAS: 通过端到端优化上下文排序的简单注意力稀疏化", method (hard top-k
// at inference, the current block always kept, log-gate over the kept set); page
// "通过Gist Token的简化稀疏注意力", method item 1 (the query scored against the gist tokens).
//
// Workgroup = one 64-block tile of representatives of one (sequence, KV head): the tile's
// 16-byte loads are issued first, then the unit queries are pooled in LDS, then the scores
// are formed with a shuffle reduction and written.  The last workgroup to finish a
// (sequence, KV head) -- found with one device-scope atomic on an arrival counter, which it
// resets to zero -- runs the top-k of that KV head's units, one wave per unit: the unit's
// scores are loaded once into registers, an MSB-first radix select (4 passes of 8 bits,
// per-wave LDS histogram, shuffle scan) finds the k-th largest key, and a ballot/popcount
// compaction writes the selected blocks in ascending order (ties go to the lower block).
#include "common.h"

namespace sas {

template <int NPL>
__device__ void wave_topk(const float *__restrict__ row, int c, bool sinkf, const Budget &bg, int kcap,
                          int32_t *__restrict__ out, int32_t *__restrict__ nsel_out, float *__restrict__ gout,
                          uint32_t *hist) {
  const int lane = threadIdx.x & 63;
  const bool sink = sinkf && c > 0;
  const int lo = sink ? 1 : 0;
  const int ncand = c - lo;
  const int k = budget_k(bg, c, ncand);
  const int base = sink ? 1 : 0;
  uint32_t key[NPL];
  float sv[NPL];
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    const int j = lane + 64 * r;
    sv[r] = (j < c) ? load_dev(row + j) : -INFINITY;
    key[r] = (j >= lo && j < c) ? float_order_key(sv[r]) : 0u;
  }
  const float s_c = load_dev(row + c);
  const float s_0 = load_dev(row);
  uint32_t T = 0u, want = 0u;
  bool all = k >= ncand;
  if (!all && k > 0) {
    want = (uint32_t)k;
    if constexpr (NPL <= 8) {
      // MSB-first, one bit per step, counted with ballots (no LDS): among the keys that match the
      // prefix, count those with the next bit set; if they hold the wanted rank the bit is set,
      // else they are all taken and the rank moves past them.  Stops once the keys at or above
      // the prefix are exactly the ones still wanted.
      uint32_t prefix = 0u;
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t m = ~0u << bit, target = prefix | (1u << bit);
        uint32_t cnt = 0;
#pragma unroll
        for (int r = 0; r < NPL; ++r) cnt += (uint32_t)__popcll(__ballot((key[r] & m) == target));
        if (cnt >= want) {
          prefix = target;
          if (cnt == want) break;
        } else {
          want -= cnt;
        }
      }
      T = prefix;
    } else {
      uint32_t prefix = 0u, pmask = 0u;
      for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int q = 0; q < 16; ++q) hist[lane * 16 + q] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        uint32_t *hc = hist + 256 * (lane >> 4);  // this 16-lane group's copy
#pragma unroll
        for (int r = 0; r < NPL; ++r) {
          const int j = lane + 64 * r;
          if (j >= lo && j < c && (key[r] & pmask) == prefix) atomicAdd(&hc[(key[r] >> shift) & 255u], 1u);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        uint32_t cnt[4], tot = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int bin = 255 - 4 * lane - q;
          cnt[q] = hist[bin] + hist[256 + bin] + hist[512 + bin] + hist[768 + bin];
          tot += cnt[q];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t v = __shfl_up(incl, o, 64);
          if (lane >= o) incl += v;
        }
        const uint32_t excl = incl - tot;
        int dsel = -1;
        uint32_t above = 0;
        if (excl < want && want <= incl) {
          uint32_t run = excl;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (dsel < 0 && run + cnt[q] >= want) {
              dsel = 255 - 4 * lane - q;
              above = run;
            }
            run += cnt[q];
          }
        }
        // broadcast from the lane that found the digit
        const uint64_t bal = __ballot(dsel >= 0);
        const int src = __ffsll((unsigned long long)bal) - 1;
        dsel = __shfl(dsel, src, 64);
        above = __shfl(above, src, 64);
        want -= above;
        prefix |= ((uint32_t)dsel) << shift;
        pmask |= 255u << shift;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      }
      T = prefix;
    }
  }
  // which candidates are kept (bit r of `selbits`: block lane + 64r)
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t selbits = 0ull;
  uint32_t eq_seen = 0;
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    const int j = lane + 64 * r;
    const bool cand = j >= lo && j < c;
    bool sel;
    if (all) {
      sel = cand;
    } else if (k == 0) {
      sel = false;
    } else {
      const bool gt = cand && key[r] > T;
      const bool eq = cand && key[r] == T;
      const uint64_t eb = __ballot(eq);
      const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eb & below);
      eq_seen += (uint32_t)__popcll(eb);
      sel = gt || (eq && eq_rank < want);
    }
    selbits |= (uint64_t)sel << r;
  }
  // log-gate: g_j = s_j - logsumexp over the selected set (forced blocks included)
  float lse = 0.f;
  if (gout) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < NPL; ++r)
      if ((selbits >> r) & 1ull) mx = fmaxf(mx, sv[r]);
    mx = fmaxf(mx, s_c);
    if (sink) mx = fmaxf(mx, s_0);
    mx = wave_max(mx);
    float sm = 0.f;
#pragma unroll
    for (int r = 0; r < NPL; ++r)
      if ((selbits >> r) & 1ull) sm += expf(sv[r] - mx);
    sm = wave_sum(sm);
    sm += expf(s_c - mx);
    if (sink) sm += expf(s_0 - mx);
    lse = mx + logf(sm);
  }
  // compaction in ascending block order
  uint32_t pos_run = 0;
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    const bool sel = (selbits >> r) & 1ull;
    const uint64_t sb = __ballot(sel);
    const uint32_t pos = pos_run + (uint32_t)__popcll(sb & below);
    pos_run += (uint32_t)__popcll(sb);
    if (sel) {
      out[base + pos] = lane + 64 * r;
      if (gout) gout[base + pos] = sv[r] - lse;
    }
  }
  const int n = base + k + 1;
  if (lane == 0) {
    if (sink) {
      out[0] = 0;
      if (gout) gout[0] = s_0 - lse;
    }
    out[base + k] = c;
    if (gout) gout[base + k] = s_c - lse;
    *nsel_out = n;
  }
  for (int p = n + lane; p < kcap; p += 64) {
    out[p] = -1;
    if (gout) gout[p] = 0.f;
  }
}

template <typename T, typename R, int D, int NPL>
__global__ __launch_bounds__(256) void select_decode_kernel(
    SeqTable st, const T *__restrict__ Q, int64_t qb, int64_t qh, const R *__restrict__ reps, int64_t rb,
    int64_t rh, int64_t rj, int gist, int blk, int S, int G, int per_head, float scale, float *__restrict__ scores,
    int64_t ld, Budget bg, int kcap, int32_t *__restrict__ idx, int32_t *__restrict__ nsel, float *__restrict__ gate,
    uint32_t *__restrict__ counters) {
  constexpr int VEC = 16 / sizeof(R);
  constexpr int TPR = D / VEC;
  constexpr int RPP = 256 / TPR;
  constexpr int PASSES = 64 / RPP;
  __shared__ float qs[16][D];
  __shared__ float qsum[D];
  __shared__ __attribute__((aligned(16))) float scs[16][64];
  __shared__ uint32_t hist[4][1024];
  __shared__ int last_sh;
  const int j0 = blockIdx.x * 64, g = blockIdx.y, b = blockIdx.z;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  if (j0 > c) return;
  const int ntile = c / 64 + 1;  // tiles covering blocks 0..c
  const int nrep = gist ? min(L / blk, c) : cdiv(L, blk);
  const int nU = per_head ? G : 1;
  const int tid = threadIdx.x;
  const int cc = tid % TPR, r = tid / TPR;
  // representative loads first: they depend on nothing else
  const R *rbase = reps + b * rb + g * rh + cc * VEC;
  u32x4 raw[PASSES];
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int j = j0 + r + ps * RPP;
    if (j <= c && j < nrep) raw[ps] = *reinterpret_cast<const u32x4 *>(rbase + (int64_t)j * rj);
    else raw[ps] = u32x4{0u, 0u, 0u, 0u};
  }
  // the group's query rows (G x D <= 16 x 128 values): one element per lane per round, loaded
  // alongside the representative loads; pooled per unit through LDS
  constexpr int QR = 16 * D / 256;
  float qv[QR];
#pragma unroll
  for (int x = 0; x < QR; ++x) {
    const int e = tid + 256 * x;
    const int h = e / D, kd = e % D;
    qv[x] = 0.f;
    if (h < G) {
      const T *q = Q + b * qb + (int64_t)(g * G + h) * qh + kd;
      qv[x] = sizeof(T) == 2 ? bf16_to_f32(*(const uint16_t *)q) : *(const float *)q;
    }
  }
#pragma unroll
  for (int x = 0; x < QR; ++x) {
    const int e = tid + 256 * x;
    if (e / D < G) qs[e / D][e % D] = qv[x];
  }
  __syncthreads();
  if (!per_head) {
    // unit 0 = mean over the group's heads (sequential sum: the same order as the two-call path)
    for (int kd = tid; kd < D; kd += 256) {
      float sum = 0.f;
      for (int h = 0; h < G; ++h) sum += qs[h][kd];
      qsum[kd] = sum / (float)G;
    }
    __syncthreads();
    for (int kd = tid; kd < D; kd += 256) qs[0][kd] = qsum[kd];
    __syncthreads();
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
      if (cc == 0) scs[u][r + ps * RPP] = (j < nrep) ? part * scale : -INFINITY;
    }
  }
  __syncthreads();
  // device-coherent 16-byte stores of the tile's scores (entries j <= c only)
  for (int e = tid; e < nU * 16; e += 256) {
    const int u = e / 16, q = e % 16;
    const int s = per_head ? g * G + u : g;
    const __amdgpu_buffer_rsrc_t rrow = dev_rsrc(scores + ((int64_t)b * S + s) * ld, (uint32_t)ld * 4u);
    const int j = j0 + 4 * q;
    if (j + 3 <= c) {
      store16_dev(rrow, (uint32_t)j * 4u, *reinterpret_cast<const f32x4 *>(&scs[u][4 * q]));
    } else {
#pragma unroll
      for (int x = 0; x < 4; ++x)
        if (j + x <= c) store4_dev(rrow, (uint32_t)(j + x) * 4u, scs[u][4 * q + x]);
    }
  }
  // ---- arrival: the last tile of this (sequence, KV head) selects for its units
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(&counters[b * gridDim.y + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_sh = (old == (uint32_t)(ntile - 1));
  }
  __syncthreads();
  if (!last_sh) return;
  const int wave = tid >> 6;
  for (int u = wave; u < nU; u += 4) {
    const int s = per_head ? g * G + u : g;
    const int64_t urow = (int64_t)b * S + s;
    wave_topk<NPL>(scores + urow * ld, c, bg.sink != 0, bg, kcap, idx + urow * kcap, nsel + urow,
                   bg.gate ? gate + urow * kcap : nullptr, hist[wave]);
  }
  if (tid == 0) __hip_atomic_store(&counters[b * gridDim.y + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename T, typename R, int D>
static hipError_t sel_dispatch(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                               const void *reps, int gist, const int64_t *rs, int32_t sel_mode, float scale,
                               float *scores, int64_t ld, const Budget &bg, int32_t kcap, int32_t *idx,
                               int32_t *nsel, float *gate, uint32_t *counters, hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  dim3 grid(maxc / 64 + 1, p.hkv, p.batch);
#define SAS_SEL_LAUNCH(NPL_)                                                                                   \
  hipLaunchKernelGGL((select_decode_kernel<T, R, D, NPL_>), grid, dim3(256), 0, s, st, (const T *)Q, qs[0],     \
                     qs[1], (const R *)reps, rs[0], rs[1], rs[2], gist, p.block, S, p.hq / p.hkv, per_head,     \
                     scale, scores, ld, bg, kcap, idx, nsel, gate, counters)
  if (maxc <= 512) SAS_SEL_LAUNCH(8);
  else SAS_SEL_LAUNCH(32);
#undef SAS_SEL_LAUNCH
  return hipGetLastError();
}

hipError_t launch_select_decode(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                                const void *reps, int32_t reps_kind, const int64_t *rs, int32_t sel_mode,
                                float scale, float *scores, int64_t ld, const Budget &bg, int32_t kcap,
                                int32_t *idx, int32_t *nsel, float *gate, uint32_t *counters, hipStream_t s) {
  const int gist = reps_kind == SAS_REPS_GIST;
  if (p.dtype == SAS_BF16) {
    if (gist)
      return p.head_dim == 128
                 ? sel_dispatch<uint16_t, uint16_t, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s)
                 : sel_dispatch<uint16_t, uint16_t, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s);
    return p.head_dim == 128
               ? sel_dispatch<uint16_t, float, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s)
               : sel_dispatch<uint16_t, float, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s);
  }
  return p.head_dim == 128
             ? sel_dispatch<float, float, 128>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s)
             : sel_dispatch<float, float, 64>(p, st, Q, qs, reps, gist, rs, sel_mode, scale, scores, ld, bg, kcap, idx, nsel, gate, counters, s);
}

}  // namespace sas
