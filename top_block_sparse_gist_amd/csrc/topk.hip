// A3: per-unit exact top-k + forced blocks + log-gate.
// Page "SAS: 通过端到端优化上下文排序的简单注意力稀疏化", method (core modules 2-4: hard
// top-k at inference over the selector's scores, the current block always kept, the
// selector score entering the softmax in log form, normalised over the kept set); page
// "稀疏注意力" section 4.6 (dynamic top-k over a cheap candidate score).
//
// One 256-lane workgroup per unit.  Scores map to order-preserving 32-bit keys; an MSB-first
// radix select (four 8-bit passes, LDS histogram, one-wave suffix scan) finds the k-th
// largest key T and how many keys equal to T are taken.  Keys equal to T are taken in
// ascending block order (ties go to the lower block index).  Selected candidates are
// compacted in ascending order with ballot/popcount block scans, so the list comes out
// sorted without a sort.  The gate is s_j - logsumexp over the selected set (fp32).
#include "common.h"
#include "decode_parts.h"

namespace sas {

// Inverse of float_order_key.
__device__ __forceinline__ float order_key_float_tk(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Exclusive prefix count of `f` over the workgroup in lane order; `total` gets the sum.
__device__ __forceinline__ uint32_t block_scan_flag(bool f, uint32_t *sh, uint32_t &total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t bal = __ballot(f);
  const uint32_t wpre = (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) sh[w] = (uint32_t)__popcll(bal);
  __syncthreads();
  uint32_t pre = 0, tot = 0;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    uint32_t v = sh[x];
    pre += (x < w) ? v : 0u;
    tot += v;
  }
  total = tot;
  __syncthreads();
  return pre + wpre;
}

__device__ __forceinline__ float block_reduce_max(float v, float *sh) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float *sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) sh[w] = v;
  __syncthreads();
  float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256) void topk_kernel(SeqTable st, const float *__restrict__ scores,
                                                   int64_t ld, int tq, int blk, int S, int QB,
                                                   Budget bg, int kcap, int32_t *__restrict__ idx,
                                                   int32_t *__restrict__ nsel,
                                                   float *__restrict__ gate) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_above;
  __shared__ uint32_t scan_sh[4];
  __shared__ float red_sh[4];

  const int64_t u = blockIdx.x;
  const int i = (int)(u % QB);
  const int b = (int)(u / QB) / S;
  const int tid = threadIdx.x;
  const int q0 = st.q0[b];
  const int c0 = q0 / blk;
  const int nqb = (q0 + tq - 1) / blk - c0 + 1;
  int32_t *out = idx + u * kcap;
  float *gout = bg.gate ? gate + u * kcap : nullptr;
  if (i >= nqb) {
    for (int p = tid; p < kcap; p += 256) {
      out[p] = -1;
      if (gout) gout[p] = 0.f;
    }
    if (tid == 0) nsel[u] = 0;
    return;
  }
  const int c = c0 + i;
  const float *row = scores + u * ld;
  const bool sink = bg.sink && c > 0;
  const int lo = sink ? 1 : 0;
  const int ncand = c - lo;
  int k = budget_k(bg, c, ncand);
  const int base = sink ? 1 : 0;
  if (bg.coverage > 0.f && k > 0) {
    // coverage budget ([SF] 2.3, threshold-based): the smallest number of candidates, in (score
    // descending, block ascending) order, whose share of the candidates' softmax mass reaches
    // bg.coverage.  Bisection over the key range for the largest key T with mass(>= T) >= the
    // target (mass at the smallest key is the total, summed in the same order), then holders of T
    // one share each, as an exact ranking takes tied candidates in block order.
    constexpr float L2E = 1.4426950408889634f;
    float smax = -INFINITY, smin = INFINITY;
    for (int j = lo + tid; j < c; j += 256) {
      smax = fmaxf(smax, row[j]);
      smin = fminf(smin, row[j]);
    }
    smax = block_reduce_max(smax, red_sh);
    smin = -block_reduce_max(-smin, red_sh);
    auto mass = [&](uint32_t t) {
      float m = 0.f;
      for (int j = lo + tid; j < c; j += 256)
        m += float_order_key(row[j]) >= t ? __builtin_amdgcn_exp2f((row[j] - smax) * L2E) : 0.f;
      return block_reduce_sum(m, red_sh);
    };
    auto count = [&](uint32_t t) {
      float n = 0.f;  // exact: at most 2^24 candidates
      for (int j = lo + tid; j < c; j += 256) n += float_order_key(row[j]) >= t ? 1.f : 0.f;
      return (uint32_t)block_reduce_sum(n, red_sh);
    };
    const uint32_t kmin = float_order_key(smin), kmax = float_order_key(smax);
    const float target = bg.coverage * mass(kmin);
    uint64_t lo_t = kmin, hi_t = (uint64_t)kmax + 1u;
    while (hi_t - lo_t > 1u) {
      const uint64_t mid = lo_t + (hi_t - lo_t) / 2u;
      if (mass((uint32_t)mid) >= target) lo_t = mid;
      else hi_t = mid;
    }
    const uint32_t T = (uint32_t)lo_t;
    const bool top = T == 0xFFFFFFFFu;
    const float m_gt = top ? 0.f : mass(T + 1u);
    const uint32_t n_gt = top ? 0u : count(T + 1u);
    const uint32_t n_eq = count(T) - n_gt;
    const float e_t = __builtin_amdgcn_exp2f((order_key_float_tk(T) - smax) * L2E);
    uint32_t take = 1u;
    while (take < n_eq && m_gt + (float)take * e_t < target) ++take;
    k = min(k, (int)(n_gt + take));
  }

  if (k >= ncand) {
    for (int j = lo + tid; j < c; j += 256) out[base + (j - lo)] = j;
  } else if (k > 0) {
    // ---- radix select of the k-th largest key among the candidates
    uint32_t prefix = 0u, pmask = 0u;
    uint32_t want = (uint32_t)k;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0u;
      __syncthreads();
      for (int j = lo + tid; j < c; j += 256) {
        uint32_t key = float_order_key(row[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        uint32_t cnt[4], tot = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          cnt[t] = hist[255 - 4 * tid - t];
          tot += cnt[t];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t v = __shfl_up(incl, o, 64);
          if (tid >= o) incl += v;
        }
        const uint32_t excl = incl - tot;
        if (excl < want && want <= incl) {
          uint32_t run = excl;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (run + cnt[t] >= want) {
              sh_digit = (uint32_t)(255 - 4 * tid - t);
              sh_above = run;
              break;
            }
            run += cnt[t];
          }
        }
      }
      __syncthreads();
      want -= sh_above;
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    const uint32_t T = prefix;
    // ---- compaction in ascending block order
    uint32_t eq_seen = 0, pos_run = 0;
    for (int j0 = lo; j0 < c; j0 += 256) {
      const int j = j0 + tid;
      const bool valid = j < c;
      const uint32_t key = valid ? float_order_key(row[j]) : 0u;
      const bool gt = valid && key > T;
      const bool eq = valid && key == T;
      uint32_t eq_tot, sel_tot;
      const uint32_t eq_rank = block_scan_flag(eq, scan_sh, eq_tot) + eq_seen;
      const bool sel = gt || (eq && eq_rank < want);
      const uint32_t pos = block_scan_flag(sel, scan_sh, sel_tot) + pos_run;
      if (sel) out[base + pos] = j;
      eq_seen += eq_tot;
      pos_run += sel_tot;
    }
  }
  const int n = base + k + 1;
  if (tid == 0) {
    if (sink) out[0] = 0;
    out[base + k] = c;
    nsel[u] = n;
  }
  for (int p = n + tid; p < kcap; p += 256) {
    out[p] = -1;
    if (gout) gout[p] = 0.f;
  }
  if (gout) {
    __syncthreads();  // the list written above is read back below by other lanes
    float mx = -INFINITY;
    for (int p = tid; p < n; p += 256) mx = fmaxf(mx, row[out[p]]);
    mx = block_reduce_max(mx, red_sh);
    float sm = 0.f;
    for (int p = tid; p < n; p += 256) sm += expf(row[out[p]] - mx);
    sm = block_reduce_sum(sm, red_sh);
    const float lse = mx + logf(sm);
    for (int p = tid; p < n; p += 256) gout[p] = row[out[p]] - lse;
  }
}

// Shared budget (per-head units): one workgroup per (sequence, KV head, query block) selects for
// the G heads of the group together.  Their candidates compete as (head, block) pairs, candidate
// e = h * ncand + (j - lo); the radix select finds the K-th largest key over all of them (K = G
// times the per-head k); then each head's list is compacted in block order, the ranks of keys
// equal to T carried from head to head, which takes tied pairs in (head, block) order.
__global__ __launch_bounds__(256) void topk_joint_kernel(SeqTable st, const float *__restrict__ scores,
                                                         int64_t ld, int tq, int blk, int G, int hkv, int QB,
                                                         Budget bg, int kcap, int32_t *__restrict__ idx,
                                                         int32_t *__restrict__ nsel, float *__restrict__ gate) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh_digit, sh_above;
  __shared__ uint32_t scan_sh[4];
  __shared__ float red_sh[4];

  const int64_t wgi = blockIdx.x;
  const int i = (int)(wgi % QB);
  const int g = (int)(wgi / QB) % hkv;
  const int b = (int)(wgi / QB) / hkv;
  const int S = hkv * G;
  const int tid = threadIdx.x;
  auto unit = [&](int h) { return ((int64_t)b * S + g * G + h) * QB + i; };
  const int q0 = st.q0[b];
  const int c0 = q0 / blk;
  const int nqb = (q0 + tq - 1) / blk - c0 + 1;
  if (i >= nqb) {
    for (int h = 0; h < G; ++h) {
      for (int p = tid; p < kcap; p += 256) {
        idx[unit(h) * kcap + p] = -1;
        if (bg.gate) gate[unit(h) * kcap + p] = 0.f;
      }
      if (tid == 0) nsel[unit(h)] = 0;
    }
    return;
  }
  const int c = c0 + i;
  const bool sink = bg.sink && c > 0;
  const int lo = sink ? 1 : 0;
  const int ncand = c - lo;
  const int base = sink ? 1 : 0;
  const int n_all = G * ncand;
  const int K = min(G * budget_k(bg, c, ncand), n_all);
  auto key_of = [&](int e) {
    const int h = e / ncand;
    return float_order_key(scores[unit(h) * ld + lo + (e - h * ncand)]);
  };
  uint32_t T = 0u, want = 0u;
  const bool all = K >= n_all;
  if (!all && K > 0) {
    uint32_t prefix = 0u, pmask = 0u;
    want = (uint32_t)K;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0u;
      __syncthreads();
      for (int e = tid; e < n_all; e += 256) {
        const uint32_t key = key_of(e);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        uint32_t cnt[4], tot = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          cnt[t] = hist[255 - 4 * tid - t];
          tot += cnt[t];
        }
        uint32_t incl = tot;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          uint32_t v = __shfl_up(incl, o, 64);
          if (tid >= o) incl += v;
        }
        const uint32_t excl = incl - tot;
        if (excl < want && want <= incl) {
          uint32_t run = excl;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (run + cnt[t] >= want) {
              sh_digit = (uint32_t)(255 - 4 * tid - t);
              sh_above = run;
              break;
            }
            run += cnt[t];
          }
        }
      }
      __syncthreads();
      want -= sh_above;
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    T = prefix;
  }
  // ---- per head: compaction in block order (ranks of T carried across heads), forced blocks, gate
  uint32_t eq_seen = 0;
  for (int h = 0; h < G; ++h) {
    const float *row = scores + unit(h) * ld;
    int32_t *out = idx + unit(h) * kcap;
    float *gout = bg.gate ? gate + unit(h) * kcap : nullptr;
    uint32_t pos_run = 0;
    if (K > 0) {
      for (int j0 = lo; j0 < c; j0 += 256) {
        const int j = j0 + tid;
        const bool valid = j < c;
        const uint32_t key = valid ? float_order_key(row[j]) : 0u;
        const bool gt = valid && (all || key > T);
        const bool eq = valid && !all && key == T;
        uint32_t eq_tot, sel_tot;
        const uint32_t eq_rank = block_scan_flag(eq, scan_sh, eq_tot) + eq_seen;
        const bool sel = gt || (eq && eq_rank < want);
        const uint32_t pos = block_scan_flag(sel, scan_sh, sel_tot) + pos_run;
        if (sel) out[base + pos] = j;
        eq_seen += eq_tot;
        pos_run += sel_tot;
      }
    }
    const int n = base + (int)pos_run + 1;
    if (tid == 0) {
      if (sink) out[0] = 0;
      out[base + pos_run] = c;
      nsel[unit(h)] = n;
    }
    for (int p = n + tid; p < kcap; p += 256) {
      out[p] = -1;
      if (gout) gout[p] = 0.f;
    }
    if (gout) {
      __syncthreads();  // the list written above is read back below by other lanes
      float mx = -INFINITY;
      for (int p = tid; p < n; p += 256) mx = fmaxf(mx, row[out[p]]);
      mx = block_reduce_max(mx, red_sh);
      float sm = 0.f;
      for (int p = tid; p < n; p += 256) sm += expf(row[out[p]] - mx);
      sm = block_reduce_sum(sm, red_sh);
      const float lse = mx + logf(sm);
      for (int p = tid; p < n; p += 256) gout[p] = row[out[p]] - lse;
    }
    __syncthreads();  // scan_sh and red_sh are reused by the next head
  }
}

// One wave per unit, four units per workgroup (no barriers: waves finish independently): the
// unit's scores are read into registers, NPL per lane, and the register-resident top-k of the
// fused decode selection (team_topk on one wave: interpolation search over order-preserving keys
// with ballot counts, ballot compaction, the gate) selects.  Plain budgets with current blocks below
// 64 NPL (a unit with fewer candidates runs a shorter register loop); many waves per SIMD overlap the
// search's dependent steps.  Same lists and gates as topk_kernel.
template <int NPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(SeqTable st, const float *__restrict__ scores, int64_t ld,
                                                        int tq, int blk, int S, int QB, Budget bg, int kcap,
                                                        int32_t *__restrict__ idx, int32_t *__restrict__ nsel,
                                                        float *__restrict__ gate, int64_t units) {
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= units) return;
  const int lane = threadIdx.x & 63;
  const int i = (int)(u % QB);
  const int b = (int)(u / QB) / S;
  const int q0 = st.q0[b];
  const int c0 = q0 / blk;
  const int nqb = (q0 + tq - 1) / blk - c0 + 1;
  int32_t *out = idx + u * kcap;
  float *gout = bg.gate ? gate + u * kcap : nullptr;
  if (i >= nqb) {
    for (int p = lane; p < kcap; p += 64) {
      out[p] = -1;
      if (gout) gout[p] = 0.f;
    }
    if (lane == 0) nsel[u] = 0;
    return;
  }
  // the unit's own register count: rows over fewer candidates take a shorter loop
  const int c = c0 + i;
  const float *row = scores + u * ld;
  if (NPL > 8 && c < 64 * 8) {
    team_topk<(NPL > 8 ? 8 : NPL), SoloTeam, TK_PLAIN>(row, c, bg.sink != 0, bg, kcap, out, nsel + u, gout, SoloTeam{});
  } else if (NPL > 16 && c < 64 * 16) {
    team_topk<(NPL > 16 ? 16 : NPL), SoloTeam, TK_PLAIN>(row, c, bg.sink != 0, bg, kcap, out, nsel + u, gout,
                                                         SoloTeam{});
  } else {
    team_topk<NPL, SoloTeam, TK_PLAIN>(row, c, bg.sink != 0, bg, kcap, out, nsel + u, gout, SoloTeam{});
  }
}

hipError_t launch_topk(const sas_problem &p, const SeqTable &st, const float *scores, int64_t ld,
                       int32_t tq, int32_t sel_mode, const Budget &bg, int32_t kcap, int32_t *idx,
                       int32_t *nsel, float *gate, hipStream_t s) {
  const int QB = num_qblocks(tq, p.block);
  if (!bg.shared && !(bg.coverage > 0.f)) {
    int maxc = 0;
    for (int b = 0; b < p.batch; ++b) maxc = std::max(maxc, (st.q0[b] + tq - 1) / p.block);
    if (maxc < 64 * 32) {
      const int S = sel_mode == SAS_SEL_HEAD ? p.hq : p.hkv;
      const int64_t units = (int64_t)p.batch * S * QB;
      const dim3 grid((unsigned)cdiv64(units, 4));
#define SAS_TKW(NPL_)                                                                                      \
  hipLaunchKernelGGL((topk_wave_kernel<NPL_>), grid, dim3(256), 0, s, st, scores, ld, tq, p.block, S, QB, bg, \
                     kcap, idx, nsel, gate, units)
      if (maxc < 64 * 4) SAS_TKW(4);
      else if (maxc < 64 * 8) SAS_TKW(8);
      else if (maxc < 64 * 16) SAS_TKW(16);
      else SAS_TKW(32);
#undef SAS_TKW
      return hipGetLastError();
    }
  }
  if (bg.shared) {
    const int64_t groups = (int64_t)p.batch * p.hkv * QB;
    hipLaunchKernelGGL(topk_joint_kernel, dim3((unsigned)groups), dim3(256), 0, s, st, scores, ld, tq, p.block,
                       p.hq / p.hkv, p.hkv, QB, bg, kcap, idx, nsel, gate);
    return hipGetLastError();
  }
  const int S = sel_mode == SAS_SEL_HEAD ? p.hq : p.hkv;
  const int64_t units = (int64_t)p.batch * S * QB;
  hipLaunchKernelGGL(topk_kernel, dim3((unsigned)units), dim3(256), 0, s, st, scores, ld, tq, p.block, S,
                     QB, bg, kcap, idx, nsel, gate);
  return hipGetLastError();
}

}  // namespace sas
