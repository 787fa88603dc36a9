// Device bodies of the decode kernels: the selection of one 64-block tile of representatives (with
// the top-k of a (sequence, KV head) by its last tile) and the attention of one workgroup's tiles
// (with the split-K merge by a unit's last workgroup).  The kernels (select_decode_kernel,
// decode_bf16_kernel) call them with their indices and LDS.
#pragma once

#include "common.h"

namespace sas {

// Inverse of float_order_key.
__device__ __forceinline__ float order_key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide reduction of a u32 to a uniform value: DPP within each 16-lane row, then the four
// row results through scalar registers.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  auto dpp = [](uint32_t x, auto ctrl) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, false);
  };
  v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // lane ^ 1
  v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // lane ^ 2
  v = op(v, dpp(v, std::integral_constant<int, 0x124>{}));  // row_ror:4
  v = op(v, dpp(v, std::integral_constant<int, 0x128>{}));  // row_ror:8
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// Number of keys >= t over the wave: one compare per register into its own scalar mask, counted with
// the scalar unit's popcount (independent compares, no cross-lane reduction).
template <int NPL>
__device__ __forceinline__ uint32_t count_ge(const uint32_t (&key)[NPL], uint32_t t) {
  uint32_t n = 0u;
#pragma unroll
  for (int r = 0; r < NPL; ++r) n += (uint32_t)__popcll(__ballot(key[r] >= t));
  return n;
}

// Keys >= ta and keys >= tb over the wave, in one pass over the registers.
template <int NPL>
__device__ __forceinline__ void count_ge2(const uint32_t (&key)[NPL], uint32_t ta, uint32_t tb, uint32_t &na,
                                          uint32_t &nb) {
  na = nb = 0u;
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    na += (uint32_t)__popcll(__ballot(key[r] >= ta));
    nb += (uint32_t)__popcll(__ballot(key[r] >= tb));
  }
}

// z with P(Z > z) = q for a standard normal Z, 0 < q < 1: the rational approximation of
// Abramowitz and Stegun, formula 26.2.23 (absolute error below 4.5e-4), mirrored for q > 1/2.
__device__ __forceinline__ float upper_normal_quantile(float q) {
  const float p = fminf(q, 1.f - q);
  const float t = sqrtf(-2.f * __logf(p));
  const float z = t - (2.515517f + t * (0.802853f + t * 0.010328f)) /
                          (1.f + t * (1.432788f + t * (0.189269f + t * 0.001308f)));
  return q > 0.5f ? -z : z;
}

// Wave-wide max / sum of a float to a uniform value: DPP within each 16-lane row, then the four row
// results through scalar registers (the same shape as wave_reduce_u32).
template <typename Op>
__device__ __forceinline__ float wave_reduce_f32(float v, Op op) {
  auto dpp = [](float x, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // lane ^ 1
  v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // lane ^ 2
  v = op(v, dpp(v, std::integral_constant<int, 0x124>{}));  // row_ror:4
  v = op(v, dpp(v, std::integral_constant<int, 0x128>{}));  // row_ror:8
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return op(op(r0, r1), op(r2, r3));
}
__device__ __forceinline__ float wave_fmax_dpp(float v) {
  return wave_reduce_f32(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ float wave_fsum_dpp(float v) {
  return wave_reduce_f32(v, [](float x, float y) { return x + y; });
}

// A team of waves that selects for one unit; each wave holds its own contiguous share of the
// candidates, and the team's values are the combination of wave-uniform partials.
// SoloTeam: one wave holds all of them.
struct SoloTeam {
  static constexpr int SIZE = 1;
  __device__ int rank() const { return 0; }
  __device__ uint32_t sum(uint32_t v) const { return v; }
  __device__ uint32_t min(uint32_t v) const { return v; }
  __device__ uint32_t max(uint32_t v) const { return v; }
  __device__ float fmax(float v) const { return v; }
  __device__ float fsum(float v) const { return v; }
  __device__ uint32_t before(uint32_t) const { return 0u; }  // sum over the earlier waves
};
// GroupTeam: the 4 waves of a workgroup; each combination passes the 4 partials through LDS
// (lane 0 of each wave writes one slot, one barrier, every wave reads all four).  The slot sets
// alternate, so a wave that is a combination ahead never overwrites slots a slower wave has yet
// to read.  Every wave of the workgroup must make the same sequence of combinations.
struct GroupTeam {
  static constexpr int SIZE = 4;
  uint32_t *slots;       // LDS [2][4]
  int w;                 // wave-uniform rank
  mutable int phase;     // slot set of the next combination
  __device__ int rank() const { return w; }
  template <typename F>
  __device__ uint32_t combine(uint32_t v, F f, bool prefix = false) const {
    uint32_t *sl = slots + 4 * phase;
    phase ^= 1;
    if ((threadIdx.x & 63) == 0) sl[w] = v;
    __syncthreads();
    const uint32_t a = sl[0], b = sl[1], c = sl[2], d = sl[3];
    if (prefix) return (w > 0 ? a : 0u) + (w > 1 ? b : 0u) + (w > 2 ? c : 0u);
    return f(f(a, b), f(c, d));
  }
  __device__ uint32_t sum(uint32_t v) const { return combine(v, [](uint32_t x, uint32_t y) { return x + y; }); }
  __device__ uint32_t min(uint32_t v) const {
    return combine(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
  }
  __device__ uint32_t max(uint32_t v) const {
    return combine(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
  }
  __device__ float fmax(float v) const {
    return __uint_as_float(
        combine(__float_as_uint(v), [](uint32_t x, uint32_t y) { return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y))); }));
  }
  __device__ float fsum(float v) const {
    return __uint_as_float(
        combine(__float_as_uint(v), [](uint32_t x, uint32_t y) { return __float_as_uint(__uint_as_float(x) + __uint_as_float(y)); }));
  }
  __device__ uint32_t before(uint32_t v) const { return combine(v, [](uint32_t x, uint32_t) { return x; }, true); }
};

// Coverage budget: the smallest number of candidates, in (key descending, block ascending) order,
// whose share of the candidates' softmax mass is >= cov.  The largest key T with mass(>= T) >= cov
// times the total is found by bisection over the key range (mass at the smallest key is the total,
// summed in the same order); the holders of keys above T are all taken, then holders of T, one
// share each, until the share is reached -- as an exact ranking takes tied candidates in block
// order.  Shares are fp32 (2^x by v_exp_f32).
template <int NPL, typename Team>
__device__ uint32_t coverage_count(const uint32_t (&key)[NPL], float cov, const Team &team) {
  constexpr float L2E = 1.4426950408889634f;
  float smax = -INFINITY;
#pragma unroll
  for (int r = 0; r < NPL; ++r)
    if (key[r]) smax = fmaxf(smax, order_key_float(key[r]));
  smax = team.fmax(wave_max(smax));
  // a candidate's share is recomputed at each use rather than held: the keys already take NPL
  // registers per lane
  auto mass = [&](uint32_t t) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < NPL; ++r)
      m += (key[r] && key[r] >= t) ? __builtin_amdgcn_exp2f((order_key_float(key[r]) - smax) * L2E) : 0.f;
    return team.fsum(wave_sum(m));
  };
  auto count = [&](uint32_t t) { return team.sum(count_ge(key, t)); };
  uint32_t kmin = ~0u, kmax = 0u;  // over key - 1: a non-candidate's 0 wraps to the top
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    kmin = min(kmin, key[r] - 1u);
    kmax = max(kmax, key[r]);
  }
  kmin = team.min(wave_reduce_u32(kmin, [](uint32_t x, uint32_t y) { return min(x, y); })) + 1u;
  kmax = team.max(wave_reduce_u32(kmax, [](uint32_t x, uint32_t y) { return max(x, y); }));
  const float target = cov * mass(kmin);  // the total: every candidate's key is >= kmin
  uint64_t lo = kmin, hi = (uint64_t)kmax + 1u;  // mass(lo) >= target > 0 = mass(hi)
  while (hi - lo > 1u) {
    const uint64_t mid = lo + (hi - lo) / 2u;
    if (mass((uint32_t)mid) >= target) lo = mid;
    else hi = mid;
  }
  const uint32_t T = (uint32_t)lo;
  const bool top = T == 0xFFFFFFFFu;
  const float m_gt = top ? 0.f : mass(T + 1u);
  const uint32_t n_gt = top ? 0u : count(T + 1u);
  const uint32_t n_eq = count(T) - n_gt;
  const float e_t = __builtin_amdgcn_exp2f((order_key_float(T) - smax) * L2E);
  uint32_t take = 1u;
  while (take < n_eq && m_gt + (float)take * e_t < target) ++take;
  return n_gt + take;
}

// Top-k modes: plain, coverage budget, shared budget (the heads of a KV group, one per wave).
enum { TK_PLAIN = 0, TK_COVERAGE = 1, TK_SHARED = 2 };

// Top-k of one unit's scores row[0..c] by a team of waves: wave w of the team holds blocks
// 64 * NPL * w + lane + 64r in its register r (the scores are read back from memory, where the
// unit's tiles left them).  Ties go to the lower block.
// TK_SHARED: wave w < nact holds all of head w's row (its own unit: row, out, nsel_out, gout) and
// the nact heads select together, G * k (head, block) pairs ranked by (key, head, block); each
// wave then writes its head's list, forced blocks and gate (the other waves hold no candidate).
template <int NPL, typename Team, int TK = TK_PLAIN>
__device__ void team_topk(const float *__restrict__ row, int c, bool sinkf, const Budget &bg, int kcap,
                          int32_t *__restrict__ out, int32_t *__restrict__ nsel_out, float *__restrict__ gout,
                          const Team &team, int nact = 1) {
  static_assert(NPL <= 32, "one selection bit per register in a 32-bit mask");
  constexpr bool COV = TK == TK_COVERAGE, JOINT = TK == TK_SHARED;
  // opaque per call: keeps the compiler from hoisting the per-register block numbers and masks out
  // of a caller's loop over units, where they would hold ~100 registers across the whole kernel
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int jw = JOINT ? 0 : 64 * NPL * team.rank();  // this wave's first block
  const bool act = !JOINT || team.rank() < nact;     // the wave holds candidates
  const bool sink = sinkf && c > 0;
  const int lo = sink ? 1 : 0;
  const int ncand = JOINT ? nact * (c - lo) : c - lo;  // over the whole team
  int k = JOINT ? min(nact * budget_k(bg, c, c - lo), ncand) : budget_k(bg, c, ncand);
  const int base = sink ? 1 : 0;
  // order-preserving keys of the candidates, 0 elsewhere: a candidate's key is never 0 (that is
  // the key of one NaN pattern only, and NaN scores are not ranked)
  uint32_t key[NPL];
  float s_c = 0.f, s_0 = 0.f;
  // the interpolation search below takes its first bracket from the candidates' score moments
  constexpr bool GUESS = NPL * Team::SIZE > 8;
  float m1 = 0.f, m2 = 0.f;
  if (act) {
    // device-coherent loads through a buffer resource (not atomics, which the compiler issues one at
    // a time, each waiting for the previous): every lane loads (entries up to c exist), all loads are
    // issued before the first key is formed
    const __amdgpu_buffer_rsrc_t rr = dev_rsrc(row, (uint32_t)(c + 1) * 4u);
    float sv[NPL];
#pragma unroll
    for (int r = 0; r < NPL; ++r) sv[r] = load4_dev(rr, (uint32_t)min(jw + lane + 64 * r, c) * 4u);
    s_c = load4_dev(rr, (uint32_t)c * 4u);
    s_0 = load4_dev(rr, 0u);
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      const int j = jw + lane + 64 * r;
      const bool cand = j >= lo && j < c;
      key[r] = cand ? max(float_order_key(sv[r]), 1u) : 0u;
      if constexpr (GUESS) {
        const float x = (cand && fabsf(sv[r]) < 1.0e18f) ? sv[r] : 0.f;
        m1 += x;
        m2 = fmaf(x, x, m2);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < NPL; ++r) key[r] = 0u;
  }
  auto count = [&](uint32_t t) { return team.sum(count_ge(key, t)); };
  if constexpr (COV) {  // compiled only into the launches that carry a coverage budget
    if (bg.coverage > 0.f && k > 0) k = min(k, (int)coverage_count(key, bg.coverage, team));
  }
  // The kept candidates: all keys > T, then the `want` lowest blocks with key == T (ties: only
  // when T is the exact k-th largest key and more keys share it).
  uint32_t T = 0u, want = 0u;
  bool ties = false;
  const bool all = k >= ncand;
  if (!all && k > 0) {
    // the candidates' key range
    uint32_t kmin = ~0u, kmax = 0u;  // kmin over key - 1: a non-candidate's 0 wraps to the top
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      kmin = min(kmin, key[r] - 1u);
      kmax = max(kmax, key[r]);
    }
    kmin = team.min(wave_reduce_u32(kmin, [](uint32_t x, uint32_t y) { return min(x, y); })) + 1u;
    kmax = team.max(wave_reduce_u32(kmax, [](uint32_t x, uint32_t y) { return max(x, y); }));
    const uint32_t c_hi = count(kmax);
    if (c_hi >= (uint32_t)k) {
      T = kmax;  // the largest key alone fills the budget: its first k holders in block order
      want = (uint32_t)k;
      ties = c_hi > (uint32_t)k;
    } else if constexpr (NPL * Team::SIZE <= 8) {
      // Few candidates per lane: MSB-first bit steps below the keys' common prefix (the bits
      // above the highest bit in which the smallest and largest key differ), each one count;
      // an exact count of k ends the search.  (kmin != kmax here: equal keys would all count.)
      const int top = 31 - __builtin_clz(kmin ^ kmax);
      uint32_t prefix = top >= 31 ? 0u : (kmax & ~((2u << top) - 1u));
      bool exact = false;
      for (int bit = top; bit >= 0; --bit) {
        const uint32_t cand_t = prefix | (1u << bit);
        const uint32_t ge = count(cand_t);
        if (ge >= (uint32_t)k) {
          prefix = cand_t;
          if (ge == (uint32_t)k) {
            exact = true;
            break;
          }
        }
      }
      T = prefix;
      want = exact ? (uint32_t)k : (uint32_t)k - count(T + 1u);
      ties = !exact;
    } else {
      // Safeguarded interpolation search for the largest key value T with at least k keys at or
      // above it (fewer probes than bit steps on many candidates per lane).  Invariant:
      // count(lo) = cl >= k > ch = count(hi).  Each probe goes where a straight line between
      // (lo, cl) and (hi, ch) reaches k -- or to the midpoint after a probe that did not halve
      // the range -- and replaces lo or hi.  A probe with exactly k keys at or above it ends the
      // search: those keys are the selection.  Otherwise the range closes to hi = lo + 1 and lo
      // is the k-th largest key, with k - ch of its holders taken.
      uint32_t lo = kmin, hi = kmax, cl = (uint32_t)ncand, ch = c_hi;
      bool exact = false, bisect = false;
      // First bracket: with the candidates' mean and spread, a normal model puts 3k/2 and 2k/3
      // scores above two values; both are counted in one pass.  A count moves lo or hi whatever
      // the model's error (counts fall as the probe rises), so the model decides only how many
      // probes follow.
      const float M1 = team.fsum(wave_fsum_dpp(m1)), M2 = team.fsum(wave_fsum_dpp(m2));
      if (hi - lo > 2u) {
        const float nc = (float)ncand, mu = M1 / nc, sd = sqrtf(fmaxf(M2 / nc - mu * mu, 0.f));
        if (sd > 0.f && sd < 1.0e18f) {
          auto probe = [&](float above) {
            const float v = fmaf(sd, upper_normal_quantile(fminf(fmaxf(above, 0.5f), nc - 0.5f) / nc), mu);
            return min(max(float_order_key(v), lo + 1u), hi - 1u);
          };
          const uint32_t ta = probe(1.5f * (float)k), tb = max(probe((float)k / 1.5f), ta);
          uint32_t ca, cb;
          count_ge2(key, ta, tb, ca, cb);
          ca = team.sum(ca);
          cb = team.sum(cb);
          if (ca >= (uint32_t)k) {
            lo = ta;
            cl = ca;
            exact = ca == (uint32_t)k;
            if (!exact && cb >= (uint32_t)k) {
              lo = tb;
              cl = cb;
              exact = cb == (uint32_t)k;
            } else if (!exact && tb < hi) {
              hi = tb;
              ch = cb;
            }
          } else {
            hi = ta;
            ch = ca;
          }
        }
      }
      while (!exact && hi - lo > 1u) {
        const uint32_t span = hi - lo;
        uint32_t step;
        if (bisect) {
          step = span >> 1;
        } else {
          // f in [0, 1): where the line between (lo, cl) and (hi, ch) reaches k; the float product is
          // clamped below 2^32 before the conversion
          const float f = (float)(cl - (uint32_t)k) * __builtin_amdgcn_rcpf((float)(cl - ch));
          step = (uint32_t)fminf((float)span * f, 4294967040.f);
          step = max(min(step, span - 1u), 1u);
        }
        const uint32_t t = lo + step;
        const uint32_t c_t = count(t);
        if (c_t >= (uint32_t)k) {
          lo = t;
          cl = c_t;
          if (c_t == (uint32_t)k) {
            exact = true;
            break;
          }
        } else {
          hi = t;
          ch = c_t;
        }
        bisect = (hi - lo) > (span >> 1);
      }
      T = lo;
      want = exact ? (uint32_t)k : (uint32_t)k - ch;
      ties = !exact;
    }
  }
  // which candidates are kept (bit r of `selbits`: block jw + lane + 64r)
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t selbits = 0u;
  if (all) {
#pragma unroll
    for (int r = 0; r < NPL; ++r) selbits |= (key[r] != 0u ? 1u : 0u) << r;
  } else if (k > 0 && !ties) {
#pragma unroll
    for (int r = 0; r < NPL; ++r) selbits |= (key[r] >= T ? 1u : 0u) << r;  // T >= 1: candidates only
  } else if (k > 0) {
    // holders of T rank in block order, after those of the team's earlier waves
    uint32_t eq_w = 0;
#pragma unroll
    for (int r = 0; r < NPL; ++r) eq_w += (uint32_t)__popcll(__ballot(key[r] == T));
    uint32_t eq_seen = team.before(eq_w);
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      const bool eq = key[r] == T;  // T >= 1 here, so both tests pass over the non-candidates
      const uint64_t eb = __ballot(eq);
      const uint32_t eq_rank = eq_seen + (uint32_t)__popcll(eb & below);
      eq_seen += (uint32_t)__popcll(eb);
      selbits |= ((key[r] > T) || (eq && eq_rank < want) ? 1u : 0u) << r;
    }
  }
  // log-gate: g_j = s_j - logsumexp over the selected set (forced blocks included)
  float lse = 0.f;
  if (gout) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < NPL; ++r) mx = fmaxf(mx, ((selbits >> r) & 1u) ? order_key_float(key[r]) : -INFINITY);
    mx = fmaxf(mx, s_c);
    if (sink) mx = fmaxf(mx, s_0);
    mx = JOINT ? wave_fmax_dpp(mx) : team.fmax(wave_fmax_dpp(mx));  // shared: each head's own set
    // exp(x - mx) as 2^((x - mx) log2 e): one v_exp_f32 each; terms that flush to 0 are below the
    // largest (1) by more than the float's precision
    constexpr float L2E = 1.4426950408889634f;
    float sm = 0.f;
#pragma unroll
    for (int r = 0; r < NPL; ++r) {
      const float e = __builtin_amdgcn_exp2f((order_key_float(key[r]) - mx) * L2E);
      sm += ((selbits >> r) & 1u) ? e : 0.f;
    }
    sm = JOINT ? wave_fsum_dpp(sm) : team.fsum(wave_fsum_dpp(sm));
    sm += __builtin_amdgcn_exp2f((s_c - mx) * L2E);
    if (sink) sm += __builtin_amdgcn_exp2f((s_0 - mx) * L2E);
    lse = mx + logf(sm);
  }
  // compaction in ascending block order, after the team's earlier waves' selections
  uint32_t sel_w = 0;
#pragma unroll
  for (int r = 0; r < NPL; ++r) sel_w += (uint32_t)__popcll(__ballot((selbits >> r) & 1u));
  uint32_t pos_run = JOINT ? 0u : team.before(sel_w);  // shared: each head its own list
#pragma unroll
  for (int r = 0; r < NPL; ++r) {
    const bool sel = (selbits >> r) & 1u;
    const uint64_t sb = __ballot(sel);
    const uint32_t pos = pos_run + (uint32_t)__popcll(sb & below);
    pos_run += (uint32_t)__popcll(sb);
    if (sel) {
      out[base + pos] = jw + lane + 64 * r;
      if (gout) gout[base + pos] = order_key_float(key[r]) - lse;
    }
  }
  const int kw = JOINT ? (int)sel_w : k;  // blocks this list keeps besides the forced ones
  const int n = base + kw + 1;
  if ((JOINT ? act : team.rank() == 0) && lane == 0) {
    if (sink) {
      out[0] = 0;
      if (gout) gout[0] = s_0 - lse;
    }
    out[base + kw] = c;
    if (gout) gout[base + kw] = s_c - lse;
    *nsel_out = n;
  }
  if (JOINT) {
    if (act)
      for (int p = n + lane; p < kcap; p += 64) {
        out[p] = -1;
        if (gout) gout[p] = 0.f;
      }
  } else {
    for (int p = n + 64 * team.rank() + lane; p < kcap; p += 64 * Team::SIZE) {
      out[p] = -1;
      if (gout) gout[p] = 0.f;
    }
  }
}

// LDS of one selection workgroup.
template <int D>
struct SelectLds {
  static constexpr int QS = 0;                              // float [16][D]  unit queries
  static constexpr int QSUM = QS + 16 * D * 4;              // float [D]      group mean
  static constexpr int SCS = QSUM + D * 4;                  // float [16][64] staged scores
  static constexpr int LAST = SCS + 16 * 64 * 4;            // int            last-arrival flag
  static constexpr int BYTES = LAST + 16;
};

// Selection tiles of one (sequence, KV head): 64-block tiles covering blocks 0..c (the current
// block's score feeds the gate), or in gist mode the gists 0..c-1 only (at least one tile, which
// runs the top-k).
__host__ __device__ inline int select_tiles(int c, int gist) { return gist ? max(1, (c + 63) / 64) : c / 64 + 1; }

// One selection workgroup: the 64-block tile bx of (sequence b, KV head g), hkv KV heads.  The last
// tile of (b, g) to arrive runs the top-k of its units.
template <typename T, typename R, int D, int NPL, int TK>
__device__ __forceinline__ void select_tile_body(
    int bx, int g, int b, int hkv, unsigned char *lds, SeqTable st, const T *__restrict__ Q, int64_t qb, int64_t qh,
    const R *__restrict__ reps, int64_t rb, int64_t rh, int64_t rj, int gist, int blk, int S, int G, int per_head,
    float scale, float *__restrict__ scores, int64_t ld, Budget bg, int kcap, int32_t *__restrict__ idx,
    int32_t *__restrict__ nsel, float *__restrict__ gate, uint32_t *__restrict__ counters) {
  constexpr int VEC = 16 / sizeof(R);
  constexpr int TPR = D / VEC;
  constexpr int RPP = 256 / TPR;
  constexpr int PASSES = 64 / RPP;
  using Lds = SelectLds<D>;
  auto qs = reinterpret_cast<float(*)[D]>(lds + Lds::QS);
  float *qsum = reinterpret_cast<float *>(lds + Lds::QSUM);
  auto scs = reinterpret_cast<float(*)[64]>(lds + Lds::SCS);
  int &last_sh = *reinterpret_cast<int *>(lds + Lds::LAST);
  const int j0 = bx * 64;
  const int L = seq_len(st, b);
  const int c = (L - 1) / blk;
  const int ntile = select_tiles(c, gist);
  if (bx >= ntile) return;
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
  if (gist && j0 + 64 == c && tid < nU) {
    // gist mode: no tile starts at the current chunk, which has no gist; the last tile writes its -inf
    const int s = per_head ? g * G + tid : g;
    store4_dev(dev_rsrc(scores + ((int64_t)b * S + s) * ld, (uint32_t)ld * 4u), (uint32_t)c * 4u, -INFINITY);
  }
  // ---- arrival: the last tile of this (sequence, KV head) selects for its units
  wait_stores();
  __syncthreads();
  if (tid == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(&counters[b * hkv + g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_sh = (old == (uint32_t)(ntile - 1));
  }
  __syncthreads();
  if (!last_sh) return;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (TK == TK_SHARED) {
    // per-head units sharing G * k: wave w holds head w's row (G <= 4, checked on the host)
    const GroupTeam team{reinterpret_cast<uint32_t *>(lds + Lds::QS), wave, 0};
    const int64_t urow = (int64_t)b * S + g * G + min(wave, G - 1);
    team_topk<NPL, GroupTeam, TK_SHARED>(scores + urow * ld, c, bg.sink != 0, bg, kcap, idx + urow * kcap,
                                         nsel + urow, bg.gate ? gate + urow * kcap : nullptr, team, G);
  } else if (NPL == 32 && nU == 1) {
    // one unit with up to 2048 candidates: the 4 waves share them (8 registers per lane each),
    // combining their counts through LDS (the pooled queries' region, no longer read)
    const int64_t urow = (int64_t)b * S + (per_head ? g * G : g);
    const GroupTeam team{reinterpret_cast<uint32_t *>(lds + Lds::QS), wave, 0};
    team_topk<NPL / 4, GroupTeam, TK>(scores + urow * ld, c, bg.sink != 0, bg, kcap, idx + urow * kcap, nsel + urow,
                       bg.gate ? gate + urow * kcap : nullptr, team);
  } else {
    for (int u = wave; u < nU; u += 4) {
      const int s = per_head ? g * G + u : g;
      const int64_t urow = (int64_t)b * S + s;
      team_topk<NPL, SoloTeam, TK>(scores + urow * ld, c, bg.sink != 0, bg, kcap, idx + urow * kcap, nsel + urow,
                     bg.gate ? gate + urow * kcap : nullptr, SoloTeam{});
    }
  }
  if (tid == 0) __hip_atomic_store(&counters[b * hkv + g], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

static constexpr int VPAD = 16;  // LDS row padding (bf16 elements) of the V tile: rows start 8 banks apart

// Split record: acc [nh][D] fp32, then m [nh] (log2 units) and l [nh], padded to 16 bytes.
__host__ __device__ inline int64_t record_floats(int nh, int D) { return (int64_t)nh * D + ((2 * nh + 3) / 4) * 4; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// LDS of one attention workgroup: the V tiles (reused for the merges), then small arrays.  VK keys
// of a wave's V tile are staged at a time: all 64, or (units of one head, whose in-workgroup merge
// needs a sixteenth of the region) 32, in two halves, which halves the workgroup's LDS.
template <int D, int WPW, int VK = 64>
struct DecodeLds {
  static constexpr int VROW = D + VPAD;
  static constexpr int TILE_BYTES = WPW * VK * VROW * 2;
  static constexpr int SMALL_FLOATS = 2 * WPW * 16 + 4 + 32;  // m, l per wave; flag; M, L per head
  static constexpr int BYTES = TILE_BYTES + SMALL_FLOATS * 4;
};

// Two-level gist mode (meta-gists): the extra inputs of the attention.  Tiles of a unit: one per
// opened-group entry (that group's gists, the expanded chunks masked), then nmt tiles of 64
// meta-gists (the opened groups masked), then the raw tiles of the expanded chunks and the current
// chunk.  All ranges are known before nsel, so every list entry loads beside it.
struct MetaArgs {
  const uint16_t *MK, *MV;
  int64_t mb, mh, mt;   // strides of the meta-gist K/V [B, Hkv, NM, d]
  const int32_t *gidx;  // [units, gcap] opened groups, ascending, the trailing group last, -1 padded
  int M, gcap, nmt;     // chunks per group; list capacity; meta tiles per unit (grid-wide)
};

// Paged K/V: block j of sequence b lives in page table[b * tld + j] of the cache (pages of one
// block; kb is then the page stride).  table == nullptr: K/V are [B, Hkv, Lmax, d].
struct PageArgs {
  const int32_t *table;
  int64_t tld;
};

// One attention workgroup: tiles bx*WPW*TPW .. +WPW*TPW-1 of unit u (TPW = 1 to 3 per wave: wave w
// takes tiles w, w + WPW, ... of the workgroup's range, each next tile's K/V loads issued as soon
// as the previous one's registers are consumed, so they overlap its softmax and PV), merged into the
// unit's record bx (records nwg apart per unit).  A unit has nsel[u] list entries (the padding
// past them is -1), so it needs only the first nwg_u of the nwg workgroups: the others exit
// before touching the records, and the last of the nwg_u to arrive merges their records and
// writes O.
template <int D, int WPW, int TPW, typename OT, bool HS = false, int VK = 64>
__device__ __forceinline__ void decode_tile_body(
    int bx, int64_t u, int nwg, unsigned char *lds, SeqTable st, const uint16_t *__restrict__ Q, int64_t qb,
    int64_t qh, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt,
    const uint16_t *__restrict__ GK, const uint16_t *__restrict__ GV, int64_t gb, int64_t gh, int64_t gt, int gist,
    int blk, int S, int G, int per_head, const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel,
    const float *__restrict__ gate, int kcap,
    float scale_log2, float *__restrict__ work, uint32_t *__restrict__ counters, OT *__restrict__ O, int64_t ob,
    int64_t oh, MetaArgs ma = MetaArgs{}, PageArgs pg = PageArgs{}) {
  constexpr int NKK = D / 32;   // MFMA k-steps over the head dim
  constexpr int NDT = D / 16;   // 16-dim output tiles
  constexpr int VROW = D + VPAD;
  constexpr int NT = WPW * 64;
  using Lds = DecodeLds<D, WPW, VK>;
  static_assert(VK == 64 || VK == 32, "V staged as a whole tile or in two halves");
  static_assert(VK == 64 || WPW * VK * VROW * 2 >= WPW * 16 * D * 4, "in-workgroup merge region");
  auto vlds = reinterpret_cast<uint16_t(*)[VK * VROW]>(lds);
  float *small = reinterpret_cast<float *>(lds + Lds::TILE_BYTES);
  auto m_sh = reinterpret_cast<float(*)[16]>(small);
  auto l_sh = reinterpret_cast<float(*)[16]>(small + WPW * 16);
  int &last_sh = *reinterpret_cast<int *>(small + 2 * WPW * 16);
  float *Mh = small + 2 * WPW * 16 + 4, *Lh = Mh + 16;

  const int b = (int)(u / S), s = (int)(u % S);
  const int g = per_head ? s / G : s;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : s * G;
  const int L = seq_len(st, b);
  const int c = (L - 1) / blk;
  const int tpb = blk / 64;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  // this wave's tiles, and their list entries and gates, loaded beside nsel so that the K/V loads
  // wait for one load only
  int tt[TPW], jraw[TPW];
  float graw[TPW];
  const int r0 = HS ? ma.gcap + ma.nmt : 0;  // first raw tile
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    tt[k] = bx * WPW * TPW + k * WPW + wave;
    if (HS && tt[k] < ma.gcap) {
      jraw[k] = ma.gidx[u * ma.gcap + tt[k]];  // an opened group
      graw[k] = 0.f;
      continue;
    }
    const int e = tt[k] >= r0 ? (tt[k] - r0) / tpb : kcap;  // meta tiles have no entry
    jraw[k] = e < kcap ? idx[u * kcap + e] : -1;
    graw[k] = (gate && e < kcap) ? gate[u * kcap + e] : 0.f;
  }
  // this unit's tiles: the raw tiles of its list entries, then (gist mode) one tile per 64 gists
  const int nent = min(max(nsel[u], 0), kcap);
  const int nraw = nent * tpb;
  const int nwg_u = max(1, (r0 + nraw + (gist ? (c + 63) / 64 : 0) + WPW * TPW - 1) / (WPW * TPW));
  if (bx >= nwg_u) return;
  const int64_t rec_sz = record_floats(nh, D);

  // ---- which keys tile k of this wave holds
  struct Tile {
    const uint16_t *kbase, *vbase;
    int64_t rstride;
    int key0, nvalid;  // position of the tile's first key; keys present
    int roff;          // row of that key from kbase (key0, or its row inside a page)
    float gl2;
    uint64_t excl;
  };
  // bits of the 64 keys from key0 on that a list names (an entry j sets bit j - key0)
  auto list_bits = [&](const int32_t *list, int n, int key0) {
    uint64_t bits = 0;
    for (int e0 = 0; e0 < n; e0 += 64) {
      uint64_t bit = 0;
      if (e0 + lane < n) {
        const int j = list[e0 + lane];
        if (j >= key0 && j < key0 + 64) bit = 1ull << (j - key0);
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)bit, o, 64);
        const uint32_t hi = __shfl_xor((uint32_t)(bit >> 32), o, 64);
        bit |= ((uint64_t)hi << 32) | lo;
      }
      bits |= bit;
    }
    return bits;
  };
  auto describe = [&](int k) {
    Tile d{nullptr, nullptr, 0, 0, 0, 0, 0.f, 0ull};
    const int tk = tt[k] - r0;  // raw tiles count from r0
    if (HS && tk < 0) {
      if (tt[k] < ma.gcap) {
        // gists of an opened group (the trailing group may hold none); expanded chunks masked
        const int gi = jraw[k];
        if (gi >= 0) {
          d.key0 = gi * ma.M;
          d.nvalid = min(ma.M, c - d.key0);
          d.kbase = GK + b * gb + g * gh;
          d.vbase = GV + b * gb + g * gh;
          d.rstride = gt;
          d.roff = d.key0;
          if (d.nvalid > 0) d.excl = list_bits(idx + u * kcap, kcap, d.key0);
        }
      } else {
        // 64 meta-gists of the complete groups; the opened ones masked
        d.key0 = (tt[k] - ma.gcap) * 64;
        d.nvalid = min(64, c / ma.M - d.key0);
        d.kbase = ma.MK + b * ma.mb + g * ma.mh;
        d.vbase = ma.MV + b * ma.mb + g * ma.mh;
        d.rstride = ma.mt;
        d.roff = d.key0;
        if (d.nvalid > 0) d.excl = list_bits(ma.gidx + u * ma.gcap, ma.gcap, d.key0);
      }
    } else if (tk < nraw) {
      const int j = jraw[k];
      if (j >= 0) {
        d.key0 = j * blk + (tk % tpb) * 64;
        d.nvalid = min(64, L - d.key0);
        if (pg.table) {
          const int64_t page = pg.table[b * pg.tld + j];
          d.kbase = K + page * kb + g * kh;
          d.vbase = V + page * kb + g * kh;
          d.roff = (tk % tpb) * 64;
        } else {
          d.kbase = K + b * kb + g * kh;
          d.vbase = V + b * kb + g * kh;
          d.roff = d.key0;
        }
        d.rstride = kt;
        d.gl2 = graw[k] * 1.4426950408889634f;
      }
    } else if (gist) {
      d.key0 = (tk - nraw) * 64;
      d.nvalid = min(64, c - d.key0);
      d.kbase = GK + b * gb + g * gh;
      d.vbase = GV + b * gb + g * gh;
      d.rstride = gt;
      d.roff = d.key0;
      // gists of selected chunks are replaced by their raw tokens: exclude them
      if (d.nvalid > 0) d.excl = list_bits(idx + u * kcap, kcap, d.key0);
    }
    d.nvalid = max(d.nvalid, 0);
    return d;
  };
  Tile tl[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) tl[k] = describe(k);
  bool any = false;
#pragma unroll
  for (int k = 0; k < TPW; ++k) any = any || tl[k].nvalid > 0;

  // ---- Q^T as the B operand: lane -> head `col`, dims 32*kk + 8*grp .. +8
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < nh && any)
      v = *reinterpret_cast<const u32x4 *>(Q + b * qb + (int64_t)(h0 + col) * qh + 32 * kk + 8 * grp);
    qreg[kk] = as_bf16x8(v);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int x = 0; x < NDT; ++x) acc_o[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- K straight to A-operand registers, V rows to registers (then LDS)
  constexpr int VCH = D / 8;  // 16-byte chunks per V row; VCH loads per lane
  u32x4 kreg[4][NKK];
  u32x4 vreg[VCH];
  uint16_t *vl = vlds[wave];
  // V loads x in [x0, x1): with half-tile staging the second half's registers are reloaded only
  // after that half has been copied to LDS
  auto issue_v = [&](const Tile &d, int x0, int x1) {
#pragma unroll
    for (int x = x0; x < x1; ++x) {
      const int e = x * 64 + lane;
      const int key = e / VCH, ch = e % VCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < d.nvalid) v = *reinterpret_cast<const u32x4 *>(d.vbase + (int64_t)(d.roff + key) * d.rstride + ch * 8);
      vreg[x] = v;
    }
  };
  auto issue = [&](const Tile &d) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key = mt * 16 + col;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < d.nvalid)
          v = *reinterpret_cast<const u32x4 *>(d.kbase + (int64_t)(d.roff + key) * d.rstride + 32 * kk + 8 * grp);
        kreg[mt][kk] = v;
      }
    }
#pragma unroll
    for (int x = 0; x < (VK == 64 ? VCH : VCH / 2); ++x) {
      const int e = x * 64 + lane;
      const int key = e / VCH, ch = e % VCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < d.nvalid) v = *reinterpret_cast<const u32x4 *>(d.vbase + (int64_t)(d.roff + key) * d.rstride + ch * 8);
      vreg[x] = v;
    }
  };
  // (half-tile staging) V rows of keys [32h, 32h + 32) to this wave's LDS rows 0..31 (register x
  // holds key (64x + lane) / VCH, so each half is a contiguous range of registers)
  auto stage_v = [&](int h) {
#pragma unroll
    for (int x = h * (VCH / 2); x < (h + 1) * (VCH / 2); ++x) {
      const int e = x * 64 + lane;
      const int key = e / VCH - 32 * h, ch = e % VCH;
      *reinterpret_cast<u32x4 *>(vl + key * VROW + ch * 8) = vreg[x];
    }
  };
  issue(tl[0]);
  if constexpr (VK == 32) issue_v(tl[0], VCH / 2, VCH);
#pragma unroll
  for (int k = 0; k < TPW; ++k) {
    const Tile &d = tl[k];
    f32x4 sacc[4];
    if (d.nvalid > 0) {
      // ---- S^T = K Q^T
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[mt][kk]), qreg[kk], a, 0, 0, 0);
        sacc[mt] = a;
      }
      // the V tile region is this wave's own: the reads of the previous tile's PV precede these
      // writes in the wave's LDS queue
      if constexpr (VK == 64) {
#pragma unroll
        for (int x = 0; x < VCH; ++x) {
          const int e = x * 64 + lane;
          const int key = e / VCH, ch = e % VCH;
          *reinterpret_cast<u32x4 *>(vl + key * VROW + ch * 8) = vreg[x];
        }
      } else {
        stage_v(0);
      }
    }
    // the registers are free: the next tile's loads fly during this tile's softmax and PV
    if (k + 1 < TPW) issue(tl[k + 1]);
    if (d.nvalid > 0) {
      // ---- online softmax over the tile's keys, per head column
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = mt * 16 + 4 * grp + r;
          const bool ok = key < d.nvalid && !((d.excl >> key) & 1ull);
          const float v = ok ? sacc[mt][r] * scale_log2 + d.gl2 : -INFINITY;
          sacc[mt][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      if (k > 0) {
        // rescale what the earlier tiles left (alpha 0 while m_run is still -inf)
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int x = 0; x < NDT; ++x) acc_o[x] *= alpha;
      }
      m_run = m_new;
      const float mref = (m_new == -INFINITY) ? 0.f : m_new;
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __builtin_amdgcn_exp2f(sacc[mt][r] - mref);
          sacc[mt][r] = p;
          ls += p;
        }
      l_run += ls;
      // P^T as the B operand of each 32-key step (keys 32ks + 4grp + {0..3} and +16)
      bf16x8 preg[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 w;
        w[0] = pack_bf16x2(sacc[2 * ks][0], sacc[2 * ks][1]);
        w[1] = pack_bf16x2(sacc[2 * ks][2], sacc[2 * ks][3]);
        w[2] = pack_bf16x2(sacc[2 * ks + 1][0], sacc[2 * ks + 1][1]);
        w[3] = pack_bf16x2(sacc[2 * ks + 1][2], sacc[2 * ks + 1][3]);
        preg[ks] = as_bf16x8(w);
      }
      // ---- O^T += V^T P^T; the V^T operand (dim 16dt + col, keys 32ks + 4grp + {0..3} then
      //      32ks + 16 + 4grp + {0..3}) comes from two transpose reads of the row-major tile
      if constexpr (VK == 64) {
        // the V tile is written and read by this wave only: wait for its LDS writes
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const uint16_t *src = vl + (ks * 32 + 4 * grp + (col >> 2)) * VROW + dt * 16 + 4 * (col & 3);
            const u32x2 lo = lds_read_tr16(src);
            const u32x2 hi = lds_read_tr16(src + 16 * VROW);
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), preg[ks], acc_o[dt], 0, 0, 0);
          }
        }
      } else {
        // two halves through the same 32 rows: keys 0..31 (staged above), then 32..63, whose
        // writes follow the first half's transposing reads in the wave's LDS queue
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          if (ks == 1) {
            stage_v(1);
            // the second half's registers are free: the next tile's loads of them fly now
            if (k + 1 < TPW) issue_v(tl[k + 1], VCH / 2, VCH);
          }
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const uint16_t *src = vl + (4 * grp + (col >> 2)) * VROW + dt * 16 + 4 * (col & 3);
            const u32x2 lo = lds_read_tr16(src);
            const u32x2 hi = lds_read_tr16(src + 16 * VROW);
            const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
            acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), preg[ks], acc_o[dt], 0, 0, 0);
          }
        }
      }
    } else if constexpr (VK == 32) {
      // an empty tile still hands the next tile its second half of V registers
      if (k + 1 < TPW) issue_v(tl[k + 1], VCH / 2, VCH);
    }
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // ---- this workgroup's record: [nh][D] acc, then m[nh], l[nh] (m in log2 units), written with
  //      device-coherent 16-byte stores so that the merging workgroup (any XCD) reads them
  const uint32_t rec_bytes = (uint32_t)rec_sz * 4u;
  const __amdgpu_buffer_rsrc_t rr = dev_rsrc(work + u * nwg * rec_sz, nwg_u * rec_bytes);
  const uint32_t my = bx * rec_bytes;
  if constexpr (WPW == 1) {
    if (col < nh) {
      if (grp == 0) {
        store4_dev(rr, my + (uint32_t)(nh * D + col) * 4u, m_run);
        store4_dev(rr, my + (uint32_t)(nh * D + nh + col) * 4u, l_run);
      }
      if (m_run != -INFINITY) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) store16_dev(rr, my + (uint32_t)(col * D + dt * 16 + 4 * grp) * 4u, acc_o[dt]);
      }
    }
  } else {
    __syncthreads();
    float *osh = reinterpret_cast<float *>(&vlds[0][0]);  // [WPW][16][D] fp32 over the V tiles
    if (grp == 0) {
      m_sh[wave][col] = m_run;
      l_sh[wave][col] = l_run;
    }
    if (col < nh) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(osh + (wave * 16 + col) * D + dt * 16 + 4 * grp) = acc_o[dt];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < nh * (D / 4); e += NT) {
      const int n = e / (D / 4), q = e % (D / 4);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WPW; ++w) M = fmaxf(M, m_sh[w][n]);
      const float Mr = (M == -INFINITY) ? 0.f : M;
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < WPW; ++w) {
        const float f = (m_sh[w][n] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_sh[w][n] - Mr);
        o += f * *reinterpret_cast<const f32x4 *>(osh + (w * 16 + n) * D + 4 * q);
        l += f * l_sh[w][n];
      }
      store16_dev(rr, my + (uint32_t)(n * D + 4 * q) * 4u, o);
      if (q == 0) {
        store4_dev(rr, my + (uint32_t)(nh * D + n) * 4u, M);
        store4_dev(rr, my + (uint32_t)(nh * D + nh + n) * 4u, l);
      }
    }
  }

  // ---- arrival; the last workgroup of the unit merges every record and writes O
  wait_stores();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&counters[u], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_sh = (old == (uint32_t)nwg_u - 1);
  }
  __syncthreads();
  if (!last_sh) return;
  const int nrec = nwg_u;
  const int tid = threadIdx.x;
  float *msh = reinterpret_cast<float *>(&vlds[0][0]);  // [nrec][nh] m, then l, then weights
  float *lsh = msh + nrec * nh;
  float *fsh = lsh + nrec * nh;
  f32x4 *red = reinterpret_cast<f32x4 *>(msh + ((3 * nrec * nh + 3) / 4) * 4);
  // (1) every record's m and l in one round of loads
  for (int e = tid; e < nrec * nh; e += NT) {
    const int x = e / nh, n = e % nh;
    msh[e] = load4_dev(rr, x * rec_bytes + (uint32_t)(nh * D + n) * 4u);
    lsh[e] = load4_dev(rr, x * rec_bytes + (uint32_t)(nh * D + nh + n) * 4u);
  }
  __syncthreads();
  if (tid < nh) {
    float M = -INFINITY;
    for (int x = 0; x < nrec; ++x) M = fmaxf(M, msh[x * nh + tid]);
    Mh[tid] = (M == -INFINITY) ? 0.f : M;
  }
  __syncthreads();
  for (int e = tid; e < nrec * nh; e += NT) {
    const float m = msh[e];
    fsh[e] = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - Mh[e % nh]);
  }
  __syncthreads();
  if (tid < nh) {
    float l = 0.f;
    for (int x = 0; x < nrec; ++x) l += fsh[x * nh + tid] * lsh[x * nh + tid];
    Lh[tid] = l;
  }
  // (2) weighted sum of the acc quads; lanes split the records into RG groups
  const int Q4 = nh * (D / 4);
  const int RG = Q4 >= NT ? 1 : NT / Q4;
  const int rg = tid / Q4 < RG ? tid / Q4 : RG;  // RG marks an idle lane
  for (int q0 = 0; q0 < Q4; q0 += NT) {
    const int qq = q0 + tid % Q4 + (Q4 >= NT ? tid - tid % Q4 : 0);
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    const bool act = rg < RG && qq < Q4;
    const int n = act ? qq / (D / 4) : 0;
    if (act) {
      for (int x0 = rg; x0 < nrec; x0 += RG * 8) {
        f32x4 v[8];
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int x = x0 + i * RG;
          const bool ok = x < nrec;
          f[i] = ok ? fsh[x * nh + n] : 0.f;
          v[i] = (ok && f[i] != 0.f) ? load16_dev(rr, x * rec_bytes + (uint32_t)(4 * qq) * 4u)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) a += f[i] * v[i];
      }
    }
    if (RG > 1) {
      __syncthreads();
      if (act) red[rg * Q4 + qq] = a;
      __syncthreads();
      if (act && rg == 0)
        for (int g2 = 1; g2 < RG; ++g2) a += red[g2 * Q4 + qq];
    } else {
      __syncthreads();
    }
    if (act && rg == 0) {
      const float inv = 1.f / Lh[n];
      const int dim = 4 * (qq % (D / 4));
      OT *dst = O + b * ob + (int64_t)(h0 + n) * oh + dim;
      if constexpr (sizeof(OT) == 2) {
        u32x2 w;
        w[0] = pack_bf16x2(a[0] * inv, a[1] * inv);
        w[1] = pack_bf16x2(a[2] * inv, a[3] * inv);
        *reinterpret_cast<u32x2 *>(dst) = w;
      } else {
        *reinterpret_cast<f32x4 *>(dst) = a * inv;
      }
    }
  }
  if (tid == 0) __hip_atomic_store(&counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keys of V staged in LDS at a time by one-tile-per-wave launches: units of one head stage half tiles
// (their workgroups need half the LDS, so more of them fit per CU).  The merge capacity below is
// taken at that size for every launch of such units.
static inline int decode_v_keys(int nh) { return nh == 1 ? 32 : 64; }

struct DecodeShape {
  int S, nh, tiles_cap, wpw, nwg_cap;
  int64_t units;
};

static inline DecodeShape decode_shape(const sas_problem &p, int32_t sel_mode, int32_t kcap, int gist, int maxc) {
  DecodeShape d;
  const int per_head = sel_mode == SAS_SEL_HEAD;
  d.S = per_head ? p.hq : p.hkv;
  d.nh = per_head ? 1 : p.hq / p.hkv;
  d.units = (int64_t)p.batch * d.S;
  d.tiles_cap = kcap * (p.block / 64) + (gist ? (maxc + 63) / 64 : 0);
  d.wpw = 4;  // 4 waves per workgroup merge in LDS first, so the final merge reads fewer records
  d.nwg_cap = (d.tiles_cap + d.wpw - 1) / d.wpw;  // at one tile per wave: the most workgroups
  return d;
}

// Tiles per wave for a launch: one on short lists, where more workgroups in flight matter more,
// and for units of one head, whose half-tile V staging lets three one-tile workgroups run per CU
// (12 waves, each with a whole tile of loads in flight, against 8 at two tiles per wave: 69.0
// against 72.8 us on a batch of 8 long per-head lists); otherwise two on long lists (the second
// tile's loads overlap the first one's compute, and the merge reads half the records), three
// when that brings a grid that would need two rounds of `slots` resident workgroups down to one.
static inline int decode_tiles_per_wave(const DecodeShape &d, int64_t slots) {
  if (d.tiles_cap < 32 || decode_v_keys(d.nh) == 32) return 1;
  const int64_t wg2 = d.units * ((d.tiles_cap + 2 * d.wpw - 1) / (2 * d.wpw));
  const int64_t wg3 = d.units * ((d.tiles_cap + 3 * d.wpw - 1) / (3 * d.wpw));
  return (wg2 > slots && wg3 <= slots) ? 3 : 2;
}

// Records the split-K merge can stage in its workgroup's V-tile region: m, l and a weight per
// (record, head), rounded up to 16 bytes, then (narrow units) RG groups of partial f32x4 sums.
static inline int decode_merge_capacity(int nh, int D, int wpw) {
  const int nt = wpw * 64, q4 = nh * (D / 4);
  const int rg = q4 >= nt ? 1 : nt / q4;
  const int tile_bytes = wpw * decode_v_keys(nh) * (D + VPAD) * 2;
  const int red_bytes = rg > 1 ? rg * q4 * 16 : 0;
  return (tile_bytes - red_bytes - 16) / (12 * nh);
}

}  // namespace sas
