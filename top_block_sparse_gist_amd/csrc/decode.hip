// A5 / A6: sparse decode (one query row per sequence and query head, at position L_b - 1).
// Page "稀疏注意力" section 5 (decode reads only the selected KV: bandwidth-bound) and
// sections 2/7 (masked softmax, computed tile by tile with an online softmax); page
// "SAS: 通过端到端优化上下文排序的简单注意力稀疏化", method (log-gate inside the softmax);
// page "通过Gist Token的简化稀疏注意力", method items 2-3 (expanded raw chunks plus the
// gist tokens of the other chunks).
//
// Split-K over 64-key tiles.  A tile is 64 raw keys of one selected block (a 128-token block
// is two tiles) or, in gist mode, 64 consecutive gist tokens.  Each wave owns one tile:
//   S^T = K Q^T  with v_mfma_f32_16x16x32_bf16 (M = 16 keys, N = 16 query heads of the unit,
//                K = 32 dims); K is read straight from HBM into the A operand (16 B per lane);
//   online softmax per head column (exp2 domain);
//   O^T += V^T P^T with the same MFMA; V goes HBM -> LDS (row-major) and is read back as
//                the A operand; P^T comes from S^T's registers without any shuffle
//                (the keys of each 32-key step are taken in the order the accumulator holds
//                them, and V^T is read in that same order).
// The 4 waves of a workgroup merge their (m, l, acc) in LDS and write one partial record;
// combine_kernel merges the partials of a unit.  All G heads of a KV group share each K/V
// load (per-group selection).
#include "common.h"

namespace sas {

static constexpr int DEC_WAVES = 4;
static constexpr int VPAD = 8;  // LDS row padding (bf16 elements) for the V tile

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D>
__global__ __launch_bounds__(DEC_WAVES * 64) void decode_bf16_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const uint16_t *__restrict__ GK,
    const uint16_t *__restrict__ GV, int64_t gb, int64_t gh, int64_t gt, int gist, int blk, int S, int G,
    int per_head, const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel,
    const float *__restrict__ gate, int kcap, float scale_log2, float *__restrict__ work,
    int nsplit_max) {
  constexpr int NKK = D / 32;   // MFMA k-steps over the head dim
  constexpr int NDT = D / 16;   // 16-dim output tiles
  constexpr int VROW = D + VPAD;
  __shared__ __attribute__((aligned(16))) uint16_t vlds[DEC_WAVES][64 * VROW];
  __shared__ float m_sh[DEC_WAVES][16], l_sh[DEC_WAVES][16];

  const int split = blockIdx.x;
  const int64_t u = blockIdx.y;
  const int b = (int)(u / S), s = (int)(u % S);
  const int g = per_head ? s / G : s;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : s * G;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  const int tpb = blk / 64;
  const int ns = nsel[u];
  const int nraw = ns * tpb;
  const int ntiles = nraw + (gist ? (c + 63) / 64 : 0);
  if (split * DEC_WAVES >= ntiles) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = split * DEC_WAVES + wave;
  const int col = lane & 15, grp = lane >> 4;

  // ---- Q^T as the B operand: lane -> head `col`, dims 32*kk + 8*grp .. +8
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < nh) v = *reinterpret_cast<const u32x4 *>(Q + b * qb + (int64_t)(h0 + col) * qh + 32 * kk + 8 * grp);
    qreg[kk] = as_bf16x8(v);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int x = 0; x < NDT; ++x) acc_o[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (t < ntiles) {
    const uint16_t *kbase, *vbase;
    int64_t rstride;
    int key0;             // position (raw) or gist index of key 0 of the tile
    int nvalid;           // keys [0, nvalid) of the tile exist
    float gl2 = 0.f;      // gate (log2 units)
    uint64_t excl = 0;    // gist mode: bit i set -> gist key0+i is not visible
    if (t < nraw) {
      const int e = t / tpb, sub = t % tpb;
      const int j = idx[u * kcap + e];
      key0 = j * blk + sub * 64;
      nvalid = min(64, L - key0);
      kbase = K + b * kb + g * kh;
      vbase = V + b * kb + g * kh;
      rstride = kt;
      if (gate) gl2 = gate[u * kcap + e] * 1.4426950408889634f;
    } else {
      key0 = (t - nraw) * 64;
      nvalid = min(64, c - key0);
      kbase = GK + b * gb + g * gh;
      vbase = GV + b * gb + g * gh;
      rstride = gt;
      // gists of selected chunks are replaced by their raw tokens: exclude them
      for (int e0 = 0; e0 < ns; e0 += 64) {
        uint64_t bit = 0;
        if (e0 + lane < ns) {
          int j = idx[u * kcap + e0 + lane];
          if (j >= key0 && j < key0 + 64) bit = 1ull << (j - key0);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          uint32_t lo = __shfl_xor((uint32_t)bit, o, 64);
          uint32_t hi = __shfl_xor((uint32_t)(bit >> 32), o, 64);
          bit |= ((uint64_t)hi << 32) | lo;
        }
        excl |= bit;
      }
    }
    // ---- issue K (A operand, straight to registers) and V (to LDS) loads
    u32x4 kreg[4][NKK];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key = mt * 16 + col;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < nvalid) v = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)(key0 + key) * rstride + 32 * kk + 8 * grp);
        kreg[mt][kk] = v;
      }
    }
    constexpr int VCH = D / 8;            // 16-byte chunks per V row
    constexpr int VLOADS = 64 * VCH / 64; // per lane
    u32x4 vreg[VLOADS];
#pragma unroll
    for (int x = 0; x < VLOADS; ++x) {
      const int e = x * 64 + lane;
      const int key = e / VCH, ch = e % VCH;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < nvalid) v = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)(key0 + key) * rstride + ch * 8);
      vreg[x] = v;
    }
    // ---- S^T = K Q^T
    f32x4 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kreg[mt][kk]), qreg[kk], a, 0, 0, 0);
      sacc[mt] = a;
    }
    // V rows to LDS (row-major, padded)
    uint16_t *vl = vlds[wave];
#pragma unroll
    for (int x = 0; x < VLOADS; ++x) {
      const int e = x * 64 + lane;
      const int key = e / VCH, ch = e % VCH;
      *reinterpret_cast<u32x4 *>(vl + key * VROW + ch * 8) = vreg[x];
    }
    // ---- softmax over the tile's keys, per head column
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = mt * 16 + 4 * grp + r;
        bool ok = key < nvalid && !((excl >> key) & 1ull);
        float v = ok ? sacc[mt][r] * scale_log2 + gl2 : -INFINITY;
        sacc[mt][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    m_run = mx;
    const float mref = (mx == -INFINITY) ? 0.f : mx;
    float ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = __builtin_amdgcn_exp2f(sacc[mt][r] - mref);
        sacc[mt][r] = p;
        ls += p;
      }
    l_run = ls;
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
    // the tile is written and read by the same wave: order the LDS accesses within the wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int dim = dt * 16 + col;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int k0 = ks * 32 + 4 * grp;
        u32x4 w;
        w[0] = (uint32_t)vl[(k0 + 0) * VROW + dim] | ((uint32_t)vl[(k0 + 1) * VROW + dim] << 16);
        w[1] = (uint32_t)vl[(k0 + 2) * VROW + dim] | ((uint32_t)vl[(k0 + 3) * VROW + dim] << 16);
        w[2] = (uint32_t)vl[(k0 + 16) * VROW + dim] | ((uint32_t)vl[(k0 + 17) * VROW + dim] << 16);
        w[3] = (uint32_t)vl[(k0 + 18) * VROW + dim] | ((uint32_t)vl[(k0 + 19) * VROW + dim] << 16);
        acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(w), preg[ks], acc_o[dt], 0, 0, 0);
      }
    }
  }
  // ---- merge the 4 waves' partials in LDS (reusing the V tiles as fp32 scratch)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();
  float *osh = reinterpret_cast<float *>(&vlds[0][0]);  // [DEC_WAVES][16][D]
  if (grp == 0) {
    m_sh[wave][col] = m_run;
    l_sh[wave][col] = l_run;
  }
  if (col < nh) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) osh[(wave * 16 + col) * D + dt * 16 + 4 * grp + r] = acc_o[dt][r];
  }
  __syncthreads();
  float *rec = work + ((u * nsplit_max + split) * nh) * (int64_t)(D + 2);
  for (int e = threadIdx.x; e < nh * D; e += DEC_WAVES * 64) {
    const int n = e / D, dim = e % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) M = fmaxf(M, m_sh[w][n]);
    const float Mr = (M == -INFINITY) ? 0.f : M;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < DEC_WAVES; ++w) {
      const float f = (m_sh[w][n] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_sh[w][n] - Mr);
      o += f * osh[(w * 16 + n) * D + dim];
      l += f * l_sh[w][n];
    }
    float *r = rec + n * (int64_t)(D + 2);
    r[dim] = o;
    if (dim == 0) {
      r[D] = M;
      r[D + 1] = l;
    }
  }
}

// Merge the split partials of one (unit, head) row; m is in log2 units.
template <typename OT, int D>
__global__ __launch_bounds__(64) void combine_kernel(SeqTable st, const float *__restrict__ work,
                                                     int nsplit_max, int gist, int blk, int S, int G,
                                                     int per_head, const int32_t *__restrict__ nsel,
                                                     OT *__restrict__ O, int64_t ob, int64_t oh) {
  const int64_t u = blockIdx.x;
  const int n = blockIdx.y;
  const int b = (int)(u / S), s = (int)(u % S);
  const int nh = per_head ? 1 : G;
  if (n >= nh) return;
  const int h = per_head ? s : s * G + n;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  const int ntiles = nsel[u] * (blk / 64) + (gist ? (c + 63) / 64 : 0);
  const int ns = (ntiles + DEC_WAVES - 1) / DEC_WAVES;
  const float *base = work + (u * nsplit_max * nh + n) * (int64_t)(D + 2);
  const int64_t rstep = (int64_t)nh * (D + 2);
  float M = -INFINITY;
  for (int x = 0; x < ns; ++x) M = fmaxf(M, base[x * rstep + D]);
  const float Mr = (M == -INFINITY) ? 0.f : M;
  constexpr int PER = D / 64;
  float o[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) o[q] = 0.f;
  float l = 0.f;
  for (int x = 0; x < ns; ++x) {
    const float *r = base + x * rstep;
    const float m = r[D];
    const float f = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - Mr);
    l += f * r[D + 1];
#pragma unroll
    for (int q = 0; q < PER; ++q) o[q] += f * r[threadIdx.x + 64 * q];
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const float v = o[q] * inv;
    OT *dst = O + b * ob + (int64_t)h * oh + threadIdx.x + 64 * q;
    if constexpr (sizeof(OT) == 2) *dst = f32_to_bf16(v);
    else *dst = v;
  }
}

size_t decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gist) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  const int nh = per_head ? 1 : p.hq / p.hkv;
  const int64_t units = (int64_t)p.batch * S;
  int maxc = (p.max_len - 1) / p.block;
  const int64_t tiles = (int64_t)kcap * (p.block / 64) + (gist ? (maxc + 63) / 64 : 0);
  const int64_t nsplit = (tiles + DEC_WAVES - 1) / DEC_WAVES;
  return (size_t)(units * nsplit * nh * (int64_t)(p.head_dim + 2) * sizeof(float));
}

template <int D>
static hipError_t decode_dispatch(const sas_problem &p, const SeqTable &st, const void *Q,
                                  const int64_t *qs, const void *K, const void *V, const int64_t *kvs,
                                  const void *gk, const void *gv, const int64_t *gs, int32_t sel_mode,
                                  const int32_t *idx, const int32_t *nsel, const float *gate,
                                  int32_t kcap, float scale, void *O, const int64_t *os, float *work,
                                  hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  const int G = p.hq / p.hkv;
  const int gist = gk != nullptr;
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  const int64_t tiles = (int64_t)kcap * (p.block / 64) + (gist ? (maxc + 63) / 64 : 0);
  const int nsplit_real = (int)((tiles + DEC_WAVES - 1) / DEC_WAVES);
  // record stride uses the capacity bound (same formula as the workspace size query)
  const int maxc_cap = (p.max_len - 1) / p.block;
  const int64_t tiles_cap = (int64_t)kcap * (p.block / 64) + (gist ? (maxc_cap + 63) / 64 : 0);
  const int nsplit_max = (int)((tiles_cap + DEC_WAVES - 1) / DEC_WAVES);
  const int64_t units = (int64_t)p.batch * S;
  const float scale_log2 = scale * 1.4426950408889634f;
  int64_t gb = 0, gh = 0, gt = 0;
  if (gist) { gb = gs[0]; gh = gs[1]; gt = gs[2]; }
  hipLaunchKernelGGL((decode_bf16_kernel<D>), dim3(nsplit_real, (unsigned)units), dim3(DEC_WAVES * 64), 0, s,
                     st, (const uint16_t *)Q, qs[0], qs[1], (const uint16_t *)K, (const uint16_t *)V, kvs[0],
                     kvs[1], kvs[2], (const uint16_t *)gk, (const uint16_t *)gv, gb, gh, gt, gist, p.block, S,
                     G, per_head, idx, nsel, gate, kcap, scale_log2, work, nsplit_max);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nh = per_head ? 1 : G;
  hipLaunchKernelGGL((combine_kernel<uint16_t, D>), dim3((unsigned)units, nh), dim3(64), 0, s, st, work,
                     nsplit_max, gist, p.block, S, G, per_head, nsel, (uint16_t *)O, os[0], os[1]);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk,
                              const void *gv, const int64_t *gs, int32_t sel_mode, const int32_t *idx,
                              const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                              const int64_t *os, float *work, hipStream_t s) {
  if (p.head_dim == 128)
    return decode_dispatch<128>(p, st, Q, qs, K, V, kvs, gk, gv, gs, sel_mode, idx, nsel, gate, kcap, scale,
                                O, os, work, s);
  return decode_dispatch<64>(p, st, Q, qs, K, V, kvs, gk, gv, gs, sel_mode, idx, nsel, gate, kcap, scale, O,
                             os, work, s);
}

}  // namespace sas
