// Two-level gist selection for decode (H-SSA).  Page "通过Gist Token的简化稀疏注意力",
// hierarchical extension: meta-gist tokens ("gists of gists") give a coarse first choice, and
// the ordinary gists inside the chosen part are then scored to pick the chunks to expand.
// Readings (the page gives no more): a group is M consecutive chunks and has a meta-gist when it
// is complete and lies before the current chunk c (groups i < c / M); level 1 opens the top-k1
// of those groups by meta-gist score, plus the trailing group (chunks floor(c/M) M .. c - 1),
// which is always open; level 2 expands the top-k2 chunks of the open groups by gist score; the
// current chunk is always attended raw.  Ties go to the lower index at both levels.
//
// One workgroup per selection unit: the unit's pooled query (its heads' mean, in LDS), the
// meta-gist scores (16 lanes per 256-byte row, partial dot products reduced with DPP inside the
// row, all loads of a few passes issued together), the level-1 top-k by one wave, the gist scores
// of the open groups' chunks in a compact row (candidate i is chunk glist[i / M] * M + i % M),
// the level-2 top-k by one wave (up to 512 candidates) or by the four waves together, and the
// mapping of the compact picks back to chunk indices.  Scores go through a small workspace row
// per unit (device-coherent stores, read back by the top-k).
#include "common.h"
#include "decode_parts.h"

namespace sas {

// a device-coherent int load (the value was stored by this workgroup in this launch)
__device__ __forceinline__ int32_t load_dev_i32(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void hssa_select_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, const uint16_t *__restrict__ GK,
    int64_t gb, int64_t gh, int64_t gt, const uint16_t *__restrict__ MK, int64_t mb, int64_t mh, int64_t mt,
    int blk, int M, int S, int G, int per_head, int k1, int k2, float scale, int kcap, int gcap,
    int32_t *__restrict__ idx, int32_t *__restrict__ nsel, int32_t *__restrict__ gidx, int32_t *__restrict__ gsel,
    float *__restrict__ work, int64_t wrow, int64_t off2, int wide) {
  constexpr int VEC = 8;          // bf16 per 16-byte load
  constexpr int TPR = D / VEC;    // lanes per row
  constexpr int RPP = 256 / TPR;  // rows per pass
  constexpr int PB = 16;          // passes whose loads are issued together (256 rows at d 128)
  __shared__ float qs[16][D];
  __shared__ float qv[D];
  __shared__ int32_t glist[512];
  __shared__ uint32_t slots[8];

  const int64_t u = blockIdx.x;
  const int b = (int)(u / S), s = (int)(u % S);
  const int g = per_head ? s / G : s;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : g * G;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  const int nm = c / M;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int cc = tid % TPR, r = tid / TPR;
  float *row1 = work + u * wrow;  // meta-gist scores [nm], then 0 for the trailing group
  float *row2 = row1 + off2;      // compact candidate scores [ncand], then 0 for the current chunk

  // ---- the unit's query: mean of its heads (summed in head order)
#pragma unroll
  for (int x = 0; x < 16 * D / 256; ++x) {
    const int e = tid + 256 * x, h = e / D, kd = e % D;
    if (h < nh) qs[h][kd] = bf16_to_f32(Q[b * qb + (int64_t)(h0 + h) * qh + kd]);
  }
  __syncthreads();
  for (int kd = tid; kd < D; kd += 256) {
    float sum = 0.f;
    for (int h = 0; h < nh; ++h) sum += qs[h][kd];
    qv[kd] = sum / (float)nh;
  }
  __syncthreads();

  // ---- scale * qv . x for n rows; rowp(i) is row i's first element, out receives score i
  auto score_rows = [&](int n, auto rowp, float *out) {
    const __amdgpu_buffer_rsrc_t ro = dev_rsrc(out, (uint32_t)(n + 1) * 4u);
    for (int base = 0; base < n; base += RPP * PB) {
      u32x4 raw[PB];
#pragma unroll
      for (int ps = 0; ps < PB; ++ps) {
        const int i = base + r + ps * RPP;
        raw[ps] = i < n ? *reinterpret_cast<const u32x4 *>(rowp(i) + cc * VEC) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int ps = 0; ps < PB; ++ps) {
        const int i = base + r + ps * RPP;
        float part = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          part = fmaf(qv[cc * VEC + 2 * x], bf16_lo(raw[ps][x]), part);
          part = fmaf(qv[cc * VEC + 2 * x + 1], bf16_hi(raw[ps][x]), part);
        }
        part = group_sum<TPR>(part);
        if (cc == 0 && i < n) store4_dev(ro, (uint32_t)i * 4u, part * scale);
      }
    }
    if (tid == 0) store4_dev(ro, (uint32_t)n * 4u, 0.f);  // the forced entry's score (no gate)
  };

  // ---- level 1: meta-gists of the complete groups; the trailing group is the forced entry
  const uint16_t *mbase = MK + b * mb + g * mh;
  score_rows(nm, [&](int i) { return mbase + (int64_t)i * mt; }, row1);
  wait_stores();
  __syncthreads();
  const int k1u = max(0, min(k1, nm));
  // one wave, with as few registers per lane as the row needs (rows of n + 1 <= 64 * NPL entries)
  auto solo_topk = [&](const float *row, int n, const Budget &bg, int cap, int32_t *out, int32_t *cnt) {
    if (n < 64) team_topk<1>(row, n, false, bg, cap, out, cnt, nullptr, SoloTeam{});
    else if (n < 128) team_topk<2>(row, n, false, bg, cap, out, cnt, nullptr, SoloTeam{});
    else if (n < 256) team_topk<4>(row, n, false, bg, cap, out, cnt, nullptr, SoloTeam{});
    else team_topk<8>(row, n, false, bg, cap, out, cnt, nullptr, SoloTeam{});
  };
  if (wave == 0) {
    const Budget b1{k1, 0, 0, 0, 0, 0};
    solo_topk(row1, nm, b1, gcap, gidx + u * gcap, gsel + u);
    wait_stores();
    for (int e = lane; e <= k1u; e += 64) glist[e] = load_dev_i32(gidx + u * gcap + e);
  }
  __syncthreads();

  // ---- level 2: gists of the open groups' chunks, compact (the trailing group, last, may be short)
  const int ncand = k1u * M + (c - nm * M);
  const uint16_t *gbase = GK + b * gb + g * gh;
  score_rows(ncand, [&](int i) { return gbase + (int64_t)(glist[i / M] * M + i % M) * gt; }, row2);
  wait_stores();
  __syncthreads();
  const Budget b2{k2, 0, 0, 0, 0, 0};
  const int k2u = max(0, min(k2, ncand));
  if (wide) {
    const GroupTeam team{slots, wave, 0};
    team_topk<8>(row2, ncand, false, b2, kcap, idx + u * kcap, nsel + u, nullptr, team);
  } else if (wave == 0) {
    solo_topk(row2, ncand, b2, kcap, idx + u * kcap, nsel + u);
  }
  wait_stores();
  __syncthreads();
  // compact picks -> chunk indices (the order is kept: candidates are ascending chunks); the
  // forced entry ncand is the current chunk
  if (wave == 0) {
    for (int e = lane; e <= k2u; e += 64) {
      const int v = load_dev_i32(idx + u * kcap + e);
      idx[u * kcap + e] = v >= ncand ? c : glist[v / M] * M + v % M;
    }
  }
}

// Workspace row per unit: meta-gist scores (+1), then the compact candidate scores (+1).
static void hssa_rows(const sas_problem &p, int32_t M, int32_t k1, int64_t *off2, int64_t *wrow, int *ncand_max) {
  const int cmax = (p.max_len - 1) / p.block;
  const int nmax = cmax / M;
  const int nc = (max(0, min(k1, nmax)) + 1) * M;
  *off2 = (nmax + 1 + 3) / 4 * 4;
  *wrow = *off2 + (nc + 1 + 3) / 4 * 4;
  *ncand_max = nc;
}

size_t hssa_select_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t M, int32_t k1) {
  int64_t off2, wrow;
  int nc;
  hssa_rows(p, M, k1, &off2, &wrow, &nc);
  const int64_t units = (int64_t)p.batch * (sel_mode == SAS_SEL_HEAD ? p.hq : p.hkv);
  return (size_t)(units * wrow) * sizeof(float);
}

int hssa_candidates_max(const sas_problem &p, int32_t M, int32_t k1) {
  int64_t off2, wrow;
  int nc;
  hssa_rows(p, M, k1, &off2, &wrow, &nc);
  return nc;
}

hipError_t launch_hssa_select(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *gk, const int64_t *gs, const void *mk, const int64_t *ms, int32_t M,
                              int32_t sel_mode, int32_t k1, int32_t k2, float scale, int32_t kcap, int32_t gcap,
                              int32_t *idx, int32_t *nsel, int32_t *gidx, int32_t *gsel, float *work, hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  int64_t off2, wrow;
  int nc;
  hssa_rows(p, M, k1, &off2, &wrow, &nc);
  const int wide = nc > 512;
  const dim3 grid((unsigned)(p.batch * S));
  if (p.head_dim == 128)
    hipLaunchKernelGGL((hssa_select_kernel<128>), grid, dim3(256), 0, s, st, (const uint16_t *)Q, qs[0], qs[1],
                       (const uint16_t *)gk, gs[0], gs[1], gs[2], (const uint16_t *)mk, ms[0], ms[1], ms[2], p.block, M,
                       S, p.hq / p.hkv, per_head, k1, k2, scale, kcap, gcap, idx, nsel, gidx, gsel, work, wrow, off2,
                       wide);
  else
    hipLaunchKernelGGL((hssa_select_kernel<64>), grid, dim3(256), 0, s, st, (const uint16_t *)Q, qs[0], qs[1],
                       (const uint16_t *)gk, gs[0], gs[1], gs[2], (const uint16_t *)mk, ms[0], ms[1], ms[2], p.block, M,
                       S, p.hq / p.hkv, per_head, k1, k2, scale, kcap, gcap, idx, nsel, gidx, gsel, work, wrow, off2,
                       wide);
  return hipGetLastError();
}

}  // namespace sas
