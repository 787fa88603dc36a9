// A4 / A5 / A6 in fp32: attention over the selected blocks for fp32 inputs (prefill rows and
// decode rows, gist mode included).  Same definition as the bf16 kernels (page "稀疏注意力"
// sections 1-2: softmax(q K^T / sqrt(d) + M) V; page "SAS: ...", method: log-gate in the
// logits; page "通过Gist Token的简化稀疏注意力", method items 2-3: hybrid key set), computed
// with fp32 FMA and IEEE exp so that results track an fp64 reference to ~1e-6.
//
// One wave per (query row, query head).  Keys are visited 64 at a time: lane k forms the
// logit of key k (a d-long fp32 dot product), the wave keeps a running max / sum, and the
// value rows are accumulated with the lanes spread over the head dim.  This path serves
// correctness-sized fp32 problems; the bf16 MFMA kernels carry the large workloads.
#include "common.h"

namespace sas {

template <int D>
__global__ __launch_bounds__(64) void attend_f32_kernel(
    SeqTable st, const float *__restrict__ Q, int64_t qb, int64_t qh, int64_t qt, const float *__restrict__ K,
    const float *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const float *__restrict__ GK,
    const float *__restrict__ GV, int64_t gb, int64_t gh, int64_t gt, int gist, int tq, int blk, int S,
    int QB, int G, int per_head, const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel,
    const float *__restrict__ gate, int kcap, float scale, float *__restrict__ O, int64_t ob, int64_t oh,
    int64_t ot) {
  constexpr int PER = D / 64;
  __shared__ float qs[D];
  const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int L = st.len[b];
  const int q0 = st.q0[b];
  const int pos = q0 + t;
  const int c = pos / blk;
  const int i = c - q0 / blk;
  const int s = per_head ? h : h / G;
  const int g = h / G;
  const int64_t u = ((int64_t)b * S + s) * QB + i;
  for (int e = lane; e < D; e += 64) qs[e] = Q[b * qb + (int64_t)h * qh + (int64_t)t * qt + e];
  __syncthreads();
  const int ns = nsel[u];
  const int32_t *ul = idx + u * kcap;
  float m = -INFINITY, l = 0.f;
  float acc[PER];
#pragma unroll
  for (int x = 0; x < PER; ++x) acc[x] = 0.f;

  // one 64-key chunk: keys key0 + k with K/V rows at kp/vp + k*rs; `vis` says which exist
  auto chunk = [&](const float *kp, const float *vp, int64_t rs, bool vis, float bias) {
    float logit = -INFINITY;
    if (vis) {
      const float *kr = kp + (int64_t)lane * rs;
      float d0 = 0.f;
#pragma unroll 8
      for (int e = 0; e < D; ++e) d0 = fmaf(qs[e], kr[e], d0);
      logit = d0 * scale + bias;
    }
    const float mx = wave_max(logit);
    const float mn = fmaxf(m, mx);
    if (mn == -INFINITY) return;
    const float alpha = expf(m - mn);
    const float p = vis ? expf(logit - mn) : 0.f;
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int x = 0; x < PER; ++x) acc[x] *= alpha;
    const uint64_t live = __ballot(vis);
    for (int k = 0; k < 64; ++k) {
      if (!((live >> k) & 1ull)) continue;
      const float pk = __shfl(p, k, 64);
      const float *vr = vp + (int64_t)k * rs;
#pragma unroll
      for (int x = 0; x < PER; ++x) acc[x] = fmaf(pk, vr[lane + 64 * x], acc[x]);
    }
    m = mn;
  };

  const float *kbase = K + b * kb + g * kh;
  const float *vbase = V + b * kb + g * kh;
  for (int e = 0; e < ns; ++e) {
    const int j = ul[e];
    const float bias = gate ? gate[u * kcap + e] : 0.f;
    const int end = min((j + 1) * blk, L);
    for (int key0 = j * blk; key0 < end; key0 += 64) {
      const int key = key0 + lane;
      const bool vis = key < end && key <= pos;
      chunk(kbase + (int64_t)key0 * kt, vbase + (int64_t)key0 * kt, kt, vis, bias);
    }
  }
  if (gist) {
    const float *gkb = GK + b * gb + g * gh;
    const float *gvb = GV + b * gb + g * gh;
    for (int j0 = 0; j0 < c; j0 += 64) {
      uint64_t excl = 0;
      for (int e0 = 0; e0 < ns; e0 += 64) {
        uint64_t bit = 0;
        if (e0 + lane < ns) {
          const int j = ul[e0 + lane];
          if (j >= j0 && j < j0 + 64) bit = 1ull << (j - j0);
        }
        for (int o = 32; o >= 1; o >>= 1) {
          uint32_t lo = __shfl_xor((uint32_t)bit, o, 64);
          uint32_t hi = __shfl_xor((uint32_t)(bit >> 32), o, 64);
          bit |= ((uint64_t)hi << 32) | lo;
        }
        excl |= bit;
      }
      const bool vis = (j0 + lane < c) && !((excl >> lane) & 1ull);
      chunk(gkb + (int64_t)j0 * gt, gvb + (int64_t)j0 * gt, gt, vis, 0.f);
    }
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int x = 0; x < PER; ++x) O[b * ob + (int64_t)h * oh + (int64_t)t * ot + lane + 64 * x] = acc[x] * inv;
}

hipError_t launch_attend_f32(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                             const void *K, const void *V, const int64_t *kvs, const void *gk, const void *gv,
                             const int64_t *gs, int32_t tq, int32_t sel_mode, const int32_t *idx,
                             const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                             const int64_t *os, hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  const int QB = num_qblocks(tq, p.block);
  const int gist = gk != nullptr;
  int64_t gb = 0, gh = 0, gt = 0;
  if (gist) { gb = gs[0]; gh = gs[1]; gt = gs[2]; }
  dim3 grid(tq, p.hq, p.batch);
  if (p.head_dim == 128)
    hipLaunchKernelGGL((attend_f32_kernel<128>), grid, dim3(64), 0, s, st, (const float *)Q, qs[0], qs[1], qs[2],
                       (const float *)K, (const float *)V, kvs[0], kvs[1], kvs[2], (const float *)gk,
                       (const float *)gv, gb, gh, gt, gist, tq, p.block, S, QB, p.hq / p.hkv, per_head, idx,
                       nsel, gate, kcap, scale, (float *)O, os[0], os[1], os[2]);
  else
    hipLaunchKernelGGL((attend_f32_kernel<64>), grid, dim3(64), 0, s, st, (const float *)Q, qs[0], qs[1], qs[2],
                       (const float *)K, (const float *)V, kvs[0], kvs[1], kvs[2], (const float *)gk,
                       (const float *)gv, gb, gh, gt, gist, tq, p.block, S, QB, p.hq / p.hkv, per_head, idx,
                       nsel, gate, kcap, scale, (float *)O, os[0], os[1], os[2]);
  return hipGetLastError();
}

}  // namespace sas
