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
// scores are loaded once into registers as order-preserving integer keys, a search over the
// key range (first bracket from the scores' moments, then interpolation; each probe counts the
// keys at or above it with one ballot popcount per register) finds the k-th largest key, and a
// ballot/popcount compaction writes the selected blocks in ascending order (ties go to the lower
// block).
#include <algorithm>

#include "common.h"
#include "decode_parts.h"

namespace sas {

// The grid lists only live tiles: sequences in descending length (their top-k tails are the
// longest, so they start first), each as ntile x hkv workgroups, tile-major.
struct SelGrid {
  int32_t b[SAS_MAX_BATCH];          // sequence of the i-th entry
  int32_t first[SAS_MAX_BATCH + 1];  // first workgroup of the i-th entry; first[nseq] = grid size
  int32_t nseq;
};

// At most 128 VGPRs (4 workgroups per CU): the top-k's 32 registers per lane of keys would
// otherwise set the register count, and the occupancy, of every tile workgroup.
template <typename T, typename R, int D, int NPL, int TK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void select_decode_kernel(
    SeqTable st, SelGrid sg, const T *__restrict__ Q, int64_t qb, int64_t qh, const R *__restrict__ reps,
    int64_t rb, int64_t rh, int64_t rj, int gist, int blk, int hkv, int S, int G, int per_head, float scale,
    float *__restrict__ scores, int64_t ld, Budget bg, int kcap, int32_t *__restrict__ idx,
    int32_t *__restrict__ nsel, float *__restrict__ gate, uint32_t *__restrict__ counters) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[SelectLds<D>::BYTES];
  const int id = blockIdx.x;
  int lo = 0, hi = sg.nseq - 1;  // last entry with first <= id
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sg.first[mid] <= id) lo = mid;
    else hi = mid - 1;
  }
  const int rem = id - sg.first[lo];
  select_tile_body<T, R, D, NPL, TK>(rem / hkv, rem % hkv, sg.b[lo], hkv, lds, st, Q, qb, qh, reps, rb, rh, rj,
                                 gist, blk, S, G, per_head, scale, scores, ld, bg, kcap, idx, nsel, gate,
                                 counters);
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
  SelGrid sg{};
  for (int b = 0; b < p.batch; ++b) sg.b[b] = b;
  std::stable_sort(sg.b, sg.b + p.batch, [&](int x, int y) { return st.len[x] > st.len[y]; });
  sg.nseq = p.batch;
  sg.first[0] = 0;
  for (int i = 0; i < p.batch; ++i) {
    const int ntile = select_tiles((st.len[sg.b[i]] - 1) / p.block, gist);
    sg.first[i + 1] = sg.first[i] + ntile * p.hkv;
  }
  const dim3 grid((unsigned)sg.first[p.batch]);
#define SAS_SEL_LAUNCH(NPL_, TK_)                                                                          \
  hipLaunchKernelGGL((select_decode_kernel<T, R, D, NPL_, TK_>), grid, dim3(256), 0, s, st, sg, (const T *)Q, \
                     qs[0], qs[1], (const R *)reps, rs[0], rs[1], rs[2], gist, p.block, p.hkv, S, p.hq / p.hkv, \
                     per_head, scale, scores, ld, bg, kcap, idx, nsel, gate, counters)
  // coverage and shared budgets get kernels of their own, so that the others carry none of that code
  const int tk = bg.shared ? TK_SHARED : bg.coverage > 0.f ? TK_COVERAGE : TK_PLAIN;
  if (maxc <= 512) {
    if (tk == TK_SHARED) SAS_SEL_LAUNCH(8, TK_SHARED);
    else if (tk == TK_COVERAGE) SAS_SEL_LAUNCH(8, TK_COVERAGE);
    else SAS_SEL_LAUNCH(8, TK_PLAIN);
  } else {
    if (tk == TK_SHARED) SAS_SEL_LAUNCH(32, TK_SHARED);
    else if (tk == TK_COVERAGE) SAS_SEL_LAUNCH(32, TK_COVERAGE);
    else SAS_SEL_LAUNCH(32, TK_PLAIN);
  }
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
