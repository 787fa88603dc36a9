// A5 / A6: sparse decode (one query row per sequence and query head, at position L_b - 1).
// Page "稀疏注意力" section 5 (decode reads only the selected KV: bandwidth-bound) and
// sections 2/7 (masked softmax, computed tile by tile with an online softmax); page
// "SAS: 通过端到端优化上下文排序的简单注意力稀疏化", method (log-gate inside the softmax);
// page "通过Gist Token的简化稀疏注意力", method items 2-3 (expanded raw chunks plus the
// gist tokens of the other chunks).
//
// Split-K over 64-key tiles, one wave per tile.  Tile t of a unit is 64 raw keys of list entry
// t / (blk/64) (a 128-token block is two tiles; padding entries -1 are empty tiles) or, past
// the raw tiles, 64 consecutive gist tokens.  The tile's block index is the only load the
// K/V loads wait for.
//   S^T = K Q^T  with v_mfma_f32_16x16x32_bf16 (M = 16 keys, N = 16 query heads of the unit,
//                K = 32 dims); K goes straight from HBM into the A operand (16 B per lane);
//   online softmax per head column (exp2 domain);
//   O^T = V^T P^T with the same MFMA; V goes HBM -> registers -> LDS (row-major) and is read
//                back as the A operand; P^T comes from S^T's registers without any shuffle
//                (each 32-key step takes the keys in accumulator order, V^T is read in that
//                same order).
// The waves of a workgroup merge their (m, l, acc) in LDS into one record; the last
// workgroup of a unit to arrive (one device-scope atomic on an arrival counter, which it
// resets) merges all records of the unit and writes O.  All G heads of a KV group share
// each K/V load (per-group selection).
#include <atomic>
#include <cstdint>

#include "common.h"
#include "decode_parts.h"

namespace sas {

// Workgroup id -> (workgroup of the unit, unit).  Workgroup i runs on XCD i % 8, each XCD with its
// own L2.  Per-head units of one (sequence, KV head) read the same K/V rows wherever their lists
// overlap (the current block, blocks every head ranks high), so with `grouped` all workgroups of
// such a pair are placed on one XCD, pairs dealt round-robin, and within a pair the G heads'
// workgroups of each list range run back to back: a tile the heads share is fetched into that
// L2 once.  Pairs past the last multiple of 8 are placed in order.  Otherwise unit-major.
__device__ __forceinline__ void decode_place(int id, int nwg, int64_t units, int G, bool grouped, int &x,
                                             int64_t &u) {
  if (!grouped) {
    u = id / nwg;
    x = id % nwg;
    return;
  }
  const int W = G * nwg;  // workgroups of one pair
  const int64_t full = units / G / 8 * 8;
  int64_t p;
  int w;
  if (id < full * W) {
    const int r = id / 8;
    p = (int64_t)(r / W) * 8 + id % 8;
    w = r % W;
  } else {
    const int64_t j = id - full * W;
    p = full + j / W;
    w = (int)(j % W);
  }
  x = w / G;
  u = p * G + w % G;
}

template <int D, int WPW, int TPW, typename OT, bool HS, int VK>
__global__ __launch_bounds__(WPW * 64) __attribute__((amdgpu_waves_per_eu(2))) void decode_bf16_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const uint16_t *__restrict__ GK,
    const uint16_t *__restrict__ GV, int64_t gb, int64_t gh, int64_t gt, int gist, int blk, int S, int G,
    int per_head, const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel, const float *__restrict__ gate,
    int kcap, float scale_log2, float *__restrict__ work, uint32_t *__restrict__ counters, OT *__restrict__ O,
    int64_t ob, int64_t oh, MetaArgs ma, PageArgs pg, int nwg, int64_t units) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[DecodeLds<D, WPW, VK>::BYTES];
  int x;
  int64_t u;
  decode_place((int)blockIdx.x, nwg, units, G, per_head && G > 1, x, u);
  decode_tile_body<D, WPW, TPW, OT, HS, VK>(x, u, nwg, lds, st, Q, qb, qh, K, V, kb, kh, kt,
                                          GK, GV, gb, gh, gt, gist, blk, S, G, per_head, idx, nsel, gate, kcap,
                                          scale_log2, work, counters, O, ob, oh, ma, pg);
}

// ---- host side -------------------------------------------------------------------------------
bool decode_merge_fits(const sas_problem &p, const SeqTable &st, int32_t sel_mode, int32_t kcap, int32_t gist,
                       int *nwg_out, int *cap_out) {
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  const DecodeShape d = decode_shape(p, sel_mode, kcap, gist, maxc);
  // validation makes no HIP call: the count is taken without the device's resident capacity, the
  // largest record count any launch of this shape uses
  const int tpw = decode_tiles_per_wave(d, INT64_MAX);
  *nwg_out = (d.tiles_cap + d.wpw * tpw - 1) / (d.wpw * tpw);
  *cap_out = decode_merge_capacity(d.nh, p.head_dim, d.wpw);
  return *nwg_out <= *cap_out;
}

size_t decode_counter_bytes(const sas_problem &p, int32_t sel_mode) {
  const DecodeShape d = decode_shape(p, sel_mode, 1, 0, 0);
  return ((size_t)d.units * 4 + 255) / 256 * 256;
}

size_t decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gist) {
  const int maxc = (p.max_len - 1) / p.block;
  DecodeShape d = decode_shape(p, sel_mode, kcap, gist, maxc);
  // arrival counters (one per unit, 256-byte aligned region) + one record per workgroup
  const size_t counters = ((size_t)d.units * 4 + 255) / 256 * 256;
  return counters + (size_t)d.units * d.nwg_cap * record_floats(d.nh, p.head_dim) * sizeof(float);
}

// Attention workgroups resident at once on the current device: as many per CU as the 160 KB LDS
// holds (the 4 V tiles of a workgroup: two at head dim 128, three at 64).
static int64_t decode_resident_workgroups(int head_dim) {
  static std::atomic<int> cus[64];
  const int per_cu = 160 * 1024 / (head_dim == 128 ? DecodeLds<128, 4>::BYTES : DecodeLds<64, 4>::BYTES);
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    n = cus[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
      if (n > 0) cus[dev].store(n, std::memory_order_relaxed);
    }
  }
  if (n <= 0) n = 256;
  return (int64_t)per_cu * n;
}

template <int D, int WPW, int TPW, bool HS, int VK>
static hipError_t decode_launch_vk(const sas_problem &p, const SeqTable &st, const DecodeShape &d, int nwg,
                                const void *Q, const int64_t *qs, const void *K, const void *V, const int64_t *kvs,
                                const void *gk, const void *gv, int64_t gb, int64_t gh, int64_t gt, int gist,
                                int per_head, const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                float scale_log2, float *work, uint32_t *counters, void *O, const int64_t *os,
                                const MetaArgs &ma, const PageArgs &pg, hipStream_t s) {
  if ((uint64_t)nwg * (uint64_t)d.units * WPW * 64 > 0xFFFFFFFFull) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_bf16_kernel<D, WPW, TPW, uint16_t, HS, VK>), dim3((unsigned)(nwg * d.units)), dim3(WPW * 64), 0,
                     s, st, (const uint16_t *)Q, qs[0], qs[1], (const uint16_t *)K, (const uint16_t *)V, kvs[0],
                     kvs[1], kvs[2], (const uint16_t *)gk, (const uint16_t *)gv, gb, gh, gt, gist, p.block, d.S,
                     p.hq / p.hkv, per_head, idx, nsel, gate, kcap, scale_log2, work, counters, (uint16_t *)O, os[0],
                     os[1], ma, pg, nwg, d.units);
  return hipGetLastError();
}

// One-tile-per-wave launches over units of one head stage V in half tiles (decode_v_keys): with
// half the LDS, three such workgroups fit per CU instead of two (their registers allow three).
template <int D, int WPW, int TPW, bool HS>
static hipError_t decode_launch(const sas_problem &p, const SeqTable &st, const DecodeShape &d, int nwg,
                                const void *Q, const int64_t *qs, const void *K, const void *V, const int64_t *kvs,
                                const void *gk, const void *gv, int64_t gb, int64_t gh, int64_t gt, int gist,
                                int per_head, const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                float scale_log2, float *work, uint32_t *counters, void *O, const int64_t *os,
                                const MetaArgs &ma, const PageArgs &pg, hipStream_t s) {
  if constexpr (TPW == 1)
    if (decode_v_keys(d.nh) == 32)
      return decode_launch_vk<D, WPW, TPW, HS, 32>(p, st, d, nwg, Q, qs, K, V, kvs, gk, gv, gb, gh, gt, gist, per_head,
                                                 idx, nsel, gate, kcap, scale_log2, work, counters, O, os, ma, pg, s);
  return decode_launch_vk<D, WPW, TPW, HS, 64>(p, st, d, nwg, Q, qs, K, V, kvs, gk, gv, gb, gh, gt, gist, per_head,
                                               idx, nsel, gate, kcap, scale_log2, work, counters, O, os, ma, pg, s);
}

hipError_t launch_decode_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk,
                              const void *gv, const int64_t *gs, int32_t sel_mode, const int32_t *idx,
                              const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                              const int64_t *os, float *workspace, hipStream_t s, const int32_t *table,
                              int64_t tld) {
  const PageArgs pg{table, tld};
  const int gist = gk != nullptr;
  const int per_head = sel_mode == SAS_SEL_HEAD;
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  // the record layout and the workgroup count follow the capacity shape; only nwg launches
  const DecodeShape cap = decode_shape(p, sel_mode, kcap, gist, (p.max_len - 1) / p.block);
  DecodeShape d = decode_shape(p, sel_mode, kcap, gist, maxc);
  d.wpw = cap.wpw;
  const int tpw = decode_tiles_per_wave(d, decode_resident_workgroups(p.head_dim));
  const int nwg = (d.tiles_cap + d.wpw * tpw - 1) / (d.wpw * tpw);
  uint32_t *counters = reinterpret_cast<uint32_t *>(workspace);
  const size_t cbytes = ((size_t)d.units * 4 + 255) / 256 * 256;
  float *work = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + cbytes);
  int64_t gb = 0, gh = 0, gt = 0;
  if (gist) { gb = gs[0]; gh = gs[1]; gt = gs[2]; }
  const float sl2 = scale * 1.4426950408889634f;
#define SAS_DEC(D_, T_)                                                                                          \
  return decode_launch<D_, 4, T_, false>(p, st, d, nwg, Q, qs, K, V, kvs, gk, gv, gb, gh, gt, gist, per_head, idx, \
                                         nsel, gate, kcap, sl2, work, counters, O, os, MetaArgs{}, pg, s)
  if (p.head_dim == 128) {
    if (tpw == 3) SAS_DEC(128, 3);
    if (tpw == 2) SAS_DEC(128, 2);
    SAS_DEC(128, 1);
  }
  if (tpw == 3) SAS_DEC(64, 3);
  if (tpw == 2) SAS_DEC(64, 2);
  SAS_DEC(64, 1);
#undef SAS_DEC
}

// ---- two-level gist mode (meta-gists) ------------------------------------------------------
// Tiles per unit: gcap opened-group tiles, nmt meta-gist tiles, then kcap raw tiles.
static DecodeShape hssa_shape(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gcap, int nmt) {
  DecodeShape d = decode_shape(p, sel_mode, kcap, 0, 0);
  d.tiles_cap += gcap + nmt;
  d.nwg_cap = (d.tiles_cap + d.wpw - 1) / d.wpw;
  return d;
}

static int hssa_meta_tiles(int maxc, int M) { return (maxc / M + 63) / 64; }

bool hssa_merge_fits(const sas_problem &p, const SeqTable &st, int32_t sel_mode, int32_t kcap, int32_t gcap,
                     int32_t M, int *nwg_out, int *cap_out) {
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  const DecodeShape d = hssa_shape(p, sel_mode, kcap, gcap, hssa_meta_tiles(maxc, M));
  const int tpw = decode_tiles_per_wave(d, INT64_MAX);
  *nwg_out = (d.tiles_cap + d.wpw * tpw - 1) / (d.wpw * tpw);
  *cap_out = decode_merge_capacity(d.nh, p.head_dim, d.wpw);
  return *nwg_out <= *cap_out;
}

size_t hssa_decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gcap, int32_t M) {
  const DecodeShape d = hssa_shape(p, sel_mode, kcap, gcap, hssa_meta_tiles((p.max_len - 1) / p.block, M));
  const size_t counters = ((size_t)d.units * 4 + 255) / 256 * 256;
  return counters + (size_t)d.units * d.nwg_cap * record_floats(d.nh, p.head_dim) * sizeof(float);
}

hipError_t launch_hssa_decode(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk, const void *gv,
                              const int64_t *gs, const void *mk, const void *mv, const int64_t *ms, int32_t M,
                              int32_t sel_mode, const int32_t *idx, const int32_t *nsel, int32_t kcap,
                              const int32_t *gidx, int32_t gcap, float scale, void *O, const int64_t *os,
                              float *workspace, hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  const int nmt = hssa_meta_tiles(maxc, M);
  const DecodeShape d = hssa_shape(p, sel_mode, kcap, gcap, nmt);
  const int tpw = decode_tiles_per_wave(d, decode_resident_workgroups(p.head_dim));
  const int nwg = (d.tiles_cap + d.wpw * tpw - 1) / (d.wpw * tpw);
  uint32_t *counters = reinterpret_cast<uint32_t *>(workspace);
  const size_t cbytes = ((size_t)d.units * 4 + 255) / 256 * 256;
  float *work = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + cbytes);
  const MetaArgs ma{(const uint16_t *)mk, (const uint16_t *)mv, ms[0], ms[1], ms[2], gidx, M, gcap, nmt};
  const float sl2 = scale * 1.4426950408889634f;
#define SAS_HDEC(D_, T_)                                                                                           \
  return decode_launch<D_, 4, T_, true>(p, st, d, nwg, Q, qs, K, V, kvs, gk, gv, gs[0], gs[1], gs[2], 0, per_head, \
                                        idx, nsel, nullptr, kcap, sl2, work, counters, O, os, ma, PageArgs{}, s)
  if (p.head_dim == 128) {
    if (tpw == 3) SAS_HDEC(128, 3);
    if (tpw == 2) SAS_HDEC(128, 2);
    SAS_HDEC(128, 1);
  }
  if (tpw == 3) SAS_HDEC(64, 3);
  if (tpw == 2) SAS_HDEC(64, 2);
  SAS_HDEC(64, 1);
#undef SAS_HDEC
}

}  // namespace sas
