// A4: sparse causal prefill over the gathered block list (bf16 inputs, fp32 accumulation).
// Page "稀疏注意力" sections 2, 4.5 and 7 (masked softmax attention; block-sparse so that
// matrix units see dense tiles; block-sparse FlashAttention: exact tiled attention that
// never stores the n x n matrix); page "SAS: 通过端到端优化上下文排序的简单注意力稀疏化",
// method (the selector score enters the logits in log form).
//
// A workgroup owns NW*32 query rows of one selection unit (rows x heads of the unit,
// flattened) and walks the unit's selected blocks in 64-key tiles:
//   K and V tiles are copied HBM -> LDS by the buffer unit (buffer_load ... lds): 128-row
//   workgroups (and all head-dim-64 ones) copy 16 bytes per lane, whole rows per instruction, into
//   XOR-swizzled unpadded rows; 64-row workgroups at head dim 128 copy one row per instruction
//   into padded rows.  128-row workgroups double-buffer: tile t+1 is in
//   flight while tile t is computed, and one barrier per tile hands the buffers over.  64-row
//   workgroups keep one K and one V buffer, so that twice as many fit per CU; their copies
//   overlap the phases of a tile that do not read that buffer.
//   S^T = K Q^T : v_mfma_f32_32x32x16_bf16, M = 32 keys, N = 32 query rows of the wave,
//                 K = 16 dims; Q^T stays in registers for the whole walk.
//   online softmax per query column (exp2 domain): the column's 64 logits sit in 32 VGPRs of
//                 the lane and 32 of the lane 32 apart, so the row max is one cross-half swap;
//                 max on the raw scores, then one FMA (scale, gate, running max) and one exp2
//                 per score; the accumulator is rescaled only when a column's max grows by
//                 more than 2^8.
//   O^T += V^T P^T : same MFMA, M = 32 dims, K = 16 keys; P^T is taken straight from the
//                 S^T accumulator (keys in accumulator order), V^T is read from the LDS tile
//                 in that same key order with transposing reads (ds_read_b64_tr_b16).
// Only the current block needs the causal mask.  Units are taken heavy-first (later query
// blocks select more blocks; per-head units grouped by (sequence, KV head) for MALL reuse) and
// dealt round-robin to the XCDs; the row tiles of one unit, which share its K/V tiles, run on
// the same XCD (one L2).
#include <algorithm>
#include <numeric>
#include <type_traits>

#include "common.h"

namespace sas {

__device__ __forceinline__ bf16x8 as_bf16x8p(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// NW = 4: 128 rows per workgroup, K/V double buffered (2 workgroups per CU).
// NW = 2: 64 rows per workgroup (one 64-row unit), single K and V buffers (4 workgroups per CU,
//         so 2 waves per SIMD as well): K of tile t+1 is copied during the softmax and PV of tile
//         t, V of tile t+1 during the S phase and softmax of tile t+1.
// Sequences in descending length (the order per-head units are walked in).
struct SeqOrder {
  int32_t b[SAS_MAX_BATCH];
};

template <int D, int NW, int BLK>
__global__ __launch_bounds__(NW * 64, 2) void prefill_bf16_kernel(
    SeqTable st, SeqOrder ord, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, int64_t qt,
    const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt,
    int tq, int blk, int S, int QB, int G, int per_head, int batch, int rtiles, int pchunks,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel, const float *__restrict__ gate,
    int kcap, float scale_log2, uint16_t *__restrict__ O, int64_t ob, int64_t oh, int64_t ot,
    const int32_t *__restrict__ table, int64_t tld, float *__restrict__ lse, int hq) {
  constexpr int NKK = D / 16;        // k-steps of S^T over the head dim
  constexpr int NDT = D / 32;        // 32-dim output tiles
  static_assert(D == 64 || D == 128, "head dim 64 or 128");
  constexpr bool SINGLE = NW == 2;   // single-buffered K and V
  constexpr int NBUF = SINGLE ? 1 : 2;
  // LDS tiles, two layouts (64 banks of 4 bytes; both keep the reads below conflict-free: a
  // 16-byte K operand read covers 16 consecutive rows at one chunk, an 8-byte transposing V read
  // 4 rows x 4 chunks x 2 halves):
  //  SWZ (128-row workgroups, and every D = 64 workgroup): unpadded rows of D bf16, the 16-byte
  //    chunk c of row r stored at chunk position c ^ fK(r) (K) or c ^ fV(r) (V); a 16-byte-per-lane
  //    copy writes 64 / (D / 8) whole rows per instruction.
  //  padded (64-row workgroups, D = 128): K rows D + 8 and V rows D + 32 bf16 apart, one row per
  //    copy instruction (4 bytes per lane).  On the per-head batches these run on, which are bound
  //    by L2 misses, it measured ~5 % faster than the swizzled copy.  (A D = 64 row would take
  //    2 bytes per lane, a copy width that does not land packed in LDS.)
  constexpr bool SWZ = true;
  constexpr int ROWK = SWZ ? D : D + 8, ROWV = SWZ ? D : D + 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int RPI = SWZ ? 64 / CPR : 1;  // rows per copy instruction
  constexpr int DMA = SWZ ? 16 : 4;  // bytes per lane of one copy instruction
  __shared__ __attribute__((aligned(16))) uint16_t klds2[NBUF][64 * ROWK];
  __shared__ __attribute__((aligned(16))) uint16_t vlds2[NBUF][64 * ROWV];
  const uint32_t klds_a = lds_base(klds2), vlds_a = lds_base(vlds2);  // LDS byte addresses
  auto fK = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  auto fV = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };

  // ---- workgroup -> (query block i (heavy first), sequence, selector head, row tile)
  // Workgroup k runs on XCD k % 8 (and the k-th workgroups of the XCDs start at about the same
  // time); all row tiles of a unit go to the same XCD, one after another, so they share the unit's
  // K/V tiles in that XCD's L2.
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int rt = q % rtiles;
  int s, b, i;
  if (per_head) {
    // Per-head lists share few tiles across the batch but many within one (sequence, KV head):
    // each key block is picked by several of the pair's QB x G units, whose ascending lists of
    // about the same length move through the key range at about the same pace.  So each pair runs
    // on one XCD with its units dispatched together (query blocks heavy-first, the group's heads
    // adjacent), and the units that pick a block read it while it is in that XCD's L2.  Pairs go
    // longest sequence first, pair p to XCD p % 8; with fewer pairs than XCDs, or a count that
    // does not split evenly, each pair is cut into pchunks interleaved query-block chunks
    // (pairs * pchunks is a multiple of 8), chunk cid on XCD cid % 8.
    const int hkv = S / G;
    const int upc = ((QB + pchunks - 1) / pchunks) * G;  // units per chunk
    const int qq = q / rtiles;
    const int cid = (qq / upc) * 8 + xcd;
    if (cid >= batch * hkv * pchunks) return;
    const int r = qq % upc;
    const int pair = cid / pchunks, ch = cid % pchunks;
    i = QB - 1 - (ch + pchunks * (r / G));
    if (i < 0) return;
    s = (pair % hkv) * G + r % G;
    b = ord.b[pair / hkv];
  } else {
    // per-group units, heavy-first over the whole batch, dealt round-robin to the XCDs so that
    // every XCD gets an even share of heavy and light units; slots past the last unit exit
    int rest = (q / rtiles) * 8 + xcd;
    if (rest >= QB * batch * S) return;
    s = rest % S;
    rest /= S;
    b = rest % batch;
    i = QB - 1 - rest / batch;
  }

  const int L = st.len[b];
  const int q0 = st.q0[b];
  const int c0 = q0 / blk;
  const int c = c0 + i;
  const int t_lo = max(0, c * blk - q0);
  const int t_hi = min(tq, (c + 1) * blk - q0);
  if (t_lo >= t_hi) return;
  const int rows = t_hi - t_lo;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : s * G;
  const int g = per_head ? s / G : s;
  const int R = rows * nh;
  const int r0 = rt * NW * 32;
  if (r0 >= R) return;
  const int64_t u = ((int64_t)b * S + s) * QB + i;
  const int ns = nsel[u];
  constexpr int tpb = BLK / 64;
  const int ntiles = ns * tpb;
  // the current block c is the last list entry: its tiles are the only ones needing the mask
  const int nplain = ntiles - tpb;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keeps row offsets scalar
  const int col = lane & 31, half = lane >> 5;

  // ---- this lane's query row (column of S^T)
  const int rq = r0 + wave * 32 + col;
  const bool qvalid = rq < R;
  const int qh_idx = h0 + (qvalid ? rq / rows : 0);
  const int qt_idx = t_lo + (qvalid ? rq % rows : 0);
  const int qpos = q0 + qt_idx;
  bf16x8 qreg[NKK];
  {
    const uint16_t *qp = Q + b * qb + (int64_t)qh_idx * qh + (int64_t)qt_idx * qt + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qvalid) v = *reinterpret_cast<const u32x4 *>(qp + 16 * kk);
      qreg[kk] = as_bf16x8p(v);
    }
  }

  const uint16_t *kbase = K + b * kb + g * kh;
  const uint16_t *vbase = V + b * kb + g * kh;
  const int32_t *ulist = idx + u * kcap;
  const float *glist = gate ? gate + u * kcap : nullptr;

  // Tile loads: HBM -> LDS directly (buffer_load ... lds).  One buffer resource spans the K (V)
  // slab of this (sequence, KV head) (the host checks that it fits 32-bit offsets).  Rows at or
  // past L (the tail of a partial last block) re-read row L-1: in bounds and finite, and those
  // keys are masked, so their p is exactly 0.
  //  SWZ: 16 bytes per lane, RPI rows per instruction; lane (row rin, chunk cslot) fetches the
  //    global chunk that the swizzle stores at its slot.  fK(row0 + rin) = fK(row0) ^ fK(rin) and
  //    fV(row0 + rin) = fV(rin) for row0 a multiple of RPI, so a whole tile takes a uniform row
  //    offset (soffset) plus a per-lane offset of rin rows and the swizzled chunk.
  //  padded: one row per instruction; row offset (soffset) and LDS row (M0) wave-uniform.
  constexpr int RPW = 64 / NW;       // rows of a tile each wave copies
  constexpr int NDMA = RPW / RPI;    // copy instructions per wave for one K (V) tile
  const uint32_t row_bytes = (uint32_t)(kt * 2);
  const uint32_t slab = (uint32_t)(L - 1) * row_bytes + D * 2;
  const i32x4 krs = lds_rsrc(kbase, slab), vrs = lds_rsrc(vbase, slab);
  // Paged K/V (table != nullptr): block j lives in page table[b * tld + j] (kb is the page stride);
  // a tile's copies then take a resource over its page and rows counted inside the page.
  struct Src {
    i32x4 k, v;
    int r0, rlast;  // the tile's first row and the last present row, from the resource's base
  };
  auto tile_src = [&](int t) {
    const int j = ulist[t / tpb];
    if (table) {
      const int64_t page = table[b * tld + j];
      const uint32_t pbytes = (uint32_t)(BLK - 1) * row_bytes + D * 2;
      return Src{lds_rsrc(K + page * kb + g * kh, pbytes), lds_rsrc(V + page * kb + g * kh, pbytes),
                 (t % tpb) * 64, min(BLK, L - j * BLK) - 1};
    }
    return Src{krs, vrs, j * BLK + (t % tpb) * 64, L - 1};
  };
  const int rin = lane / CPR, cslot = lane % CPR;
  const uint32_t lrow = (uint32_t)rin * row_bytes;
  const int kx = cslot ^ fK(rin);
  const uint32_t voff_v = lrow + (uint32_t)(cslot ^ fV(rin)) * 16u;
  // copy tile t's rows of K and / or V into buffer buf
  auto load_tile = [&](int t, int buf, bool k, bool v) {
    const Src sr = tile_src(t);
    const int key0 = sr.r0;
    if constexpr (SWZ) {
      if (key0 + 63 <= sr.rlast) {
#pragma unroll
        for (int x = 0; x < NDMA; ++x) {
          const int row0 = wave * RPW + x * RPI;  // wave-uniform
          const uint32_t soff = (uint32_t)(key0 + row0) * row_bytes;
          if (k) buf_load_lds<16>(sr.k, klds_a + 2u * (buf * 64 * ROWK + row0 * D), lrow + (uint32_t)(kx ^ fK(row0)) * 16u, soff);
          if (v) buf_load_lds<16>(sr.v, vlds_a + 2u * (buf * 64 * ROWV + row0 * D), voff_v, soff);
        }
      } else {
#pragma unroll
        for (int x = 0; x < NDMA; ++x) {
          const int row0 = wave * RPW + x * RPI;
          const int row = row0 + rin;
          const uint32_t roff = (uint32_t)min(key0 + row, sr.rlast) * row_bytes;
          if (k) buf_load_lds<16>(sr.k, klds_a + 2u * (buf * 64 * ROWK + row0 * D), roff + (uint32_t)(cslot ^ fK(row)) * 16u, 0u);
          if (v) buf_load_lds<16>(sr.v, vlds_a + 2u * (buf * 64 * ROWV + row0 * D), roff + (uint32_t)(cslot ^ fV(row)) * 16u, 0u);
        }
      }
    } else {
#pragma unroll
      for (int x = 0; x < RPW; ++x) {
        const int row = wave + x * NW;
        const uint32_t soff = (uint32_t)min(key0 + row, sr.rlast) * row_bytes;
        if (k) buf_load_lds<DMA>(sr.k, klds_a + 2u * (buf * 64 * ROWK + row * ROWK), lane * DMA, soff);
        if (v) buf_load_lds<DMA>(sr.v, vlds_a + 2u * (buf * 64 * ROWV + row * ROWV), lane * DMA, soff);
      }
    }
  };

  // running max (log2 units), running sum (this lane's half of the keys), O^T accumulators
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 acc_o[NDT];
#pragma unroll
  for (int x = 0; x < NDT; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc_o[x][r] = 0.f;

  // one 64-key tile; DIAG: the current block (keys beyond the row's position masked)
  auto tile = [&](int t, auto diag_tag) {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const uint16_t *klds = klds2[SINGLE ? 0 : (t & 1)];
    const uint16_t *vlds = vlds2[SINGLE ? 0 : (t & 1)];
    const int key0 = ulist[t / tpb] * BLK + (t % tpb) * 64;
    const float gl2 = glist ? glist[t / tpb] * 1.4426950408889634f : 0.f;
    // ---- S^T = K Q^T (two 32-key halves)
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x16 a;
#pragma unroll
      for (int r = 0; r < 16; ++r) a[r] = 0.f;
      const uint16_t *kr = klds + (mt * 32 + col) * ROWK;  // fK(mt * 32 + col) = fK(col)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int ch = SWZ ? (2 * kk + half) ^ fK(col) : 2 * kk + half;
        const u32x4 kv = *reinterpret_cast<const u32x4 *>(kr + 8 * ch);
        a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8p(kv), qreg[kk], a, 0, 0, 0);
      }
      sacc[mt] = a;
    }
    if constexpr (SINGLE) {
      // every wave has read K of tile t: its buffer takes tile t+1 (on the last tile, tile t
      // again: unconditional copies keep the wait counts static; nobody reads that copy)
      __syncthreads();
      load_tile(min(t + 1, ntiles - 1), 0, true, false);
    }
    // ---- max over the raw scores (scale > 0 keeps the order), causal mask on the current block
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if constexpr (DIAG) {
          const int key = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key0 + key > qpos) sacc[mt][r] = -INFINITY;
        }
        mx = fmaxf(mx, sacc[mt][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * scale_log2 + gl2;
    // lazy rescale: keep the stale running max unless some column's max grows by more than 2^8,
    // so that p = exp2(logit - m_run) stays <= 256 (exact in fp32, representable in bf16)
    if (__ballot(m_tile > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int x = 0; x < NDT; ++x)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_o[x][r] *= alpha;
    }
    // p = exp2(scale_log2 * s + gate - m_run): one FMA and one exp2 per score
    const float bias = gl2 - ((m_run == -INFINITY) ? 0.f : m_run);
    float ls = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], scale_log2, bias));
        sacc[mt][r] = p;
        ls += p;
      }
    l_run += ls;
    // ---- P^T operands: 16-key step ks uses accumulator registers 8*(ks&1) .. +7 of half ks>>1
    bf16x8 preg[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int mt = ks >> 1, r0p = 8 * (ks & 1);
      u32x4 w;
      w[0] = pack_bf16x2(sacc[mt][r0p + 0], sacc[mt][r0p + 1]);
      w[1] = pack_bf16x2(sacc[mt][r0p + 2], sacc[mt][r0p + 3]);
      w[2] = pack_bf16x2(sacc[mt][r0p + 4], sacc[mt][r0p + 5]);
      w[3] = pack_bf16x2(sacc[mt][r0p + 6], sacc[mt][r0p + 7]);
      preg[ks] = as_bf16x8p(w);
    }
    if constexpr (SINGLE) {
      // V of tile t (issued before K of tile t+1) has landed in every wave
      wait_vmcnt<NDMA>();  // the K copy of tile t+1 may still be in flight
      __syncthreads();
    }
    // ---- O^T += V^T P^T; step ks holds keys 16ks + 4half + {0..3} and 16ks + 8 + 4half + {0..3};
    //      the V^T operand (dim 32dt + col) comes from two transpose reads of the tile
    //      (row 16ks + 4half + c16/4 (+8), columns 32dt + 16chi + 4(c16%4) .. +3: chunk
    //      4dt + 2chi + (c16%4)/2, half-chunk c16%2; fV of those rows is fV(c16/4))
    const int c16 = col & 15, chi = col >> 4;
    const int fv = SWZ ? fV(c16 >> 2) : 0;
    const uint16_t *vb = vlds + (4 * half + (c16 >> 2)) * ROWV + 4 * (c16 & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint16_t *src = vb + 16 * ks * ROWV + 8 * ((4 * dt + 2 * chi + ((c16 & 3) >> 1)) ^ fv);
        const u32x2 lo = lds_read_tr16(src);
        const u32x2 hi = lds_read_tr16(src + 8 * ROWV);
        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
        acc_o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8p(w), preg[ks], acc_o[dt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) load_tile(0, 0, true, true);
  wait_stores();  // vmcnt(0): this wave's loads (Q, tile 0) have landed
  __syncthreads();
  if constexpr (SINGLE) {
    // one buffer each: after tile t, K of tile t+1 has landed and V of tile t is no longer read
    for (int t = 0; t < ntiles; ++t) {
      if (t < nplain) tile(t, std::integral_constant<bool, false>{});
      else tile(t, std::integral_constant<bool, true>{});
      wait_stores();
      __syncthreads();
      load_tile(min(t + 1, ntiles - 1), 0, false, true);
    }
    wait_stores();  // no copy into LDS may outlive the workgroup
  } else {
    // tile t+1 streams into the other buffer while tile t is computed; that buffer was last read
    // in iteration t-1, which every wave finished before the barrier that closed it
    for (int t = 0; t < nplain; ++t) {
      load_tile(t + 1, (t + 1) & 1, true, true);
      tile(t, std::integral_constant<bool, false>{});
      wait_stores();
      __syncthreads();
    }
    for (int t = max(nplain, 0); t < ntiles; ++t) {
      if (t + 1 < ntiles) load_tile(t + 1, (t + 1) & 1, true, true);
      tile(t, std::integral_constant<bool, true>{});
      wait_stores();
      __syncthreads();
    }
  }
  // ---- normalise and write O (lane holds dims 32dt + 8(r/4) + 4half + r%4 of its query)
  l_run += __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  // row log-sum-exp of the logits (natural log): p = exp2(logit log2 e - m_run) summed to l_run
  if (lse && half == 0)
    lse[((int64_t)b * hq + qh_idx) * tq + qt_idx] = (m_run + log2f(l_run)) * 0.6931471805599453f;
  const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
  uint16_t *op = O + b * ob + (int64_t)qh_idx * oh + (int64_t)qt_idx * ot;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int dim = dt * 32 + 8 * rb + 4 * half;
      u32x2 w;
      w[0] = pack_bf16x2(acc_o[dt][4 * rb + 0] * inv, acc_o[dt][4 * rb + 1] * inv);
      w[1] = pack_bf16x2(acc_o[dt][4 * rb + 2] * inv, acc_o[dt][4 * rb + 3] * inv);
      *reinterpret_cast<u32x2 *>(op + dim) = w;
    }
}

template <int D, int NW, int BLK>
static hipError_t prefill_dispatch(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                                   const void *K, const void *V, const int64_t *kvs, int32_t tq,
                                   int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                                   const float *gate, int32_t kcap, float scale, void *O, const int64_t *os,
                                   hipStream_t s, const int32_t *table, int64_t tld, float *lse) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int S = per_head ? p.hq : p.hkv;
  const int G = p.hq / p.hkv;
  const int QB = num_qblocks(tq, p.block);
  const int nh = per_head ? 1 : G;
  const int rows_max = min(tq, p.block);
  const int rtiles = cdiv(rows_max * nh, NW * 32);
  const int64_t units = (int64_t)QB * p.batch * S;
  // per-head: (sequence, KV head) pairs, each cut into pchunks query-block chunks so that the
  // chunk count is a multiple of the 8 XCDs
  const int pairs = p.batch * p.hkv;
  const int pchunks = per_head ? 8 / std::gcd(pairs, 8) : 1;
  const int64_t nwg = per_head ? 8 * cdiv64((int64_t)pairs * pchunks, 8) * (cdiv(QB, pchunks) * G) * rtiles
                               : 8 * cdiv64(units, 8) * rtiles;
  const float scale_log2 = scale * 1.4426950408889634f;
  SeqOrder ord{};
  for (int b = 0; b < p.batch; ++b) ord.b[b] = b;
  std::stable_sort(ord.b, ord.b + p.batch, [&](int x, int y) { return st.len[x] > st.len[y]; });
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NW, BLK>), dim3((unsigned)nwg), dim3(NW * 64), 0, s, st, ord,
                     (const uint16_t *)Q, qs[0], qs[1], qs[2], (const uint16_t *)K, (const uint16_t *)V, kvs[0],
                     kvs[1], kvs[2], tq, p.block, S, QB, G, per_head, p.batch, rtiles, pchunks, idx, nsel, gate, kcap,
                     scale_log2, (uint16_t *)O, os[0], os[1], os[2], table, tld, lse, p.hq);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                               const void *K, const void *V, const int64_t *kvs, int32_t tq,
                               int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                               const float *gate, int32_t kcap, float scale, void *O, const int64_t *os,
                               hipStream_t s, const int32_t *table, int64_t tld, float *lse) {
  // rows per unit: blk (x G when the group shares one list); 2 waves cover a 64-row unit
  const int nh = sel_mode == SAS_SEL_HEAD ? 1 : p.hq / p.hkv;
  const bool small = std::min(tq, p.block) * nh <= 64;
#define SAS_PF(D_, NW_, B_) \
  return prefill_dispatch<D_, NW_, B_>(p, st, Q, qs, K, V, kvs, tq, sel_mode, idx, nsel, gate, kcap, scale, O, os, s, \
                                       table, tld, lse)
#define SAS_PF_NW(D_, B_) \
  if (small) SAS_PF(D_, 2, B_);  \
  SAS_PF(D_, 4, B_)
  if (p.head_dim == 128) {
    if (p.block == 64) { SAS_PF_NW(128, 64); }
    SAS_PF_NW(128, 128);
  }
  if (p.block == 64) { SAS_PF_NW(64, 64); }
  SAS_PF_NW(64, 128);
#undef SAS_PF_NW
#undef SAS_PF
}

}  // namespace sas
