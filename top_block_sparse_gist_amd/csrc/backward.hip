// Backward of A4: gradients of the gated sparse causal prefill (bf16 inputs, fp32 gradients).
// Page "稀疏注意力" sections 2 and 7 (the masked softmax attention the forward computes, block by
// block); page "SAS: 通过端到端优化上下文排序的简单注意力稀疏化", method, core modules 2-3 (the
// selector score enters the logits through a log-softmax over the kept set, so the loss reaches the
// scores through it).
//
// For each selection unit and each (row, head) of it, the forward takes logits
// l = scale q.k + g(block of k) over the unit's visible keys, P = softmax(l) and O = P V.  Given dO:
//   D_row = dO . O,  dP = dO V^T,  dS = P (dP - D_row)
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO,  dgate(j) = sum of dS over the keys of block j
//   dscore(j) = dgate(j) - exp(g(j)) sum_j' dgate(j')      (g = s - logsumexp of the list's scores)
// Kernels, in stream order:
//   bwd_clear  zero the selection bitmap and per-block counts (a fill kernel)
//   bwd_mark   one lane per list entry: set the unit's bit in its block's row, count it, note the
//              entry's list position
//   bwd_plan   one workgroup per (sequence, KV head): cut each block's unit list into segments of
//              bounded work; zero the dK/dV rows of blocks cut into more than one segment
//   bwd_dq     a unit's row tile, as in the forward (S^T = K Q^T with Q^T in registers): pass 1 walks
//              the list for each row's log-sum-exp (skipped when the forward's is given), pass 2
//              recomputes P, dP^T = V dO^T and dS, and
//              accumulates dQ^T += K^T dS^T (transposing LDS reads of the K tile); writes LSE, D_row
//              and per-32-row partial sums of dgate
//   bwd_dkv    a (block, segment): K^T in registers and V in LDS while the units that selected the
//              block stream their rows through LDS 32 at a time (one wave per 32 keys, or two
//              that split the head dim of dK and dV for 64-key blocks); S = Q K^T, dP = dO V^T,
//              then dV^T += dO^T P and dK^T += Q^T dS (transposing LDS reads).  A step of 32 rows of
//              one head is copied through a buffer resource based at its first row (lane offsets
//              fixed for the whole walk), and only steps on a causal or length edge are masked.
//   bwd_gate   per unit: dgate (partials summed in a fixed order) and dscore
// dQ, dgate and dscore are deterministic; dK and dV too, except in blocks whose unit list was cut
// into several segments (their partial sums meet in fp32 atomic adds).
#include <algorithm>
#include <numeric>
#include <type_traits>

#include "common.h"

namespace sas {

namespace {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// XOR swizzle of the 16-byte chunks of an LDS row (rows of D bf16, unpadded): row-operand reads
// (16 consecutive rows at one logical chunk) stay on distinct banks.  TR: the tile is also read by
// transposing reads (4 consecutive rows, 4-row aligned, over one aligned group of 4 chunks).  At
// D = 128 (16 chunks per row, a row per pass of the 64 banks) that swizzle sends the low two row
// bits to the chunk's high two bits and the next two row bits to its low two bits, so 4 aligned
// rows also move an aligned 4-chunk group to 4 distinct groups (r & 15 puts them on one group:
// four-way bank conflicts).  The dK/dV kernel's staged rows take it; in the dQ kernel the extra
// address arithmetic spilled registers and cost more than the conflicts it removed.
template <int D, bool TR = false>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return TR ? (((r & 3) << 2) | ((r >> 2) & 3)) : (r & 15);
  return (r >> 1) & 7;
}
// Geometry of selection unit u = (b * S + s) * QB + i.
struct UnitGeo {
  int b, s, i, c, t_lo, rows, h0, nh, g;
};
__device__ __forceinline__ UnitGeo unit_geo(const SeqTable &st, int64_t u, int S, int QB, int G, int per_head,
                                            int tq, int blk) {
  UnitGeo x;
  x.i = (int)(u % QB);
  x.s = (int)((u / QB) % S);
  x.b = (int)(u / ((int64_t)QB * S));
  const int q0 = st.q0[x.b];
  x.c = q0 / blk + x.i;
  x.t_lo = max(0, x.c * blk - q0);
  const int t_hi = min(tq, (x.c + 1) * blk - q0);
  x.rows = max(0, t_hi - x.t_lo);
  x.nh = per_head ? 1 : G;
  x.h0 = per_head ? x.s : x.s * G;
  x.g = per_head ? x.s / G : x.s;
  return x;
}

// 64 rows of a K or V slab into a swizzled LDS tile at LDS byte address lds: NW waves, 16 bytes per
// lane, rows past rlast
// re-read row rlast (in bounds; their keys are masked).
template <int D, int NW, bool TR = false>
__device__ __forceinline__ void copy_tile(i32x4 rs, uint32_t lds, int key0, int rlast,
                                          uint32_t row_bytes, int wave, int lane) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, RPW = 64 / NW, NDMA = RPW / RPI;
  static_assert(NDMA >= 1, "rows per wave");
  const int rin = lane / CPR, cslot = lane % CPR;
#pragma unroll
  for (int x = 0; x < NDMA; ++x) {
    const int row0 = wave * RPW + x * RPI;
    const int row = row0 + rin;
    const uint32_t roff = (uint32_t)min(key0 + row, rlast) * row_bytes;
    buf_load_lds<16>(rs, lds + 2u * (row0 * D), roff + (uint32_t)(cslot ^ swz<D, TR>(row)) * 16u, 0u);
  }
}

// C = A B^T over the head dim for 32 LDS rows (A: rows row0 .. row0+31 of a swizzled tile, one
// row per lane column) and a register operand (8 bf16 of the head dim per k-step).
template <int D>
__device__ __forceinline__ f32x16 rows_dot(const uint16_t *lds, int row0, const bf16x8 *breg, int col, int half) {
  constexpr int NKK = D / 16;
  f32x16 a;
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
  const int row = row0 + col;
  const uint16_t *p = lds + row * D;
  const int f = swz<D>(row);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(p + 8 * ((2 * kk + half) ^ f));
    a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(v), breg[kk], a, 0, 0, 0);
  }
  return a;
}

// Transposed operand of a swizzled LDS tile for k-step ks: lane (col, half) gets column 32 dt + col
// of rows 16 ks + 4 half + {0..3} and 16 ks + 8 + 4 half + {0..3}, the row order in which an
// accumulator's registers 8 (ks & 1) .. + 7 hold their rows (keys).
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t *lds, int ks, int dt, int col, int half) {
  const int c16 = col & 15, chi = col >> 4;
  const int rlo = 16 * ks + 4 * half + (c16 >> 2), rhi = rlo + 8;
  const int chunk = 4 * dt + 2 * chi + ((c16 & 3) >> 1);
  const int sub = 4 * (c16 & 1);
  const u32x2 lo = lds_read_tr16(lds + rlo * D + 8 * (chunk ^ swz<D>(rlo)) + sub);
  const u32x2 hi = lds_read_tr16(lds + rhi * D + 8 * (chunk ^ swz<D>(rhi)) + sub);
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf8(w);
}

// Per-lane element offsets of the reads above, as three bases that an immediate XOR completes (a
// loop keeps three registers of addresses; the k-step, the tensor and the buffer only add constants):
//   row(kk) = rb ^ 16 kk: chunk 2kk + half of row `col` (rows_dot's read with row0 = 0; the same
//            offsets serve row0 = 32w, since the swizzle of row 32w + col is that of row col)
//   tlo(x) = tlb ^ 32 x, thi(x) = thb ^ 32 x: tr_operand's two reads at ks = 0 for output tile
//            dt = dt0 + x (dt0 a multiple of the tile count; ks adds 16 ks rows)
// The chunk index is (2kk) ^ (half ^ swizzle) and (4dt) ^ (2chi + bit) ^ swizzle, and 8 x chunk sits
// below the row's multiple of D, so the XOR with 16 kk or 32 dt acts on the bits that hold kk or dt.
template <int D, bool TR = false>
struct LdsOffsets {
  int rb, tlb, thb;
  __device__ __forceinline__ LdsOffsets(int col, int half, int dt0 = 0) {
    rb = col * D + 8 * (swz<D, TR>(col) ^ half);
    const int c16 = col & 15, chi = col >> 4;
    const int rlo = 4 * half + (c16 >> 2), rhi = rlo + 8;
    const int sub = 4 * (c16 & 1);
    const int m = 2 * chi + ((c16 & 3) >> 1);
    tlb = (rlo * D + 8 * (m ^ swz<D, TR>(rlo)) + sub) ^ (32 * dt0);
    thb = (rhi * D + 8 * (m ^ swz<D, TR>(rhi)) + sub) ^ (32 * dt0);
  }
};

// registers 8 (ks & 1) .. + 7 of accumulator a as a bf16 B operand
__device__ __forceinline__ bf16x8 pack_operand(const f32x16 &a, int r0) {
  u32x4 w;
  w[0] = pack_bf16x2(a[r0 + 0], a[r0 + 1]);
  w[1] = pack_bf16x2(a[r0 + 2], a[r0 + 3]);
  w[2] = pack_bf16x2(a[r0 + 4], a[r0 + 5]);
  w[3] = pack_bf16x2(a[r0 + 6], a[r0 + 7]);
  return as_bf8(w);
}

}  // namespace

// ---------------------------------------------------------------------------------------------
// selection bitmap
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_clear_kernel(uint32_t *p, int64_t n) {
  for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = 0u;
}

__global__ __launch_bounds__(256) void bwd_mark_kernel(const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel,
                                                      int64_t units, int kcap, int S, int QB, int G, int per_head,
                                                      int hkv, int NBm, int W, int UG, uint32_t *bits,
                                                      int32_t *counts, int16_t *epos) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t u = gid / kcap;
  const int e = (int)(gid % kcap);
  if (u >= units || e >= nsel[u]) return;
  const int j = idx[u * kcap + e];
  if (j < 0 || j >= NBm) return;
  const int i = (int)(u % QB), s = (int)((u / QB) % S);
  const int b = (int)(u / ((int64_t)QB * S));
  const int g = per_head ? s / G : s;
  const int ug = per_head ? i * G + s % G : i;
  const int64_t row = (int64_t)(b * hkv + g) * NBm + j;
  atomicOr(&bits[row * W + (ug >> 5)], 1u << (ug & 31));
  atomicAdd(&counts[row], 1);
  if (epos) epos[row * UG + ug] = (int16_t)e;
}

// Work items of the dK/dV kernel: block kt, matches first .. first+count-1 of its unit list (in
// unit order), multi = the block has several items.
struct BwdItem {
  int32_t kt, first, count, multi;
};

// Workgroup-wide exclusive prefix sum over 256 threads (4 waves); total in *tot.
__device__ __forceinline__ int block_scan256(int v, int *lds4, int *tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds4[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int t = lds4[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();
  *tot = all;
  return before + x - v;
}

template <int D>
__global__ __launch_bounds__(256) void bwd_plan_kernel(SeqTable st, int hkv, int NBm, int blk, int segm, int cap,
                                                      const int32_t *__restrict__ counts, BwdItem *items,
                                                      int32_t *icount, float *dK, float *dV, int64_t kb, int64_t kh,
                                                      int64_t kt_) {
  __shared__ int scan4[4];
  __shared__ int multi[256];
  __shared__ int nmulti;
  const int pair = blockIdx.x, tid = threadIdx.x;
  const int b = pair / hkv, g = pair % hkv;
  const int L = st.len[b];
  const int nb = cdiv(L, blk);
  int off = 0;
  for (int k0 = 0; k0 < nb; k0 += 256) {
    if (tid == 0) nmulti = 0;
    const int kt = k0 + tid;  // block
    const bool valid = kt < nb;
    const int cnt = valid ? counts[(int64_t)pair * NBm + kt] : 0;
    const int nseg = valid ? max(1, cdiv(cnt, segm)) : 0;
    int tot;
    const int ex = block_scan256(nseg, scan4, &tot);
    for (int s = 0; s < nseg; ++s) {
      const int n = off + ex + s;
      if (n < cap) items[(int64_t)pair * cap + n] = BwdItem{kt, s * segm, min(segm, cnt - s * segm), nseg > 1};
    }
    if (nseg > 1) multi[atomicAdd(&nmulti, 1)] = kt;
    __syncthreads();
    // blocks cut into several segments accumulate with atomic adds: clear their rows first
    const int nm = nmulti;
    constexpr int V4 = D / 4;  // float4 per row
    for (int x = tid; x < nm * blk * V4; x += 256) {
      const int m = x / (blk * V4), r = (x / V4) % blk, c4 = x % V4;
      const int key = multi[m] * blk + r;
      if (key < L) {
        const int64_t o = (int64_t)b * kb + (int64_t)g * kh + (int64_t)key * kt_ + 4 * c4;
        *reinterpret_cast<f32x4 *>(dK + o) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4 *>(dV + o) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    off += tot;
    __syncthreads();
  }
  if (tid == 0) icount[pair] = min(off, cap);
}

// ---------------------------------------------------------------------------------------------
// dQ, row log-sum-exp, D_row and dgate partials
// ---------------------------------------------------------------------------------------------
template <int D, int NW, int BLK>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, int64_t qt, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const uint16_t *__restrict__ O,
    const uint16_t *__restrict__ dO, int64_t ob, int64_t oh, int64_t ot, int tq, int S, int QB, int G, int per_head,
    int batch, int hq, int rtiles, const int32_t *__restrict__ idx, const int32_t *__restrict__ nsel,
    const float *__restrict__ gate, int kcap, float scale_log2, float scale, float *__restrict__ dQ, int64_t dqb,
    int64_t dqh, int64_t dqt, float *__restrict__ lse_ws, float *__restrict__ dd_ws, float *__restrict__ gpart,
    int gslots, const float *__restrict__ lse_in) {
  constexpr int NKK = D / 16, NDT = D / 32, tpb = BLK / 64;
  // 64-row workgroups keep one K and one V buffer (32 KiB at d 128), so that four fit per CU and
  // their copies overlap across workgroups; 128-row workgroups double-buffer (tile t+1 in flight
  // while tile t is computed)
  constexpr int NBUF = NW == 2 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint16_t klds[NBUF][64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vlds[NBUF][64 * D];

  // workgroup -> (query block heavy-first, sequence, selector head, row tile); the row tiles of a
  // unit run on one XCD and share its K/V tiles in that L2
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int rt = q % rtiles;
  int rest = (q / rtiles) * 8 + xcd;
  if (rest >= QB * batch * S) return;
  const int s = rest % S;
  rest /= S;
  const int b = rest % batch;
  const int i = QB - 1 - rest / batch;
  const int64_t u = ((int64_t)b * S + s) * QB + i;
  const UnitGeo ug = unit_geo(st, u, S, QB, G, per_head, tq, BLK);
  const int R = ug.rows * ug.nh;
  const int r0 = rt * NW * 32;
  if (ug.rows <= 0 || r0 >= R) return;
  const int ns = nsel[u];
  const int ntiles = ns * tpb;
  const int nplain = ntiles - tpb;  // the current block (last entry) needs the causal mask
  const int L = st.len[b], q0 = st.q0[b];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int rq = r0 + wave * 32 + col;
  const bool qvalid = rq < R;
  const int h = ug.h0 + (qvalid ? rq / ug.rows : 0);
  const int t = ug.t_lo + (qvalid ? rq % ug.rows : 0);
  const int qpos = q0 + t;

  // Q^T, dO^T operands and D_row = dO . O (this lane's half of the head dim, then the other half)
  bf16x8 qreg[NKK], doreg[NKK];
  float drow = 0.f;
  {
    const uint16_t *qp = Q + b * qb + (int64_t)h * qh + (int64_t)t * qt + 8 * half;
    const int64_t oo = b * ob + (int64_t)h * oh + (int64_t)t * ot + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 vq = {0u, 0u, 0u, 0u}, vd = vq, vo = vq;
      if (qvalid) {
        vq = *reinterpret_cast<const u32x4 *>(qp + 16 * kk);
        vd = *reinterpret_cast<const u32x4 *>(dO + oo + 16 * kk);
        vo = *reinterpret_cast<const u32x4 *>(O + oo + 16 * kk);
      }
      qreg[kk] = as_bf8(vq);
      doreg[kk] = as_bf8(vd);
#pragma unroll
      for (int x = 0; x < 4; ++x) drow += bf16_lo(vd[x]) * bf16_lo(vo[x]) + bf16_hi(vd[x]) * bf16_hi(vo[x]);
    }
    drow += __shfl_xor(drow, 32, 64);
  }

  const int32_t *ulist = idx + u * kcap;
  const float *glist = gate ? gate + u * kcap : nullptr;
  const uint32_t row_bytes = (uint32_t)(kt * 2);
  const uint32_t slab = (uint32_t)(L - 1) * row_bytes + D * 2;
  const i32x4 krs = lds_rsrc(K + b * kb + ug.g * kh, slab);
  const i32x4 vrs = lds_rsrc(V + b * kb + ug.g * kh, slab);
  auto key0_of = [&](int tt) { return ulist[tt / tpb] * BLK + (tt % tpb) * 64; };
  auto load = [&](int tt, int buf, bool withv) {
    const int k0 = key0_of(tt);
    copy_tile<D, NW>(krs, lds_base(klds) + 2u * (buf * 64 * D), k0, L - 1, row_bytes, wave, lane);
    if (withv) copy_tile<D, NW>(vrs, lds_base(vlds) + 2u * (buf * 64 * D), k0, L - 1, row_bytes, wave, lane);
  };
  // S^T of tile tt (two 32-key halves), keys past the row's position at -inf on the current block
  auto scores = [&](int tt, f32x16 *sacc) {
    const uint16_t *kl = klds[NBUF == 2 ? (tt & 1) : 0];
    sacc[0] = rows_dot<D>(kl, 0, qreg, col, half);
    sacc[1] = rows_dot<D>(kl, 32, qreg, col, half);
    if (tt >= nplain) {
      const int k0 = key0_of(tt);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = mt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (k0 + key > qpos) sacc[mt][r] = -INFINITY;
        }
    }
  };

  // ---- pass 1: running max and sum (log2 units) -> lse2 = log2 sum_k exp2(l_k log2 e); skipped
  //      when the forward's log-sum-exp is given
  float m_run = -INFINITY, l_run = 0.f;
  const int ntiles1 = lse_in ? 0 : ntiles;
  if (ntiles1 > 0) load(0, 0, false);
  wait_stores();
  __syncthreads();
  for (int tt = 0; tt < ntiles1; ++tt) {
    if (NBUF == 2 && tt + 1 < ntiles1) load(tt + 1, (tt + 1) & 1, false);
    f32x16 sacc[2];
    scores(tt, sacc);
    const float gl2 = glist ? glist[tt / tpb] * LOG2E : 0.f;
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_tile = (mx == -INFINITY) ? -INFINITY : mx * scale_log2 + gl2;
    const float m_new = fmaxf(m_run, m_tile);
    if (m_new != -INFINITY) {
      l_run *= __builtin_amdgcn_exp2f(m_run - m_new);
      const float bias = gl2 - m_new;
      float ls = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) ls += __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], scale_log2, bias));
      l_run += ls;
      m_run = m_new;
    }
    if constexpr (NBUF == 1) {
      __syncthreads();  // every wave has read tile tt
      if (tt + 1 < ntiles1) load(tt + 1, 0, false);
    }
    wait_stores();
    __syncthreads();
  }
  l_run += __shfl_xor(l_run, 32, 64);
  float lse2 = qvalid && l_run > 0.f ? m_run + log2f(l_run) : INFINITY;
  if (lse_in) lse2 = qvalid ? lse_in[((int64_t)b * hq + h) * tq + t] * LOG2E : INFINITY;

  // ---- pass 2: P, dP^T, dS^T; dQ^T += K^T dS^T; dgate partials per block
  f32x16 acc[NDT];
#pragma unroll
  for (int x = 0; x < NDT; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[x][r] = 0.f;
  const int slot = r0 / 32 + wave;
  const bool wave_rows = r0 + wave * 32 < R;
  float gsum = 0.f;
  if (ntiles > 0) load(0, 0, true);
  wait_stores();
  __syncthreads();
  for (int tt = 0; tt < ntiles; ++tt) {
    if (NBUF == 2 && tt + 1 < ntiles) load(tt + 1, (tt + 1) & 1, true);
    f32x16 sacc[2];
    scores(tt, sacc);
    const float gl2 = glist ? glist[tt / tpb] * LOG2E : 0.f;
    const float bias = gl2 - lse2;
    const uint16_t *vl = vlds[NBUF == 2 ? (tt & 1) : 0];
    f32x16 dp[2];
    dp[0] = rows_dot<D>(vl, 0, doreg, col, half);
    dp[1] = rows_dot<D>(vl, 32, doreg, col, half);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[mt][r], scale_log2, bias));
        const float ds = p * (dp[mt][r] - drow);
        sacc[mt][r] = ds;
        gsum += ds;
      }
    const uint16_t *kl = klds[NBUF == 2 ? (tt & 1) : 0];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 dsop = pack_operand(sacc[ks >> 1], 8 * (ks & 1));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<D>(kl, ks, dt, col, half), dsop, acc[dt], 0, 0, 0);
    }
    if (gpart && tt % tpb == tpb - 1) {
      const float gs = wave_sum(gsum);
      if (lane == 0 && wave_rows) gpart[((int64_t)u * gslots + slot) * kcap + tt / tpb] = gs;
      gsum = 0.f;
    }
    if constexpr (NBUF == 1) {
      __syncthreads();  // every wave has read tile tt
      if (tt + 1 < ntiles) load(tt + 1, 0, true);
    }
    wait_stores();
    __syncthreads();
  }
  if (!qvalid) return;
  // ---- dQ = scale * (dQ^T)^T (lane holds dims 32dt + 8(r/4) + 4half + r%4 of its row), LSE, D
  float *dqp = dQ + b * dqb + (int64_t)h * dqh + (int64_t)t * dqt;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const f32x4 v = {acc[dt][4 * rb] * scale, acc[dt][4 * rb + 1] * scale, acc[dt][4 * rb + 2] * scale,
                       acc[dt][4 * rb + 3] * scale};
      *reinterpret_cast<f32x4 *>(dqp + dt * 32 + 8 * rb + 4 * half) = v;
    }
  if (half == 0) {
    const int64_t o = ((int64_t)b * hq + h) * tq + t;
    lse_ws[o] = lse2;
    dd_ws[o] = drow;
  }
}

// ---------------------------------------------------------------------------------------------
// dK, dV
// ---------------------------------------------------------------------------------------------
// One workgroup per (block j, segment of its unit list), BLK / 32 waves, wave w owning keys
// 32w .. 32w+31 of the block: K^T of those keys stays in registers and V in LDS for the whole walk,
// while the units' rows stream through LDS 32 at a time (double-buffered: the copy of the next
// 32 rows overlaps the compute of these).  A loaded row serves BLK keys.
// NDH waves share each 32 keys, wave dh accumulating dK and dV over head-dim tiles
// [dh NDT / NDH, (dh + 1) NDT / NDH); each recomputes the keys' S and dP.  With NDH = 2 a 64-key
// block's wave holds half the accumulators, so two waves fit per SIMD (the LDS of two workgroups per
// CU allows no more), at 1.5 times the matrix work of one wave per 32 keys.
template <int D, int BLK, int NDH>
__global__ __launch_bounds__(BLK * 2 * NDH, 2) void bwd_dkv_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, int64_t qt, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const uint16_t *__restrict__ dO, int64_t ob,
    int64_t oh, int64_t ot, int tq, int S, int QB, int G, int per_head, int hq, int hkv, int npairs, int pchunks,
    int Ic, int cap, const BwdItem *__restrict__ items, const int32_t *__restrict__ icount,
    const uint32_t *__restrict__ bits, const int16_t *__restrict__ epos, int NBm, int W, int UG,
    const float *__restrict__ gate, int kcap, const float *__restrict__ lse_ws, const float *__restrict__ dd_ws,
    float scale_log2, float scale, float *__restrict__ dK, float *__restrict__ dV, int64_t gb, int64_t gh,
    int64_t gt) {
  constexpr int NKK = D / 16, NDT = D / 32, CPR = D / 8, NKW = BLK / 32, NWV = NKW * NDH, NT = NWV * 64;
  constexpr int NX = NDT / NDH;  // head-dim tiles per wave
  constexpr int NI = 32 * CPR / NT;  // 16-byte copies per thread per staged tensor
  static_assert(NI >= 1 && 32 * CPR % NT == 0, "staging split");
  __shared__ __attribute__((aligned(16))) uint16_t qs[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t dos[2][32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vlds[BLK * D];
  __shared__ __attribute__((aligned(16))) float lse_s[2][64];
  __shared__ __attribute__((aligned(16))) float dd_s[2][64];
  __shared__ int mu[BWD_SEGMAX];
  __shared__ float mgl[BWD_SEGMAX];
  __shared__ __attribute__((aligned(16))) i32x4 ginfo[BWD_SEGMAX];  // h0, t_lo, c, rows | inverse << 8
  __shared__ int scan_w[NWV];

  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int cid = xcd + 8 * (q / Ic);
  const int pair = cid / pchunks;
  if (pair >= npairs) return;
  const int n = cid % pchunks + pchunks * (q % Ic);
  if (n >= icount[pair]) return;
  const BwdItem it = items[(int64_t)pair * cap + n];
  const int b = pair / hkv, g = pair % hkv;
  const int L = st.len[b], q0 = st.q0[b];
  const int j = it.kt;
  const int key0 = j * BLK;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % NKW, dh = wave / NKW;  // this wave's 32 keys and head-dim share
  const int col = lane & 31, half = lane >> 5;
  const int mykey = key0 + kw * 32 + col;
  if (it.count == 0) {
    // no unit selected this block: its gradients are zero (a block of one item only)
    if (mykey < L) {
      const int64_t o = b * gb + (int64_t)g * gh + (int64_t)mykey * gt;
#pragma unroll
      for (int d4 = dh * (D / 4 / NDH); d4 < (dh + 1) * (D / 4 / NDH); d4 += 2) {
        *reinterpret_cast<f32x4 *>(dK + o + 4 * (d4 + half)) = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4 *>(dV + o + 4 * (d4 + half)) = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  // ---- V tile into LDS, K^T of this wave's keys into registers (rows past L re-read row L-1;
  //      their keys are masked below)
  {
    const uint32_t row_bytes = (uint32_t)(kt * 2);
    const uint32_t slab = (uint32_t)(L - 1) * row_bytes + D * 2;
    const i32x4 vrs = lds_rsrc(V + b * kb + (int64_t)g * kh, slab);
#pragma unroll
    for (int t0 = 0; t0 < BLK; t0 += 64)
      copy_tile<D, NWV, true>(vrs, lds_base(vlds) + 2u * (t0 * D), key0 + t0, L - 1, row_bytes, wave, lane);
  }
  bf16x8 kreg[NKK];
  {
    const int64_t ro = b * kb + (int64_t)g * kh + (int64_t)min(mykey, L - 1) * kt + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kreg[kk] = as_bf8(*reinterpret_cast<const u32x4 *>(K + ro + 16 * kk));
  }

  // ---- the item's units: ranks first .. first+count-1 of the set bits of block j's row
  const int cnt = min(it.count, BWD_SEGMAX);
  if (cnt > 0) {
    const uint32_t *row = bits + ((int64_t)pair * NBm + j) * W;
    int base = 0;
    for (int w0 = 0; w0 < W && base < it.first + cnt; w0 += NT) {
      const int w = w0 + tid;
      uint32_t word = w < W ? row[w] : 0u;
      const int pc = __popc(word);
      int x = pc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) scan_w[wave] = x;
      __syncthreads();
      int before = 0, all = 0;
#pragma unroll
      for (int v = 0; v < NWV; ++v) {
        before += v < wave ? scan_w[v] : 0;
        all += scan_w[v];
      }
      int r = base + before + x - pc;
      while (word) {
        const int bit = __ffs(word) - 1;
        word &= word - 1;
        if (r >= it.first && r < it.first + cnt) mu[r - it.first] = w * 32 + bit;
        ++r;
      }
      base += all;
      __syncthreads();
    }
    for (int k = tid; k < cnt; k += NT) {
      const int ugi = mu[k];
      const int i = per_head ? ugi / G : ugi;
      const int s = per_head ? g * G + ugi % G : g;
      const int64_t u = ((int64_t)b * S + s) * QB + i;
      float gl2 = 0.f;
      if (gate) {
        const int e = epos[((int64_t)pair * NBm + j) * UG + ugi];
        gl2 = gate[u * kcap + e] * LOG2E;
      }
      mgl[k] = gl2;
      const UnitGeo x = unit_geo(st, u, S, QB, G, per_head, tq, BLK);
      // rows <= 128 and flattened rows f < rows * 64 (the host rejects more than BWD_MAX_GROUP heads
      // per unit): f / rows = (f * inv) >> 20 exactly, and f * inv < 2^27 fits 32 bits
      const int inv = ((1 << 20) + x.rows - 1) / max(x.rows, 1);
      ginfo[k] = i32x4{x.h0, x.t_lo, x.c, x.rows | (inv << 8)};
    }
  }
  struct Geo {
    int h0, t_lo, c, rows, inv, F;
  };
  // (k is wave-uniform, so is the unit's geometry: scalar registers)
  auto geo_of = [&](int k) {
    const i32x4 v = ginfo[k];
    const int w3 = __builtin_amdgcn_readfirstlane(v[3]);
    const int rows = w3 & 255, inv = (int)((uint32_t)w3 >> 8);
    return Geo{__builtin_amdgcn_readfirstlane(v[0]), __builtin_amdgcn_readfirstlane(v[1]),
               __builtin_amdgcn_readfirstlane(v[2]), rows, inv, rows * (per_head ? 1 : G)};
  };
  auto head_row = [](const Geo &x, int f, int &hh, int &tt) {
    const int qd = (int)(((uint32_t)f * (uint32_t)x.inv) >> 20);
    hh = x.h0 + qd;
    tt = x.t_lo + f - qd * x.rows;
  };
  // Byte offsets of this thread's 16-byte chunks within 32 consecutive rows of one head (the same
  // for every step whose rows are that: a unit whose row count is a multiple of 32).  When a copy
  // instruction covers a multiple of 16 rows, copy y's rows are copy 0's moved by y such row groups, with the
  // same swizzle (it depends on the row's low 4 bits): one lane offset and a scalar row offset serve.
  constexpr int RPC = NT / CPR;  // rows per copy instruction of the workgroup
  constexpr int NOFF = RPC % 16 == 0 ? 1 : NI;
  uint32_t qoff[NOFF], ooff[NOFF];
#pragma unroll
  for (int y = 0; y < NOFF; ++y) {
    const int e = y * NT + tid;
    const int r = e / CPR, off = 8 * ((e % CPR) ^ swz<D, true>(r));
    qoff[y] = 2u * (uint32_t)(r * qt + off);
    ooff[y] = 2u * (uint32_t)(r * ot + off);
  }
  // issue the copies of 32 rows (from flattened row c0 of unit k) into buffer buf
  auto stage = [&](int k, int c0, int buf) {
    const Geo x = geo_of(k);
    if (x.rows % 32 == 0) {
      // the 32 rows are rows tt0 .. tt0 + 31 of head hh: one buffer resource per tensor, based at
      // the first row, spans them; the lanes' offsets were formed above
      const int qd = (int)(((uint32_t)c0 * (uint32_t)x.inv) >> 20);
      const int hh = x.h0 + qd, tt0 = x.t_lo + c0 - qd * x.rows;
      const i32x4 rq = lds_rsrc(Q + b * qb + (int64_t)hh * qh + (int64_t)tt0 * qt, (uint32_t)(31 * qt + D) * 2u);
      const i32x4 ro = lds_rsrc(dO + b * ob + (int64_t)hh * oh + (int64_t)tt0 * ot, (uint32_t)(31 * ot + D) * 2u);
#pragma unroll
      for (int y = 0; y < NI; ++y) {
        const uint32_t lo16 = 2u * (buf * 32 * D + 8 * (y * NT + wave * 64));
        const int yo = NOFF == 1 ? 0 : y;
        const uint32_t rows_q = NOFF == 1 ? (uint32_t)(y * RPC * qt) * 2u : 0u;
        const uint32_t rows_o = NOFF == 1 ? (uint32_t)(y * RPC * ot) * 2u : 0u;
        buf_load_lds<16>(rq, lds_base(qs) + lo16, qoff[yo], rows_q);
        buf_load_lds<16>(ro, lds_base(dos) + lo16, ooff[yo], rows_o);
      }
      if (wave == 0) {
        const int64_t o = ((int64_t)b * hq + hh) * tq + tt0;
        const uint32_t lo4 = 4u * (uint32_t)min(lane, 31);
        buf_load_lds<4>(lds_rsrc(lse_ws + o, 128u), lds_base(lse_s) + 4u * (buf * 64), lo4, 0u);
        buf_load_lds<4>(lds_rsrc(dd_ws + o, 128u), lds_base(dd_s) + 4u * (buf * 64), lo4, 0u);
      }
      return;
    }
#pragma unroll
    for (int y = 0; y < NI; ++y) {
      const int e = y * NT + tid;
      const int r = e / CPR, cs = e % CPR;
      int hh, tt;
      head_row(x, min(c0 + r, x.F - 1), hh, tt);
      const int off = 8 * (cs ^ swz<D, true>(r));
      const uint32_t lo16 = 2u * (buf * 32 * D + 8 * (y * NT + wave * 64));
      load_lds16(Q + b * qb + (int64_t)hh * qh + (int64_t)tt * qt + off, lds_base(qs) + lo16);
      load_lds16(dO + b * ob + (int64_t)hh * oh + (int64_t)tt * ot + off, lds_base(dos) + lo16);
    }
    if (wave == 0) {
      int hh, tt;
      head_row(x, min(c0 + min(lane, 31), x.F - 1), hh, tt);
      const int64_t o = ((int64_t)b * hq + hh) * tq + tt;
      load_lds<4>(lse_ws + o, lds_base(lse_s) + 4u * (buf * 64));
      load_lds<4>(dd_ws + o, lds_base(dd_s) + 4u * (buf * 64));
    }
  };

  f32x16 adk[NX], adv[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x)
#pragma unroll
    for (int r = 0; r < 16; ++r) adk[x][r] = adv[x][r] = 0.f;

  const LdsOffsets<D, true> lo0(col, half, dh * NX);
  __syncthreads();  // mu, mgl visible
  int k = 0, c0 = 0, buf = 0;
  if (cnt > 0) stage(0, 0, 0);
  while (k < cnt) {
    const Geo x = geo_of(k);
    const int F = x.F;
    const float gl2 = mgl[k];
    const bool diag = j == x.c;
    // the next step (the following 32 rows of this unit, or the first rows of the next unit)
    int kn = k, cn = c0 + 32;
    if (cn >= F) {
      ++kn;
      cn = 0;
    }
    wait_stores();
    __syncthreads();  // this step's rows have landed; every wave is done with the other buffer
    if (kn < cnt) stage(kn, cn, buf ^ 1);
    const uint16_t *qsb = qs[buf], *dsb = dos[buf];
    // the offsets' bases, opaque per step so that the XORed offsets are formed where they are used
    // instead of being kept in registers across the loop
    LdsOffsets<D, true> lo = lo0;
    asm volatile("" : "+v"(lo.rb), "+v"(lo.tlb), "+v"(lo.thb));
    // S and dP (rows x this wave's keys): register r holds row 8(r/4) + 4half + r%4, key col
    f32x16 pa, dsa;
#pragma unroll
    for (int r = 0; r < 16; ++r) pa[r] = dsa[r] = 0.f;
    const uint16_t *vw = vlds + kw * 32 * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int ro = lo.rb ^ (16 * kk);
      const u32x4 qv = *reinterpret_cast<const u32x4 *>(qsb + ro);
      pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(qv), kreg[kk], pa, 0, 0, 0);
      const u32x4 dv = *reinterpret_cast<const u32x4 *>(dsb + ro);
      const u32x4 vv = *reinterpret_cast<const u32x4 *>(vw + ro);
      dsa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(dv), as_bf8(vv), dsa, 0, 0, 0);
    }
    // P and dS; only the unit's current block, a step past the unit's last row and the sequence's
    // last block need masks (wave-uniform test)
    auto softmax = [&](auto edge_t) {
      constexpr bool EDGE = decltype(edge_t)::value;
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lse_s[buf][8 * rb + 4 * half]);
        const f32x4 d4 = *reinterpret_cast<const f32x4 *>(&dd_s[buf][8 * rb + 4 * half]);
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          const int r = 4 * rb + y;
          float p = __builtin_amdgcn_exp2f(fmaf(pa[r], scale_log2, gl2 - l4[y]));
          if constexpr (EDGE) {
            const int f = c0 + 8 * rb + 4 * half + y;
            bool vis = f < F && mykey < L;
            if (diag) {
              int hh, tt;
              head_row(x, min(f, F - 1), hh, tt);
              vis = vis && mykey <= q0 + tt;
            }
            p = vis ? p : 0.f;
          }
          pa[r] = p;
          dsa[r] = p * (dsa[r] - d4[y]);
        }
      }
    };
    if (diag || c0 + 32 > F || key0 + BLK > L) softmax(std::true_type{});
    else softmax(std::false_type{});
    // dV^T += dO^T P, dK^T += Q^T dS over the 32 rows (two 16-row steps)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 pop = pack_operand(pa, 8 * ks);
      const bf16x8 dsop = pack_operand(dsa, 8 * ks);
#pragma unroll
      for (int x = 0; x < NX; ++x) {
        const int tl = (lo.tlb ^ (32 * x)) + 16 * ks * D, th = (lo.thb ^ (32 * x)) + 16 * ks * D;
        const u32x2 dlo = lds_read_tr16(dsb + tl), dhi = lds_read_tr16(dsb + th);
        const u32x2 qlo = lds_read_tr16(qsb + tl), qhi = lds_read_tr16(qsb + th);
        const u32x4 dw = {dlo[0], dlo[1], dhi[0], dhi[1]}, qw = {qlo[0], qlo[1], qhi[0], qhi[1]};
        adv[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(dw), pop, adv[x], 0, 0, 0);
        adk[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(qw), dsop, adk[x], 0, 0, 0);
      }
    }
    k = kn;
    c0 = cn;
    buf ^= 1;
  }
  wait_stores();  // no copy into LDS may outlive the workgroup
  // ---- write (lane holds dims 32dt + 8(r/4) + 4half + r%4 of key mykey)
  if (mykey >= L) return;
  const int64_t o = b * gb + (int64_t)g * gh + (int64_t)mykey * gt;
#pragma unroll
  for (int x = 0; x < NX; ++x)
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      const int dim = (dh * NX + x) * 32 + 8 * rb + 4 * half;
      const f32x4 vk = {adk[x][4 * rb] * scale, adk[x][4 * rb + 1] * scale, adk[x][4 * rb + 2] * scale,
                        adk[x][4 * rb + 3] * scale};
      const f32x4 vv = {adv[x][4 * rb], adv[x][4 * rb + 1], adv[x][4 * rb + 2], adv[x][4 * rb + 3]};
      if (it.multi) {
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          unsafeAtomicAdd(dK + o + dim + y, vk[y]);
          unsafeAtomicAdd(dV + o + dim + y, vv[y]);
        }
      } else {
        *reinterpret_cast<f32x4 *>(dK + o + dim) = vk;
        *reinterpret_cast<f32x4 *>(dV + o + dim) = vv;
      }
    }
}

// ---------------------------------------------------------------------------------------------
// dgate, dscore
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_gate_kernel(SeqTable st, int64_t units, int S, int QB, int G, int per_head,
                                                      int tq, int blk, const int32_t *__restrict__ nsel,
                                                      const float *__restrict__ gate, int kcap,
                                                      const float *__restrict__ gpart, int gslots,
                                                      float *__restrict__ dgate, float *__restrict__ dscore) {
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= units) return;
  const UnitGeo x = unit_geo(st, u, S, QB, G, per_head, tq, blk);
  const int ns = x.rows > 0 ? nsel[u] : 0;
  const int nsl = cdiv(x.rows * x.nh, 32);
  auto dg_of = [&](int e) {
    float a = 0.f;
    for (int sl = 0; sl < nsl; ++sl) a += gpart[((int64_t)u * gslots + sl) * kcap + e];
    return a;
  };
  float tot = 0.f;
  for (int e = lane; e < ns; e += 64) tot += dg_of(e);
  tot = wave_sum(tot);
  for (int e = lane; e < kcap; e += 64) {
    float dg = 0.f, dsc = 0.f;
    if (e < ns) {
      dg = dg_of(e);
      dsc = dg - expf(gate[u * kcap + e]) * tot;
    }
    dgate[u * kcap + e] = dg;
    dscore[u * kcap + e] = dsc;
  }
}

// ---------------------------------------------------------------------------------------------
// through the selector: dscore -> dQ (pooled query) and the block means (dK)
// ---------------------------------------------------------------------------------------------
// One workgroup per unit.  s_j = scale qbar . r_j with qbar the mean of the unit's F query vectors
// and r_j the mean of block j's present keys: dqbar = scale sum_j dscore_j r_j goes to each query
// vector as dqbar / F; scale qbar is kept per unit for the block means' gradient
// dr_j = sum over the units keeping j of dscore_j scale qbar (bwd_chain_k_kernel).
template <int D>
__global__ __launch_bounds__(256) void bwd_chain_kernel(SeqTable st, const uint16_t *__restrict__ Q, int64_t qb,
                                                       int64_t qh, int64_t qt, int tq, int S, int QB, int G,
                                                       int per_head, int hkv, const int32_t *__restrict__ idx,
                                                       const int32_t *__restrict__ nsel, int kcap,
                                                       const float *__restrict__ dscore, const float *__restrict__ reps,
                                                       int64_t rb, int64_t rh, int64_t rj, float scale,
                                                       float *__restrict__ dQ, int64_t dqb, int64_t dqh, int64_t dqt,
                                                       float *__restrict__ qbs, int blk) {
  constexpr int RG = 256 / D;  // row groups: thread (rg, dim)
  __shared__ float part[RG][D];
  __shared__ float qbar[D], dqbar[D];
  const int64_t u = blockIdx.x;
  const UnitGeo ug = unit_geo(st, u, S, QB, G, per_head, tq, blk);
  const int ns = ug.rows > 0 ? nsel[u] : 0;
  if (ns == 0) return;
  const int F = ug.rows * ug.nh;
  const int tid = threadIdx.x, dim = tid % D, rg = tid / D;
  const uint16_t *qbase = Q + ug.b * qb;
  float a = 0.f;
  for (int f = rg; f < F; f += RG)
    a += bf16_to_f32(qbase[(int64_t)(ug.h0 + f / ug.rows) * qh + (int64_t)(ug.t_lo + f % ug.rows) * qt + dim]);
  part[rg][dim] = a;
  __syncthreads();
  if (rg == 0) {
    float t = 0.f;
#pragma unroll
    for (int y = 0; y < RG; ++y) t += part[y][dim];
    qbar[dim] = t / (float)F;
    qbs[u * D + dim] = scale * (t / (float)F);
  }
  __syncthreads();
  const int32_t *ul = idx + u * kcap;
  const float *ds = dscore + u * kcap;
  const float *rbase = reps + ug.b * rb + (int64_t)ug.g * rh;
  a = 0.f;
  for (int e = rg; e < ns; e += RG) a += ds[e] * rbase[(int64_t)ul[e] * rj + dim];
  part[rg][dim] = a;
  __syncthreads();
  if (rg == 0) {
    float t = 0.f;
#pragma unroll
    for (int y = 0; y < RG; ++y) t += part[y][dim];
    dqbar[dim] = scale * t / (float)F;
  }
  __syncthreads();
  for (int f = rg; f < F; f += RG)
    dQ[ug.b * dqb + (int64_t)(ug.h0 + f / ug.rows) * dqh + (int64_t)(ug.t_lo + f % ug.rows) * dqt + dim] += dqbar[dim];
}

// dK[key] += dr_j / n_j for every present key of block j (n_j its present keys), with
// dr_j = sum over the units keeping j of dscore_j (scale qbar).  One workgroup per (sequence, KV
// head, block): the units come from the selection bitmap in ascending order, thread group rg takes
// every RG-th of them, and the partial sums are added in a fixed order, so dK does not depend on the
// order in which workgroups run.
template <int D>
__global__ __launch_bounds__(256) void bwd_chain_k_kernel(SeqTable st, int hkv, int blk, int NBm, int W, int UG, int S,
                                                         int QB, int G, int per_head, const uint32_t *__restrict__ bits,
                                                         const int16_t *__restrict__ epos,
                                                         const float *__restrict__ dscore, int kcap,
                                                         const float *__restrict__ qbs, float *__restrict__ dK,
                                                         int64_t gb, int64_t gh, int64_t gt) {
  constexpr int RG = 256 / D;
  __shared__ float part[RG][D];
  const int64_t row = blockIdx.x;  // (sequence, KV head) pair * NBm + block
  const int j = (int)(row % NBm);
  const int pair = (int)(row / NBm);
  const int b = pair / hkv, g = pair % hkv;
  const int L = st.len[b];
  if (j * blk >= L) return;
  const int tid = threadIdx.x, dim = tid % D, rg = tid / D;
  const uint32_t *brow = bits + row * W;
  float a = 0.f;
  int n = 0;
  for (int w = 0; w < W; ++w) {
    uint32_t word = brow[w];
    while (word) {
      const int bit = __ffs(word) - 1;
      word &= word - 1;
      if (n++ % RG != rg) continue;
      const int ugi = w * 32 + bit;
      const int i = per_head ? ugi / G : ugi;
      const int s = per_head ? g * G + ugi % G : g;
      const int64_t u = ((int64_t)b * S + s) * QB + i;
      const int e = epos[row * UG + ugi];
      a += dscore[u * kcap + e] * qbs[u * D + dim];
    }
  }
  if (n == 0) return;  // no unit keeps this block (uniform across the workgroup)
  part[rg][dim] = a;
  __syncthreads();
  if (rg == 0) {
    float t = 0.f;
#pragma unroll
    for (int y = 0; y < RG; ++y) t += part[y][dim];
    part[0][dim] = t;
  }
  __syncthreads();
  const int nj = min(blk, L - j * blk);
  for (int x = tid; x < nj * D; x += 256) {
    const int key = j * blk + x / D, d2 = x % D;
    dK[b * gb + (int64_t)g * gh + (int64_t)key * gt + d2] += part[0][d2] / (float)nj;
  }
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
BwdPlan bwd_plan(const sas_problem &p, int32_t tq, int32_t sel_mode, int32_t kcap, bool gate) {
  BwdPlan x{};
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int G = p.hq / p.hkv;
  const int S = per_head ? p.hq : p.hkv;
  x.QB = num_qblocks(tq, p.block);
  x.units = (int64_t)p.batch * S * x.QB;
  x.nh = per_head ? 1 : G;
  const int rows_max = std::min(tq, p.block);
  x.gslots = cdiv(rows_max * x.nh, 32);
  x.NBm = cdiv(p.max_len, p.block);
  x.UG = x.QB * (per_head ? G : 1);
  x.W = cdiv(x.UG, 32);
  x.npairs = p.batch * p.hkv;
  // a segment holds about BWD_SEG_ROWS flattened rows (its units' rows x heads)
  x.segm = std::max(1, std::min(BWD_SEGMAX, BWD_SEG_ROWS / std::max(1, rows_max * x.nh)));
  x.cap = (int)std::min<int64_t>(INT32_MAX / 2, x.NBm + cdiv64((int64_t)x.UG * kcap, x.segm));
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = 0;
  const size_t rowsz = (size_t)p.batch * p.hq * tq * sizeof(float);
  x.off_lse = off;
  off += al(rowsz);
  x.off_dd = off;
  off += al(rowsz);
  x.off_gpart = off;
  if (gate) off += al((size_t)x.units * x.gslots * kcap * sizeof(float));
  x.off_bits = off;
  // bits, then counts
  x.clear_words = (int64_t)x.npairs * x.NBm * (x.W + 1);
  off += al((size_t)x.clear_words * sizeof(uint32_t));
  x.off_qbar = off;
  // (with a gate) each unit's scaled mean query, for the selector path into dK
  if (gate) off += al((size_t)x.units * p.head_dim * sizeof(float));
  x.off_epos = off;
  if (gate) off += al((size_t)x.npairs * x.NBm * x.UG * sizeof(int16_t));
  x.off_items = off;
  off += al((size_t)x.npairs * x.cap * sizeof(BwdItem));
  x.off_icount = off;
  off += al((size_t)x.npairs * sizeof(int32_t));
  x.bytes = off;
  return x;
}

template <int D, int BLK>
static hipError_t bwd_dispatch(const sas_problem &p, const SeqTable &st, const BwdPlan &pl, const void *Q,
                               const int64_t *qs, const void *K, const void *V, const int64_t *kvs, const void *O,
                               const void *dO, const int64_t *os, const float *lse_in, int32_t tq, int32_t sel_mode,
                               const int32_t *idx,
                               const int32_t *nsel, const float *gate, int32_t kcap, float scale, float *dQ,
                               const int64_t *dqs, float *dK, float *dV, const int64_t *dkvs, float *dgate,
                               float *dscore, const float *reps, const int64_t *rs, char *ws, hipStream_t s) {
  const int per_head = sel_mode == SAS_SEL_HEAD;
  const int G = p.hq / p.hkv;
  const int S = per_head ? p.hq : p.hkv;
  float *lse = (float *)(ws + pl.off_lse), *dd = (float *)(ws + pl.off_dd);
  float *gpart = gate ? (float *)(ws + pl.off_gpart) : nullptr;
  uint32_t *bits = (uint32_t *)(ws + pl.off_bits);
  int32_t *counts = (int32_t *)(bits + (int64_t)pl.npairs * pl.NBm * pl.W);
  int16_t *epos = gate ? (int16_t *)(ws + pl.off_epos) : nullptr;
  BwdItem *items = (BwdItem *)(ws + pl.off_items);
  int32_t *icount = (int32_t *)(ws + pl.off_icount);
  const float scale_log2 = scale * LOG2E;
  const uint16_t *q16 = (const uint16_t *)Q, *k16 = (const uint16_t *)K, *v16 = (const uint16_t *)V;
  const uint16_t *o16 = (const uint16_t *)O, *do16 = (const uint16_t *)dO;

  // selection bitmap, counts, entry positions, work items
  {
    const int64_t n = pl.clear_words;
    const unsigned g = (unsigned)std::min<int64_t>(4096, std::max<int64_t>(1, cdiv64(n, 256)));
    hipLaunchKernelGGL(bwd_clear_kernel, dim3(g), dim3(256), 0, s, bits, n);
    const int64_t m = pl.units * kcap;
    hipLaunchKernelGGL(bwd_mark_kernel, dim3((unsigned)std::max<int64_t>(1, cdiv64(m, 256))), dim3(256), 0, s, idx,
                       nsel, pl.units, kcap, S, pl.QB, G, per_head, p.hkv, pl.NBm, pl.W, pl.UG, bits, counts, epos);
    hipLaunchKernelGGL((bwd_plan_kernel<D>), dim3(pl.npairs), dim3(256), 0, s, st, p.hkv, pl.NBm, p.block, pl.segm,
                       pl.cap, (const int32_t *)counts, items, icount, dK, dV, dkvs[0], dkvs[1], dkvs[2]);
  }
  // dQ, LSE, D, gate partials
  {
    const bool small = std::min(tq, p.block) * pl.nh <= 64;
    const int NW = small ? 2 : 4;
    const int rtiles = cdiv(std::min(tq, p.block) * pl.nh, NW * 32);
    const int64_t nwg = 8 * cdiv64(pl.units, 8) * rtiles;
#define SAS_BDQ(NW_)                                                                                                \
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW_, BLK>), dim3((unsigned)nwg), dim3(NW_ * 64), 0, s, st, q16, qs[0], qs[1], \
                     qs[2], k16, v16, kvs[0], kvs[1], kvs[2], o16, do16, os[0], os[1], os[2], tq, S, pl.QB, G,       \
                     per_head, p.batch, p.hq, rtiles, idx, nsel, gate, kcap, scale_log2, scale, dQ, dqs[0], dqs[1],  \
                     dqs[2], lse, dd, gpart, pl.gslots, lse_in)
    if (small) SAS_BDQ(2);
    else SAS_BDQ(4);
#undef SAS_BDQ
  }
  // dK, dV
  {
    const int pchunks = 8 / std::gcd(pl.npairs, 8);
    const int Ic = cdiv(pl.cap, pchunks);
    const int64_t nwg = (int64_t)8 * cdiv(pl.npairs * pchunks, 8) * Ic;
    constexpr int NDH = (D == 128 && BLK == 64) ? 2 : 1;
    hipLaunchKernelGGL((bwd_dkv_kernel<D, BLK, NDH>), dim3((unsigned)nwg), dim3(BLK * 2 * NDH), 0, s, st, q16, qs[0],
                       qs[1], qs[2],
                       k16, v16, kvs[0], kvs[1], kvs[2], do16, os[0], os[1], os[2], tq, S, pl.QB, G, per_head, p.hq,
                       p.hkv, pl.npairs, pchunks, Ic, pl.cap, (const BwdItem *)items, (const int32_t *)icount,
                       (const uint32_t *)bits, (const int16_t *)epos, pl.NBm, pl.W, pl.UG, gate, kcap, lse, dd,
                       scale_log2, scale, dK, dV, dkvs[0], dkvs[1], dkvs[2]);
  }
  if (gate) {
    hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)cdiv64(pl.units, 4)), dim3(256), 0, s, st, pl.units, S, pl.QB,
                       G, per_head, tq, p.block, nsel, gate, kcap, (const float *)gpart, pl.gslots, dgate, dscore);
  }
  if (gate && reps) {
    // on through the selector scores: into dQ (pooled query) and, via the block means, dK
    float *qbs = (float *)(ws + pl.off_qbar);
    hipLaunchKernelGGL((bwd_chain_kernel<D>), dim3((unsigned)pl.units), dim3(256), 0, s, st, q16, qs[0], qs[1], qs[2],
                       tq, S, pl.QB, G, per_head, p.hkv, idx, nsel, kcap, (const float *)dscore, reps, rs[0], rs[1],
                       rs[2], scale, dQ, dqs[0], dqs[1], dqs[2], qbs, p.block);
    hipLaunchKernelGGL((bwd_chain_k_kernel<D>), dim3((unsigned)((int64_t)pl.npairs * pl.NBm)), dim3(256), 0, s, st,
                       p.hkv, p.block, pl.NBm, pl.W, pl.UG, S, pl.QB, G, per_head, (const uint32_t *)bits,
                       (const int16_t *)epos, (const float *)dscore, kcap, (const float *)qbs, dK, dkvs[0], dkvs[1],
                       dkvs[2]);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_backward(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                                   const void *K, const void *V, const int64_t *kvs, const void *O, const void *dO,
                                   const int64_t *os, const float *lse_in, int32_t tq, int32_t sel_mode,
                                   const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                   float scale, float *dQ, const int64_t *dqs, float *dK, float *dV,
                                   const int64_t *dkvs, float *dgate, float *dscore, const float *reps,
                                   const int64_t *rs, void *workspace, hipStream_t s) {
  const BwdPlan pl = bwd_plan(p, tq, sel_mode, kcap, gate != nullptr);
  char *ws = (char *)workspace;
#define SAS_BWD(D_, B_)                                                                                            \
  return bwd_dispatch<D_, B_>(p, st, pl, Q, qs, K, V, kvs, O, dO, os, lse_in, tq, sel_mode, idx, nsel, gate, kcap, scale, \
                              dQ, dqs, dK, dV, dkvs, dgate, dscore, reps, rs, ws, s)
  if (p.head_dim == 128) {
    if (p.block == 64) SAS_BWD(128, 64);
    SAS_BWD(128, 128);
  }
  if (p.block == 64) SAS_BWD(64, 64);
  SAS_BWD(64, 128);
#undef SAS_BWD
}

}  // namespace sas
