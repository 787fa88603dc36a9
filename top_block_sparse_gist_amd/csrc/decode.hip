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
#include "common.h"

namespace sas {

static constexpr int VPAD = 16;  // LDS row padding (bf16 elements) of the V tile: rows start 8 banks apart

// Split record: acc [nh][D] fp32, then m [nh] (log2 units) and l [nh], padded to 16 bytes.
__host__ __device__ inline int64_t record_floats(int nh, int D) { return (int64_t)nh * D + ((2 * nh + 3) / 4) * 4; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int D, int WPW, typename OT>
__global__ __launch_bounds__(WPW * 64) void decode_bf16_kernel(
    SeqTable st, const uint16_t *__restrict__ Q, int64_t qb, int64_t qh, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kb, int64_t kh, int64_t kt, const uint16_t *__restrict__ GK,
    const uint16_t *__restrict__ GV, int64_t gb, int64_t gh, int64_t gt, int gist, int blk, int S, int G,
    int per_head, const int32_t *__restrict__ idx, const float *__restrict__ gate, int kcap, float scale_log2,
    float *__restrict__ work, uint32_t *__restrict__ counters, OT *__restrict__ O, int64_t ob, int64_t oh) {
  constexpr int NKK = D / 32;   // MFMA k-steps over the head dim
  constexpr int NDT = D / 16;   // 16-dim output tiles
  constexpr int VROW = D + VPAD;
  constexpr int NT = WPW * 64;
  __shared__ __attribute__((aligned(16))) uint16_t vlds[WPW][64 * VROW];
  __shared__ float m_sh[WPW][16], l_sh[WPW][16];
  __shared__ int last_sh;

  const int64_t u = blockIdx.y;
  const int b = (int)(u / S), s = (int)(u % S);
  const int g = per_head ? s / G : s;
  const int nh = per_head ? 1 : G;
  const int h0 = per_head ? s : s * G;
  const int L = st.len[b];
  const int c = (L - 1) / blk;
  const int tpb = blk / 64;
  const int nraw = kcap * tpb;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * WPW + wave;
  const int col = lane & 15, grp = lane >> 4;
  const int64_t rec_sz = record_floats(nh, D);
  float *rec = work + (u * gridDim.x + blockIdx.x) * rec_sz;

  // ---- which keys this wave's tile holds (one dependent load: the block index)
  const uint16_t *kbase = nullptr, *vbase = nullptr;
  int64_t rstride = 0;
  int key0 = 0, nvalid = 0;
  float gl2 = 0.f;
  uint64_t excl = 0;
  if (t < nraw) {
    const int e = t / tpb, sub = t % tpb;
    const int j = idx[u * kcap + e];
    if (j >= 0) {
      key0 = j * blk + sub * 64;
      nvalid = min(64, L - key0);
      kbase = K + b * kb + g * kh;
      vbase = V + b * kb + g * kh;
      rstride = kt;
      if (gate) gl2 = gate[u * kcap + e] * 1.4426950408889634f;
    }
  } else if (gist) {
    key0 = (t - nraw) * 64;
    nvalid = min(64, c - key0);
    kbase = GK + b * gb + g * gh;
    vbase = GV + b * gb + g * gh;
    rstride = gt;
    if (nvalid > 0) {
      // gists of selected chunks are replaced by their raw tokens: exclude them
      for (int e0 = 0; e0 < kcap; e0 += 64) {
        uint64_t bit = 0;
        if (e0 + lane < kcap) {
          const int j = idx[u * kcap + e0 + lane];
          if (j >= key0 && j < key0 + 64) bit = 1ull << (j - key0);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
          const uint32_t lo = __shfl_xor((uint32_t)bit, o, 64);
          const uint32_t hi = __shfl_xor((uint32_t)(bit >> 32), o, 64);
          bit |= ((uint64_t)hi << 32) | lo;
        }
        excl |= bit;
      }
    }
  }
  nvalid = max(nvalid, 0);

  // ---- Q^T as the B operand: lane -> head `col`, dims 32*kk + 8*grp .. +8
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < nh && nvalid > 0)
      v = *reinterpret_cast<const u32x4 *>(Q + b * qb + (int64_t)(h0 + col) * qh + 32 * kk + 8 * grp);
    qreg[kk] = as_bf16x8(v);
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[NDT];
#pragma unroll
  for (int x = 0; x < NDT; ++x) acc_o[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nvalid > 0) {
    // ---- K straight to A-operand registers, V rows to registers (then LDS)
    u32x4 kreg[4][NKK];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int key = mt * 16 + col;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (key < nvalid)
          v = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)(key0 + key) * rstride + 32 * kk + 8 * grp);
        kreg[mt][kk] = v;
      }
    }
    constexpr int VCH = D / 8;  // 16-byte chunks per V row; VCH loads per lane
    u32x4 vreg[VCH];
#pragma unroll
    for (int x = 0; x < VCH; ++x) {
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
    uint16_t *vl = vlds[wave];
#pragma unroll
    for (int x = 0; x < VCH; ++x) {
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
        const bool ok = key < nvalid && !((excl >> key) & 1ull);
        const float v = ok ? sacc[mt][r] * scale_log2 + gl2 : -INFINITY;
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
        const float p = __builtin_amdgcn_exp2f(sacc[mt][r] - mref);
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
    // the V tile is written and read by this wave only: wait for its LDS writes
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    // ---- O^T = V^T P^T; the V^T operand (dim 16dt + col, keys 32ks + 4grp + {0..3} then
    //      32ks + 16 + 4grp + {0..3}) comes from two transpose reads of the row-major tile
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
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  // ---- this workgroup's record: [nh][D] acc, then m[nh], l[nh] (m in log2 units), written with
  //      device-coherent 16-byte stores so that the merging workgroup (any XCD) reads them
  const uint32_t rec_bytes = (uint32_t)rec_sz * 4u;
  const __amdgpu_buffer_rsrc_t rr = dev_rsrc(work + u * gridDim.x * rec_sz, gridDim.x * rec_bytes);
  const uint32_t my = blockIdx.x * rec_bytes;
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
    last_sh = (old == gridDim.x - 1);
  }
  __syncthreads();
  if (!last_sh) return;
  const int nrec = gridDim.x;
  const int tid = threadIdx.x;
  float *msh = reinterpret_cast<float *>(&vlds[0][0]);  // [nrec][nh] m, then l, then weights
  float *lsh = msh + nrec * nh;
  float *fsh = lsh + nrec * nh;
  f32x4 *red = reinterpret_cast<f32x4 *>(msh + ((3 * nrec * nh + 3) / 4) * 4);
  __shared__ float Mh[16], Lh[16];
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

// ---- host side -------------------------------------------------------------------------------
struct DecodeShape {
  int S, nh, tiles_cap, wpw, nwg_cap;
  int64_t units;
};

static DecodeShape decode_shape(const sas_problem &p, int32_t sel_mode, int32_t kcap, int gist, int maxc) {
  DecodeShape d;
  const int per_head = sel_mode == SAS_SEL_HEAD;
  d.S = per_head ? p.hq : p.hkv;
  d.nh = per_head ? 1 : p.hq / p.hkv;
  d.units = (int64_t)p.batch * d.S;
  d.tiles_cap = kcap * (p.block / 64) + (gist ? (maxc + 63) / 64 : 0);
  // one wave per workgroup keeps every CU busy; wide units (many heads x many tiles) merge
  // 4 waves per workgroup first so that the final merge reads fewer records
  d.wpw = 4;
  auto fits = [&](int wpw) {
    const int nwg = (d.tiles_cap + wpw - 1) / wpw;
    const int lds = wpw * 64 * (p.head_dim + VPAD) * 2;
    return 12 * nwg * d.nh + 16 + 16 * 64 * wpw <= lds;
  };
  if (!fits(d.wpw)) d.wpw = 4;
  d.nwg_cap = (d.tiles_cap + d.wpw - 1) / d.wpw;
  return d;
}

size_t decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gist) {
  const int maxc = (p.max_len - 1) / p.block;
  DecodeShape d = decode_shape(p, sel_mode, kcap, gist, maxc);
  // arrival counters (one per unit, 256-byte aligned region) + one record per workgroup
  const size_t counters = ((size_t)d.units * 4 + 255) / 256 * 256;
  return counters + (size_t)d.units * d.nwg_cap * record_floats(d.nh, p.head_dim) * sizeof(float);
}

template <int D, int WPW>
static hipError_t decode_launch(const sas_problem &p, const SeqTable &st, const DecodeShape &d, int nwg,
                                const void *Q, const int64_t *qs, const void *K, const void *V, const int64_t *kvs,
                                const void *gk, const void *gv, int64_t gb, int64_t gh, int64_t gt, int gist,
                                int per_head, const int32_t *idx, const float *gate, int32_t kcap, float scale_log2,
                                float *work, uint32_t *counters, void *O, const int64_t *os, hipStream_t s) {
  hipLaunchKernelGGL((decode_bf16_kernel<D, WPW, uint16_t>), dim3(nwg, (unsigned)d.units), dim3(WPW * 64), 0, s,
                     st, (const uint16_t *)Q, qs[0], qs[1], (const uint16_t *)K, (const uint16_t *)V, kvs[0], kvs[1],
                     kvs[2], (const uint16_t *)gk, (const uint16_t *)gv, gb, gh, gt, gist, p.block, d.S,
                     p.hq / p.hkv, per_head, idx, gate, kcap, scale_log2, work, counters, (uint16_t *)O, os[0],
                     os[1]);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk,
                              const void *gv, const int64_t *gs, int32_t sel_mode, const int32_t *idx,
                              const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                              const int64_t *os, float *workspace, hipStream_t s) {
  (void)nsel;
  const int gist = gk != nullptr;
  const int per_head = sel_mode == SAS_SEL_HEAD;
  int maxc = 0;
  for (int b = 0; b < p.batch; ++b) maxc = max(maxc, (st.len[b] - 1) / p.block);
  // the record layout and the workgroup count follow the capacity shape; only nwg launches
  const DecodeShape cap = decode_shape(p, sel_mode, kcap, gist, (p.max_len - 1) / p.block);
  DecodeShape d = decode_shape(p, sel_mode, kcap, gist, maxc);
  d.wpw = cap.wpw;
  const int nwg = (d.tiles_cap + d.wpw - 1) / d.wpw;
  uint32_t *counters = reinterpret_cast<uint32_t *>(workspace);
  const size_t cbytes = ((size_t)d.units * 4 + 255) / 256 * 256;
  float *work = reinterpret_cast<float *>(reinterpret_cast<char *>(workspace) + cbytes);
  int64_t gb = 0, gh = 0, gt = 0;
  if (gist) { gb = gs[0]; gh = gs[1]; gt = gs[2]; }
  const float sl2 = scale * 1.4426950408889634f;
#define SAS_DEC(D_, W_)                                                                                          \
  return decode_launch<D_, W_>(p, st, d, nwg, Q, qs, K, V, kvs, gk, gv, gb, gh, gt, gist, per_head, idx, gate,   \
                               kcap, sl2, work, counters, O, os, s)
  if (p.head_dim == 128) {
    if (d.wpw == 1) SAS_DEC(128, 1);
    SAS_DEC(128, 4);
  }
  if (d.wpw == 1) SAS_DEC(64, 1);
  SAS_DEC(64, 4);
#undef SAS_DEC
}

}  // namespace sas
