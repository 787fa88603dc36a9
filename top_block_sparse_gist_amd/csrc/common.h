// Internal definitions shared by the HIP kernels and the host layer of libsas.
// gfx950 (CDNA4) only: wave64, MFMA bf16 16x16x32 / 32x32x16, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

#include "../../include/sas.h"

namespace sas {

// Per-call sequence table, passed by value as a kernel argument (no device upload).  With the
// lengths in device memory (dlen != nullptr: a decode loop replayed from a captured graph while the
// lengths grow) len[] holds the capacity max_len, which sizes the grids, and kernels read L_b from
// dlen through seq_len().
struct SeqTable {
  int32_t len[SAS_MAX_BATCH];  // L_b (device lengths: max_len)
  int32_t q0[SAS_MAX_BATCH];   // position of the first query row (decode: L_b - 1)
  const int32_t *dlen;         // DEVICE [B] lengths, or nullptr
};

// L_b of sequence b; a device length is clamped to [1, max_len] (the host cannot check it).
__device__ __forceinline__ int seq_len(const SeqTable &st, int b) {
  return st.dlen ? min(max(st.dlen[b], 1), st.len[b]) : st.len[b];
}

struct Budget {
  int32_t k_fixed, frac_num, frac_den, count_current, sink, gate;
  float coverage;  // 0: off (see coverage_count in the top-k bodies)
  int32_t shared;  // 1: the G heads of a KV group share G * k (per-head selection)
  int32_t sqrt_num, sqrt_den;  // sqrt_den > 0: k = ceil(sqrt_num * sqrt(c + count_current) / sqrt_den)
};

// ---------------------------------------------------------------------------------------
// host + device helpers
// ---------------------------------------------------------------------------------------
__host__ __device__ inline int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ceil((tq-1)/blk) + 1: blocks that tq consecutive positions can touch.
__host__ __device__ inline int32_t num_qblocks(int32_t tq, int32_t blk) {
  return tq <= 1 ? 1 : cdiv(tq - 1, blk) + 1;
}

// ceil(sqrt(x)) for 0 <= x < 2^62, exact: a floating-point estimate corrected with integer compares.
__host__ __device__ inline int64_t ceil_isqrt(int64_t x) {
  if (x <= 0) return 0;
  int64_t r = (int64_t)sqrt((double)x);
  while (r > 0 && r * r > x) --r;
  while ((r + 1) * (r + 1) <= x) ++r;  // r = floor(sqrt(x))
  return r * r == x ? r : r + 1;
}

// Number of top-k blocks for a unit with current block c and n_cand candidates.
__host__ __device__ inline int32_t budget_k(const Budget &bg, int32_t c, int32_t n_cand) {
  int32_t k;
  if (bg.coverage > 0.f && bg.k_fixed <= 0 && bg.frac_den == 0 && bg.sqrt_den == 0) {
    k = n_cand;  // an uncapped coverage budget may keep every candidate
  } else if (bg.sqrt_den > 0) {
    // square-root budget: the smallest k with k * sqrt_den >= sqrt_num * sqrt(n), n = c + count_current;
    // k * sqrt_den is an integer, so that is ceil(ceil(sqrt(sqrt_num^2 n)) / sqrt_den)
    const int64_t n = (int64_t)c + bg.count_current;
    const int64_t r = ceil_isqrt((int64_t)bg.sqrt_num * bg.sqrt_num * n);
    k = (int32_t)((r + bg.sqrt_den - 1) / bg.sqrt_den);
  } else if (bg.frac_den == 0) {
    k = bg.k_fixed;
  } else {
    int64_t num = (int64_t)bg.frac_num * (int64_t)(c + bg.count_current);
    k = (int32_t)((num + bg.frac_den - 1) / bg.frac_den);
  }
  if (k > n_cand) k = n_cand;
  if (k < 0) k = 0;
  return k;
}

// ---------------------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16 round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32 (two values per instruction).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return (uint16_t)(pack_bf16x2(f, 0.f) & 0xffffu); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Cross-workgroup hand-off without whole-L2 maintenance.  The 8 XCDs have separate L2s, and a
// device-scope release/acquire fence writes back and invalidates the whole L2 of the XCD.
// Data handed to another workgroup is instead written with device-coherent stores (sc1) and
// read with device-coherent loads (sc1); the writer waits for its stores to be acknowledged
// (vmcnt 0) before it bumps the arrival counter with a device-scope atomic, and the reader
// issues its loads only after its own atomic has returned.
__device__ __forceinline__ void store_dev(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); /* vmcnt(0) */ }
// s_waitcnt vmcnt(N) (N < 64; the count is split over bits 3:0 and 15:14), other counters free
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// 16-byte device-coherent accesses through a raw buffer resource (aux 16 = sc1).  Accesses
// past `bytes` read 0 / are dropped by the hardware range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0, 16);
}
__device__ __forceinline__ f32x4 load16_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16));
}
__device__ __forceinline__ void store4_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(v), r, (int)off, 0, 16);
}
__device__ __forceinline__ float load4_dev(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 16));
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane i of
// the group receives element (i % 4) of the 64-bit words addressed by lanes (i / 4) + 4e of the
// group, for e = 0..3.  So when lane s of a group addresses 4 consecutive bf16 of a row-major
// tile at row R(s / 4), columns c0 + 4 (s % 4), lane i receives column c0 + i of rows
// R(0..3): the MFMA operand layout of the transposed tile, with no scalar LDS reads.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
  return __builtin_bit_cast(u32x2, v);
}

// Copies from global memory straight into LDS (global_load_lds / buffer_load ... lds).
// They are issued from inline asm.  The compiler treats a copy it emits itself as a store to LDS
// that may alias every later LDS read, so it puts `s_waitcnt vmcnt` before those reads, and that
// wait also covers the copies of the next tile.  A double-buffered loop then stalls on its own
// prefetch every iteration.  The asm copies are invisible to that tracking.  Every kernel that
// uses them therefore waits for its copies explicitly (s_waitcnt vmcnt, then a barrier) before it
// reads the LDS they fill, and it lets no copy outlive the workgroup.  Waits the compiler places
// for its own loads stay correct: the copies only add to the count of outstanding operations it
// waits down to.  The copies have no register results, and the asm sets M0 (the LDS address;
// one wait state before the copy reads it) and declares it clobbered.
// M0 is named as clobbered on purpose (each copy sets it); clang warns that it is reserved.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// LDS addresses are passed as integers: the byte address of a __shared__ array itself (lds_base,
// a link-time constant) plus offsets computed as integers.  (Converting a pointer into such an
// array at run time would go through a 64-bit generic address.)
template <typename T>
__device__ __forceinline__ uint32_t lds_base(T *shared_array) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)shared_array;
}

// 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4): the wave writes 64 x
// 16 B contiguously at LDS byte address `lds` (wave-uniform), lane l at lds + 16 l.  Tracked by vmcnt.
__device__ __forceinline__ void load_lds16(const void *g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
               "v"(g)
               : "memory", "m0");
}

// BYTES (4 or 16) per lane from global memory into LDS (global_load_lds): the wave writes 64 x
// BYTES contiguously at LDS byte address `lds`, lane l at lds + l * BYTES.  Tracked by vmcnt.
template <int BYTES>
__device__ __forceinline__ void load_lds(const void *g, uint32_t lds) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte copies");
  if constexpr (BYTES == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(g)
                 : "memory", "m0");
  else
    load_lds16(g, lds);
}

// BYTES (4 or 16) per lane through a buffer resource into LDS (buffer_load ... lds): the wave
// writes 64 x BYTES contiguously at LDS byte address `lds`, lane i at lds + BYTES * i; the lane reads
// rsrc + soff + voff, and an access past the resource's range writes zeros.  Row offsets can stay
// scalar (soff).  Tracked by vmcnt.  (2-byte copies are not offered: a head-dim-64 prefill that
// used them read wrong values.)
// Buffer resource for these copies, in scalar registers: base address, no stride, `bytes` in range,
// the same flags as dev_rsrc (words 0-3 of the descriptor).
__device__ __forceinline__ i32x4 lds_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return i32x4{(int32_t)__builtin_amdgcn_readfirstlane((uint32_t)a),
               (int32_t)(__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu),
               (int32_t)__builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
template <int BYTES>
__device__ __forceinline__ void buf_load_lds(i32x4 rv, uint32_t lds, uint32_t voff, uint32_t soff) {
  static_assert(BYTES == 4 || BYTES == 16, "4- or 16-byte copies");
  // the descriptor is wave-uniform; this keeps it in scalar registers whatever path formed it
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rv[0]), __builtin_amdgcn_readfirstlane(rv[1]),
                   __builtin_amdgcn_readfirstlane(rv[2]), __builtin_amdgcn_readfirstlane(rv[3])};
  if constexpr (BYTES == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Sum over aligned groups of W lanes (W = 8, 16 or 32), valid in the group's first lane (lane %
// W == 0).  Within a 16-lane row the adds use DPP (quad xor 1, quad xor 2, then row rotates: a
// rotate right by N hands lane i the value of lane i - N mod 16, so rotating by 12 adds the next
// quad, lanes i + 4, and rotating by 8 the other half row; no LDS round trip); W = 32 adds the
// other row with one cross-lane read.  The order of the adds is fixed, so every kernel that uses
// it gets the same bits for the same inputs.
template <int W>
__device__ __forceinline__ float group_sum(float s) {
  static_assert(W == 8 || W == 16 || W == 32, "group of 8, 16 or 32 lanes");
  auto dpp = [](float v, auto ctrl) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value, 0xF, 0xF, false));
  };
  s += dpp(s, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]: lane ^ 1
  s += dpp(s, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]: lane ^ 2
  s += dpp(s, std::integral_constant<int, 0x12C>{});  // row_ror:12: quads q and q+1
  if constexpr (W >= 16) s += dpp(s, std::integral_constant<int, 0x128>{});  // row_ror:8: whole row
  if constexpr (W == 32) s += __shfl_xor(s, 16, 64);
  return s;
}

// Order-preserving map of fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace sas

// ---------------------------------------------------------------------------------------
// launchers (defined in the kernel files, called by the host layer)
// ---------------------------------------------------------------------------------------
namespace sas {

// first: host [batch] first block to compute per sequence, or NULL for every block; current: only the
// block holding position L_b - 1 of each sequence (found on the device)
hipError_t launch_reps(const sas_problem &p, const SeqTable &st, const void *K, const int64_t *ks,
                       float *reps, const int64_t *rs, const int32_t *first, hipStream_t s,
                       const int32_t *table = nullptr, int64_t tld = 0, bool current = false);

hipError_t launch_pool_queries(const sas_problem &p, const SeqTable &st, const void *Q,
                               const int64_t *qs, int32_t tq, int32_t sel_mode, float *qbar,
                               hipStream_t s);

hipError_t launch_scores_prefill(const sas_problem &p, const SeqTable &st, const float *qbar,
                                 int32_t tq, const void *reps, int32_t reps_kind, const int64_t *rs,
                                 int32_t sel_mode, float scale, float *scores, int64_t ld,
                                 hipStream_t s);

hipError_t launch_scores_decode(const sas_problem &p, const SeqTable &st, const void *Q,
                                const int64_t *qs, const void *reps, int32_t reps_kind,
                                const int64_t *rs, int32_t sel_mode, float scale, float *scores,
                                int64_t ld, hipStream_t s);

hipError_t launch_topk(const sas_problem &p, const SeqTable &st, const float *scores, int64_t ld,
                       int32_t tq, int32_t sel_mode, const Budget &bg, int32_t kcap, int32_t *idx,
                       int32_t *nsel, float *gate, hipStream_t s);

hipError_t launch_prefill_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                               const void *K, const void *V, const int64_t *kvs, int32_t tq,
                               int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                               const float *gate, int32_t kcap, float scale, void *O, const int64_t *os,
                               hipStream_t s,
                               const int32_t *table = nullptr, int64_t tld = 0, float *lse = nullptr);

// table: DEVICE [B, tld] page of each block (paged K/V; kv strides are then {page, head, token}), or nullptr
hipError_t launch_decode_bf16(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk,
                              const void *gv, const int64_t *gs, int32_t sel_mode, const int32_t *idx,
                              const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                              const int64_t *os, float *work, hipStream_t s,
                              const int32_t *table = nullptr, int64_t tld = 0);

hipError_t launch_attend_f32(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                             const void *K, const void *V, const int64_t *kvs, const void *gk, const void *gv,
                             const int64_t *gs, int32_t tq, int32_t sel_mode, const int32_t *idx,
                             const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                             const int64_t *os, hipStream_t s);

hipError_t launch_select_decode(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                                const void *reps, int32_t reps_kind, const int64_t *rs, int32_t sel_mode,
                                float scale, float *scores, int64_t ld, const Budget &bg, int32_t kcap,
                                int32_t *idx, int32_t *nsel, float *gate, uint32_t *counters, hipStream_t s);

// Largest current-block index the fused decode selection handles (its scores stay in registers).
constexpr int32_t SELECT_DECODE_MAX_C = 2048;

// Bytes of split-K partials the decode path needs (host formula shared with the size query).
size_t decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gist);
// leading bytes of that workspace that hold the per-unit arrival counters (256-byte aligned)
size_t decode_counter_bytes(const sas_problem &p, int32_t sel_mode);
// whether the split-K merge of the bf16 decode fits its LDS for this list capacity (nwg records
// per unit against cap)
bool decode_merge_fits(const sas_problem &p, const SeqTable &st, int32_t sel_mode, int32_t kcap, int32_t gist,
                       int *nwg, int *cap);
// two-level gist mode (meta-gists): selection and attention
size_t hssa_select_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t M, int32_t k1);
int hssa_candidates_max(const sas_problem &p, int32_t M, int32_t k1);
hipError_t launch_hssa_select(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *gk, const int64_t *gs, const void *mk, const int64_t *ms, int32_t M,
                              int32_t sel_mode, int32_t k1, int32_t k2, float scale, int32_t kcap, int32_t gcap,
                              int32_t *idx, int32_t *nsel, int32_t *gidx, int32_t *gsel, float *work, hipStream_t s);
bool hssa_merge_fits(const sas_problem &p, const SeqTable &st, int32_t sel_mode, int32_t kcap, int32_t gcap,
                     int32_t M, int *nwg_out, int *cap_out);
size_t hssa_decode_workspace_bytes(const sas_problem &p, int32_t sel_mode, int32_t kcap, int32_t gcap, int32_t M);
hipError_t launch_hssa_decode(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                              const void *K, const void *V, const int64_t *kvs, const void *gk, const void *gv,
                              const int64_t *gs, const void *mk, const void *mv, const int64_t *ms, int32_t M,
                              int32_t sel_mode, const int32_t *idx, const int32_t *nsel, int32_t kcap,
                              const int32_t *gidx, int32_t gcap, float scale, void *O, const int64_t *os,
                              float *workspace, hipStream_t s);


// Backward of the sparse prefill: sizes and workspace layout (host formula shared with the size
// query).  Workspace regions, 256-byte aligned: row LSE and D [B, Hq, tq] fp32; gate partials
// [units, gslots, kcap] fp32 (with a gate); selection bitmap [pairs, NBm, W] u32 and per-block
// counts [pairs, NBm]; (with a gate) each unit's scaled mean query [units, d] fp32 and entry
// positions [pairs, NBm, UG] int16; work items [pairs, cap] x 16 bytes; item counts [pairs].
constexpr int BWD_SEGMAX = 256;       // units per dK/dV work item
constexpr int BWD_MAX_GROUP = 64;     // query heads per KV head with per-group units (row mapping)
constexpr int BWD_SEG_ROWS = 32768;   // flattened rows per dK/dV work item (a block's list is cut
                                      // into items of about this much work)
struct BwdPlan {
  int QB, nh, gslots, NBm, UG, W, npairs, segm, cap;
  int64_t units, clear_words;
  size_t off_lse, off_dd, off_gpart, off_bits, off_qbar, off_epos, off_items, off_icount, bytes;
};
BwdPlan bwd_plan(const sas_problem &p, int32_t tq, int32_t sel_mode, int32_t kcap, bool gate);
hipError_t launch_prefill_backward(const sas_problem &p, const SeqTable &st, const void *Q, const int64_t *qs,
                                   const void *K, const void *V, const int64_t *kvs, const void *O, const void *dO,
                                   const int64_t *os, const float *lse, int32_t tq, int32_t sel_mode,
                                   const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                   float scale, float *dQ, const int64_t *dqs, float *dK, float *dV,
                                   const int64_t *dkvs, float *dgate, float *dscore, const float *reps,
                                   const int64_t *rs, void *workspace, hipStream_t s);

}  // namespace sas
