// Host layer of libsas: argument validation (no HIP call), launch configuration, error text.
// The exported entry points and their contracts are declared and documented in sas.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "common.h"

using namespace sas;

namespace {

thread_local char g_err[512] = "";

sas_status fail(sas_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

sas_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return SAS_OK;
  return fail(SAS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int elem_bytes(int32_t dtype) { return dtype == SAS_BF16 ? 2 : 4; }

// 16-byte vector loads need every row start 16-byte aligned.
bool strides_ok(const int64_t *st, int n, int esize) {
  const int64_t v = 16 / esize;
  for (int x = 0; x < n; ++x)
    if (st[x] < 0 || st[x] % v != 0) return false;
  return true;
}

sas_status check_problem(const sas_problem *p, SeqTable *tab) {
  if (!p) return fail(SAS_ERR_NULL, "problem is NULL");
  if (!p->seq_lens) return fail(SAS_ERR_NULL, "seq_lens is NULL");
  if (p->batch < 1) return fail(SAS_ERR_SHAPE, "batch must be >= 1 (got %d)", p->batch);
  if (p->batch > SAS_MAX_BATCH)
    return fail(SAS_ERR_UNSUPPORTED, "batch %d exceeds SAS_MAX_BATCH (%d) per call", p->batch, SAS_MAX_BATCH);
  if (p->hq < 1 || p->hkv < 1 || p->hq % p->hkv != 0)
    return fail(SAS_ERR_SHAPE, "hq (%d) must be a positive multiple of hkv (%d)", p->hq, p->hkv);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(SAS_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128)", p->head_dim);
  if (p->block != 64 && p->block != 128)
    return fail(SAS_ERR_UNSUPPORTED, "block %d not supported (64, 128)", p->block);
  if (p->dtype != SAS_F32 && p->dtype != SAS_BF16) return fail(SAS_ERR_UNSUPPORTED, "dtype %d", p->dtype);
  if (p->max_len < 1) return fail(SAS_ERR_SHAPE, "max_len must be >= 1");
  if (p->seq_lens_device != 0 && p->seq_lens_device != 1)
    return fail(SAS_ERR_SHAPE, "seq_lens_device must be 0 or 1 (got %d)", p->seq_lens_device);
  if (p->seq_lens_device) {
    // lengths in device memory: the host sizes everything for the capacity; kernels read the lengths
    if (tab) {
      for (int b = 0; b < p->batch; ++b) {
        tab->len[b] = p->max_len;
        tab->q0[b] = p->max_len - 1;
      }
      tab->dlen = p->seq_lens;
    }
    return SAS_OK;
  }
  for (int b = 0; b < p->batch; ++b) {
    const int L = p->seq_lens[b];
    if (L < 1 || L > p->max_len)
      return fail(SAS_ERR_SHAPE, "seq_lens[%d] = %d outside [1, max_len = %d]", b, L, p->max_len);
    if (tab) {
      tab->len[b] = L;
      tab->q0[b] = L - 1;
    }
  }
  return SAS_OK;
}

// Entry points that need the lengths on the host refuse device lengths.
sas_status host_lengths_only(const sas_problem *p, const char *what) {
  if (p && p->seq_lens_device)
    return fail(SAS_ERR_UNSUPPORTED, "%s needs seq_lens in host memory (seq_lens_device = 0)", what);
  return SAS_OK;
}

// The problem as the host sees it: with device lengths, a copy whose lengths are the capacity held by
// the checked table (valid while `tab` lives).
sas_problem host_view(const sas_problem *p, const SeqTable &tab) {
  sas_problem h = *p;
  if (p->seq_lens_device) {
    h.seq_lens = tab.len;
    h.seq_lens_device = 0;
  }
  return h;
}

// Prefill rows: q_start (host) gives the first row position, rows [q0, q0 + tq) within [0, L).
sas_status check_rows(const sas_problem *p, int32_t tq, const int32_t *q_start, SeqTable *tab) {
  // the entry points that take rows (scores, top-k, prefill, backward, kcap) work from host lengths
  sas_status st;
  if ((st = host_lengths_only(p, "this entry point")) != SAS_OK) return st;
  if (tq < 1) return fail(SAS_ERR_SHAPE, "tq must be >= 1 (got %d)", tq);
  if (!q_start) {
    if (tq != 1) return fail(SAS_ERR_SHAPE, "decode (q_start == NULL) needs tq == 1 (got %d)", tq);
    return SAS_OK;
  }
  for (int b = 0; b < p->batch; ++b) {
    const int q0 = q_start[b];
    if (q0 < 0 || (int64_t)q0 + tq > p->seq_lens[b])
      return fail(SAS_ERR_SHAPE, "rows [%d, %d) of sequence %d exceed its length %d", q0, q0 + tq, b,
                  p->seq_lens[b]);
    if (tab) tab->q0[b] = q0;
  }
  return SAS_OK;
}

sas_status check_sel(int32_t sel_mode) {
  if (sel_mode != SAS_SEL_GROUP && sel_mode != SAS_SEL_HEAD)
    return fail(SAS_ERR_SHAPE, "sel_mode %d is neither SAS_SEL_GROUP nor SAS_SEL_HEAD", sel_mode);
  return SAS_OK;
}

sas_status check_budget(const sas_budget *bg) {
  if (!bg) return fail(SAS_ERR_NULL, "budget is NULL");
  if (bg->k_fixed < 0 || bg->frac_num < 0 || bg->frac_den < 0)
    return fail(SAS_ERR_SHAPE, "budget fields must be >= 0");
  if (bg->sqrt_num < 0 || bg->sqrt_den < 0 || bg->sqrt_num > 65535 || bg->sqrt_den > 65535)
    return fail(SAS_ERR_SHAPE, "sqrt_num and sqrt_den must be in [0, 65535]");
  if (bg->count_current != 0 && bg->count_current != 1)
    return fail(SAS_ERR_SHAPE, "count_current must be 0 or 1");
  if (!(bg->coverage >= 0.f && bg->coverage <= 1.f)) return fail(SAS_ERR_SHAPE, "coverage must be in [0, 1]");
  if (bg->shared_heads != 0 && bg->shared_heads != 1) return fail(SAS_ERR_SHAPE, "shared_heads must be 0 or 1");
  if (bg->shared_heads && bg->coverage > 0.f)
    return fail(SAS_ERR_UNSUPPORTED, "a shared budget with a coverage budget is not defined here");
  return SAS_OK;
}

float resolve_scale(float scale, int d) { return scale == 0.f ? 1.f / sqrtf((float)d) : scale; }

int32_t required_kcap(const sas_problem *p, int32_t tq, const int32_t *q_start, const sas_budget *bg) {
  Budget b{bg->k_fixed, bg->frac_num, bg->frac_den, bg->count_current, bg->force_sink ? 1 : 0, bg->gate,
           bg->coverage, bg->shared_heads, bg->sqrt_num, bg->sqrt_den};
  const int G = p->hq / p->hkv;
  int32_t need = 1;
  for (int s = 0; s < p->batch; ++s) {
    const int L = p->seq_lens[s];
    const int lo_pos = q_start ? q_start[s] : L - 1;
    const int hi_pos = q_start ? q_start[s] + tq - 1 : L - 1;
    for (int c = lo_pos / p->block; c <= hi_pos / p->block; ++c) {
      const bool sink = b.sink && c > 0;
      const int ncand = c - (sink ? 1 : 0);
      // a shared budget may give one head up to G times its own k
      const int k = b.shared ? std::min(G * budget_k(b, c, ncand), ncand) : budget_k(b, c, ncand);
      const int n = k + 1 + (sink ? 1 : 0);
      need = std::max(need, n);
    }
  }
  return need;
}

}  // namespace

extern "C" {

const char *sas_last_error(void) { return g_err; }

int32_t sas_num_qblocks(int32_t tq, int32_t block) {
  if (tq < 1 || block < 1) return (int32_t)fail(SAS_ERR_SHAPE, "tq and block must be >= 1");
  return num_qblocks(tq, block);
}

int32_t sas_required_kcap(const sas_problem *p, int32_t tq, const int32_t *q_start, const sas_budget *budget) {
  sas_status st;
  if ((st = check_problem(p, nullptr)) != SAS_OK) return st;
  if ((st = host_lengths_only(p, "sas_required_kcap")) != SAS_OK) return st;
  if ((st = check_rows(p, tq, q_start, nullptr)) != SAS_OK) return st;
  if ((st = check_budget(budget)) != SAS_OK) return st;
  return required_kcap(p, tq, q_start, budget);
}

sas_status sas_block_reps(const sas_problem *p, const void *K, const int64_t k_stride[3], float *reps,
                          const int64_t rep_stride[3], void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!K || !reps || !k_stride || !rep_stride) return fail(SAS_ERR_NULL, "K, reps or a stride array is NULL");
  if (!aligned16(K) || !aligned16(reps) || !strides_ok(k_stride, 3, elem_bytes(p->dtype)) ||
      !strides_ok(rep_stride, 3, 4))
    return fail(SAS_ERR_SHAPE, "K / reps must be 16-byte aligned with 16-byte-multiple row strides");
  return hip_status(launch_reps(*p, tab, K, k_stride, reps, rep_stride, nullptr, (hipStream_t)stream),
                    "sas_block_reps");
}

sas_status sas_block_reps_update(const sas_problem *p, const void *K, const int64_t k_stride[3], float *reps,
                                 const int64_t rep_stride[3], const int32_t *first_block, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!K || !reps || !k_stride || !rep_stride) return fail(SAS_ERR_NULL, "K, reps or a stride array is NULL");
  if (!aligned16(K) || !aligned16(reps) || !strides_ok(k_stride, 3, elem_bytes(p->dtype)) ||
      !strides_ok(rep_stride, 3, 4))
    return fail(SAS_ERR_SHAPE, "K / reps must be 16-byte aligned with 16-byte-multiple row strides");
  if (p->seq_lens_device) {
    // lengths in device memory: the block of each sequence's last position, found on the device
    if (first_block)
      return fail(SAS_ERR_SHAPE, "with device seq_lens, first_block must be NULL (the current block is pooled)");
    return hip_status(launch_reps(*p, tab, K, k_stride, reps, rep_stride, nullptr, (hipStream_t)stream, nullptr, 0,
                                  true),
                      "sas_block_reps_update");
  }
  if (!first_block) return fail(SAS_ERR_NULL, "first_block is NULL");
  for (int b = 0; b < p->batch; ++b) {
    const int nb = cdiv(tab.len[b], p->block);
    if (first_block[b] < 0 || first_block[b] > nb)
      return fail(SAS_ERR_SHAPE, "first_block[%d] = %d is outside [0, %d]", b, first_block[b], nb);
  }
  return hip_status(launch_reps(*p, tab, K, k_stride, reps, rep_stride, first_block, (hipStream_t)stream),
                    "sas_block_reps_update");
}

size_t sas_block_scores_workspace(const sas_problem *p, int32_t tq, int32_t sel_mode) {
  if (!p || tq <= 1) return 0;
  const int S = sel_mode == SAS_SEL_HEAD ? p->hq : p->hkv;
  return (size_t)p->batch * S * num_qblocks(tq, p->block) * p->head_dim * sizeof(float);
}

sas_status sas_block_scores(const sas_problem *p, const void *Q, const int64_t q_stride[3], int32_t tq,
                            const int32_t *q_start, const void *reps, int32_t reps_kind,
                            const int64_t rep_stride[3], int32_t sel_mode, float scale, float *scores,
                            int64_t scores_ld, void *workspace, size_t workspace_bytes, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if ((st = check_rows(p, tq, q_start, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !reps || !rep_stride || !scores) return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if (reps_kind != SAS_REPS_POOLED && reps_kind != SAS_REPS_GIST)
    return fail(SAS_ERR_SHAPE, "reps_kind %d", reps_kind);
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  const int rep_bytes = reps_kind == SAS_REPS_GIST ? elem_bytes(p->dtype) : 4;
  if (!aligned16(Q) || !aligned16(reps) || !strides_ok(q_stride, 3, elem_bytes(p->dtype)) ||
      !strides_ok(rep_stride, 3, rep_bytes))
    return fail(SAS_ERR_SHAPE, "Q / reps must be 16-byte aligned with 16-byte-multiple row strides");
  int nbmax = 0;
  for (int b = 0; b < p->batch; ++b) nbmax = std::max(nbmax, cdiv(p->seq_lens[b], p->block));
  if (scores_ld < nbmax) return fail(SAS_ERR_SHAPE, "scores_ld %lld < %d blocks", (long long)scores_ld, nbmax);
  const float sc = resolve_scale(scale, p->head_dim);
  const hipStream_t s = (hipStream_t)stream;
  if (!q_start && sel_mode == SAS_SEL_HEAD && p->hq / p->hkv > 16)
    return fail(SAS_ERR_UNSUPPORTED, "per-head decode scoring supports at most 16 query heads per KV head");
  if (!q_start)
    return hip_status(launch_scores_decode(*p, tab, Q, q_stride, reps, reps_kind, rep_stride, sel_mode, sc, scores,
                                           scores_ld, s),
                      "sas_block_scores");
  const size_t need = sas_block_scores_workspace(p, tq, sel_mode);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (need > 0 && !aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  // the prefill score product addresses one (sequence, KV head) slab of representatives with
  // 32-bit byte offsets
  if ((int64_t)(cdiv(p->max_len, p->block) - 1) * rep_stride[2] * rep_bytes + (int64_t)p->head_dim * rep_bytes >
      0xFFFFFFFFll)
    return fail(SAS_ERR_UNSUPPORTED, "one (sequence, KV head) slab of representatives must span less than 4 GiB");
  // and reads the pooled queries with 32-bit byte offsets
  if (need > 0xFFFFF000ull) return fail(SAS_ERR_UNSUPPORTED, "the pooled queries must span less than 4 GiB");
  float *qbar = (float *)workspace;
  hipError_t e = launch_pool_queries(*p, tab, Q, q_stride, tq, sel_mode, qbar, s);
  if (e != hipSuccess) return hip_status(e, "sas_block_scores (pool)");
  return hip_status(launch_scores_prefill(*p, tab, qbar, tq, reps, reps_kind, rep_stride, sel_mode, sc, scores,
                                          scores_ld, s),
                    "sas_block_scores");
}

sas_status sas_topk_select(const sas_problem *p, const float *scores, int64_t scores_ld, int32_t tq,
                           const int32_t *q_start, int32_t sel_mode, const sas_budget *budget, int32_t kcap,
                           int32_t *idx, int32_t *nsel, float *gate, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if ((st = check_rows(p, tq, q_start, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if ((st = check_budget(budget)) != SAS_OK) return st;
  if (budget->shared_heads && sel_mode != SAS_SEL_HEAD)
    return fail(SAS_ERR_SHAPE, "a shared budget needs per-head selection");
  if (!scores || !idx || !nsel) return fail(SAS_ERR_NULL, "scores, idx or nsel is NULL");
  if (budget->gate && !gate) return fail(SAS_ERR_NULL, "budget->gate is set but gate is NULL");
  int nbmax = 0;
  for (int b = 0; b < p->batch; ++b) nbmax = std::max(nbmax, cdiv(p->seq_lens[b], p->block));
  if (scores_ld < nbmax) return fail(SAS_ERR_SHAPE, "scores_ld %lld < %d blocks", (long long)scores_ld, nbmax);
  const int32_t need = required_kcap(p, tq, q_start, budget);
  if (kcap < need) return fail(SAS_ERR_SHAPE, "kcap %d < %d selected blocks", kcap, need);
  Budget bg{budget->k_fixed,   budget->frac_num,         budget->frac_den,
            budget->count_current, budget->force_sink ? 1 : 0, budget->gate ? 1 : 0,
            budget->coverage,    budget->shared_heads ? 1 : 0, budget->sqrt_num,
            budget->sqrt_den};
  return hip_status(launch_topk(*p, tab, scores, scores_ld, tq, sel_mode, bg, kcap, idx, nsel,
                                budget->gate ? gate : nullptr, (hipStream_t)stream),
                    "sas_topk_select");
}

sas_status sas_sparse_prefill(const sas_problem *p, const void *Q, const int64_t q_stride[3], const void *K,
                              const void *V, const int64_t kv_stride[3], int32_t tq, const int32_t *q_start,
                              int32_t sel_mode, const int32_t *idx, const int32_t *nsel, const float *gate,
                              int32_t kcap, float scale, void *O, const int64_t o_stride[3], void *stream) {
  return sas_sparse_prefill_lse(p, Q, q_stride, K, V, kv_stride, tq, q_start, sel_mode, idx, nsel, gate, kcap, scale,
                                O, o_stride, nullptr, stream);
}

sas_status sas_sparse_prefill_lse(const sas_problem *p, const void *Q, const int64_t q_stride[3], const void *K,
                                  const void *V, const int64_t kv_stride[3], int32_t tq, const int32_t *q_start,
                                  int32_t sel_mode, const int32_t *idx, const int32_t *nsel, const float *gate,
                                  int32_t kcap, float scale, void *O, const int64_t o_stride[3], float *lse,
                                  void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!q_start) return fail(SAS_ERR_NULL, "q_start is NULL (prefill needs the first row position)");
  if ((st = check_rows(p, tq, q_start, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !K || !V || !kv_stride || !idx || !nsel || !O || !o_stride)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if (kcap < 1) return fail(SAS_ERR_SHAPE, "kcap must be >= 1");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  const int eb = elem_bytes(p->dtype);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !strides_ok(q_stride, 3, eb) ||
      !strides_ok(kv_stride, 3, eb) || !strides_ok(o_stride, 3, eb))
    return fail(SAS_ERR_SHAPE, "Q/K/V/O must be 16-byte aligned with 16-byte-multiple row strides");
  // the bf16 kernel addresses one (sequence, KV head) K/V slab with 32-bit byte offsets
  if (p->dtype == SAS_BF16 && (int64_t)(p->max_len - 1) * kv_stride[2] * eb + (int64_t)p->head_dim * eb > 0xFFFFFFFFll)
    return fail(SAS_ERR_UNSUPPORTED, "one (sequence, KV head) K/V slab must span less than 4 GiB");
  const float sc = resolve_scale(scale, p->head_dim);
  const hipStream_t s = (hipStream_t)stream;
  if (lse && (p->dtype != SAS_BF16 || !aligned16(lse)))
    return fail(SAS_ERR_UNSUPPORTED, "the row log-sum-exp is written by the bf16 path (16-byte aligned)");
  if (p->dtype == SAS_BF16)
    return hip_status(launch_prefill_bf16(*p, tab, Q, q_stride, K, V, kv_stride, tq, sel_mode, idx, nsel, gate, kcap,
                                          sc, O, o_stride, s, nullptr, 0, lse),
                      "sas_sparse_prefill");
  return hip_status(launch_attend_f32(*p, tab, Q, q_stride, K, V, kv_stride, nullptr, nullptr, nullptr, tq, sel_mode,
                                      idx, nsel, gate, kcap, sc, O, o_stride, s),
                    "sas_sparse_prefill");
}

size_t sas_select_decode_workspace(const sas_problem *p) {
  if (!p || p->batch < 1 || p->hkv < 1) return 0;
  return ((size_t)p->batch * p->hkv * 4 + 255) / 256 * 256;
}

sas_status sas_select_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2], const void *reps,
                             int32_t reps_kind, const int64_t rep_stride[3], int32_t sel_mode, float scale,
                             const sas_budget *budget, int32_t kcap, float *scores, int64_t scores_ld, int32_t *idx,
                             int32_t *nsel, float *gate, void *workspace, size_t workspace_bytes, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if ((st = check_budget(budget)) != SAS_OK) return st;
  if (budget->shared_heads && sel_mode != SAS_SEL_HEAD)
    return fail(SAS_ERR_SHAPE, "a shared budget needs per-head selection");
  if (budget->shared_heads && p->hq / p->hkv > 4)
    return fail(SAS_ERR_UNSUPPORTED, "the fused selection shares a budget over at most 4 heads per KV head; "
                "use sas_block_scores + sas_topk_select");
  if (!Q || !q_stride || !reps || !rep_stride || !scores || !idx || !nsel)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if (budget->gate && !gate) return fail(SAS_ERR_NULL, "budget->gate is set but gate is NULL");
  if (reps_kind != SAS_REPS_POOLED && reps_kind != SAS_REPS_GIST)
    return fail(SAS_ERR_SHAPE, "reps_kind %d", reps_kind);
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  if (p->hq / p->hkv > 16)
    return fail(SAS_ERR_UNSUPPORTED, "the fused decode selection supports at most 16 query heads per KV head");
  const int rep_bytes = reps_kind == SAS_REPS_GIST ? elem_bytes(p->dtype) : 4;
  if (!aligned16(Q) || !aligned16(reps) || !strides_ok(q_stride, 2, elem_bytes(p->dtype)) ||
      !strides_ok(rep_stride, 3, rep_bytes))
    return fail(SAS_ERR_SHAPE, "Q / reps must be 16-byte aligned with 16-byte-multiple row strides");
  // with device lengths every bound below is taken at the capacity max_len
  const sas_problem hv = host_view(p, tab);
  int nbmax = 0, maxc = 0;
  for (int b = 0; b < p->batch; ++b) {
    nbmax = std::max(nbmax, cdiv(tab.len[b], p->block));
    maxc = std::max(maxc, (tab.len[b] - 1) / p->block);
  }
  if (maxc > SELECT_DECODE_MAX_C)
    return fail(SAS_ERR_UNSUPPORTED, "current block %d > %d: use sas_block_scores + sas_topk_select", maxc,
                SELECT_DECODE_MAX_C);
  if (scores_ld < nbmax) return fail(SAS_ERR_SHAPE, "scores_ld %lld < %d blocks", (long long)scores_ld, nbmax);
  const int32_t need = required_kcap(&hv, 1, nullptr, budget);
  if (kcap < need) return fail(SAS_ERR_SHAPE, "kcap %d < %d selected blocks", kcap, need);
  const size_t wneed = sas_select_decode_workspace(p);
  if (!workspace || workspace_bytes < wneed)
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", wneed, workspace_bytes);
  if (!aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  Budget bg{budget->k_fixed,   budget->frac_num,         budget->frac_den,
            budget->count_current, budget->force_sink ? 1 : 0, budget->gate ? 1 : 0,
            budget->coverage,    budget->shared_heads ? 1 : 0, budget->sqrt_num,
            budget->sqrt_den};
  const int64_t qs3[3] = {q_stride[0], q_stride[1], 0};
  return hip_status(launch_select_decode(*p, tab, Q, qs3, reps, reps_kind, rep_stride, sel_mode,
                                         resolve_scale(scale, p->head_dim), scores, scores_ld, bg, kcap, idx, nsel,
                                         budget->gate ? gate : nullptr, (uint32_t *)workspace, (hipStream_t)stream),
                    "sas_select_decode");
}

size_t sas_sparse_decode_workspace(const sas_problem *p, int32_t sel_mode, int32_t kcap, int32_t gist) {
  if (!p || kcap < 1 || p->dtype != SAS_BF16 || p->block < 64 || p->max_len < 1) return 0;
  return decode_workspace_bytes(*p, sel_mode, kcap, gist);
}

}  // extern "C"

namespace {

// Scratch of sas_sparse_decode_noalloc: one array per GPU (each device that loads the library holds its
// own copy until the process ends).  Host code must not pass `scratch` itself to a kernel: its host-side
// name is not a device address.  The device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[SAS_DECODE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[MAX_DEVICES] = {};

// device address of the current device's scratch array (looked up on the first call on that device)
sas_status scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "sas_sparse_decode_noalloc (hipGetDevice)");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(SAS_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "sas_sparse_decode_noalloc (hipGetSymbolAddress)");
    if (!ptr) return fail(SAS_ERR_HIP, "sas_sparse_decode_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SAS_OK;
}

// zeroes n 32-bit words (a fill kernel rather than a memset, so the call may sit in a captured graph)
__global__ void clear_words_kernel(uint32_t *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// sas_sparse_decode's body.  noalloc: the scratch is the static array above instead of `workspace`.
sas_status sparse_decode_impl(const sas_problem *p, const void *Q, const int64_t q_stride[2], const void *K,
                              const void *V, const int64_t kv_stride[3], const void *gist_k, const void *gist_v,
                              const int64_t gist_stride[3], int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                              const float *gate, int32_t kcap, float scale, void *O, const int64_t o_stride[2],
                              void *workspace, size_t workspace_bytes, bool noalloc, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !K || !V || !kv_stride || !idx || !nsel || !O || !o_stride)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  const bool gist = gist_k != nullptr || gist_v != nullptr;
  if (gist && (!gist_k || !gist_v || !gist_stride)) return fail(SAS_ERR_NULL, "gist mode needs gist_k, gist_v and gist_stride");
  if (gist && gate) return fail(SAS_ERR_UNSUPPORTED, "the log-gate is not defined for gist tokens");
  if (kcap < 1) return fail(SAS_ERR_SHAPE, "kcap must be >= 1");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  const int eb = elem_bytes(p->dtype);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !strides_ok(q_stride, 2, eb) ||
      !strides_ok(kv_stride, 3, eb) || !strides_ok(o_stride, 2, eb) ||
      (gist && (!aligned16(gist_k) || !aligned16(gist_v) || !strides_ok(gist_stride, 3, eb))))
    return fail(SAS_ERR_SHAPE, "Q/K/V/O/gist must be 16-byte aligned with 16-byte-multiple row strides");
  const float sc = resolve_scale(scale, p->head_dim);
  const hipStream_t s = (hipStream_t)stream;
  if (p->dtype == SAS_F32) {
    if ((st = host_lengths_only(p, "the fp32 decode")) != SAS_OK) return st;
    const int64_t qs3[3] = {q_stride[0], q_stride[1], 0};
    const int64_t os3[3] = {o_stride[0], o_stride[1], 0};
    return hip_status(launch_attend_f32(*p, tab, Q, qs3, K, V, kv_stride, gist_k, gist_v, gist_stride, 1, sel_mode,
                                        idx, nsel, gate, kcap, sc, O, os3, s),
                      "sas_sparse_decode");
  }
  if (sel_mode == SAS_SEL_GROUP && p->hq / p->hkv > 16)
    return fail(SAS_ERR_UNSUPPORTED, "per-group decode supports at most 16 query heads per KV head");
  int nwg = 0, cap = 0;
  if (!decode_merge_fits(*p, tab, sel_mode, kcap, gist ? 1 : 0, &nwg, &cap))
    return fail(SAS_ERR_UNSUPPORTED, "kcap %d needs %d split-K records per unit; the merge holds %d", kcap, nwg,
                cap);
  const size_t need = decode_workspace_bytes(*p, sel_mode, kcap, gist ? 1 : 0);
  if (noalloc) {
    if (need > (size_t)SAS_DECODE_NOALLOC_SCRATCH_BYTES)
      return fail(SAS_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the library's static array holds %zu",
                  need, (size_t)SAS_DECODE_NOALLOC_SCRATCH_BYTES);
    void *ptr = nullptr;
    if ((st = scratch_address(&ptr)) != SAS_OK) return st;
    // the array keeps the last call's contents: clear the arrival counters, which must start at zero
    const int64_t words = (int64_t)(decode_counter_bytes(*p, sel_mode) / 4);
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)cdiv64(words, 256)), dim3(256), 0, s, (uint32_t *)ptr,
                       words);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "sas_sparse_decode_noalloc (clear)");
    workspace = ptr;
  } else {
    if (!workspace || workspace_bytes < need)
      return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (!aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  }
  return hip_status(launch_decode_bf16(*p, tab, Q, q_stride, K, V, kv_stride, gist_k, gist_v, gist_stride, sel_mode,
                                       idx, nsel, gate, kcap, sc, O, o_stride, (float *)workspace, s),
                    noalloc ? "sas_sparse_decode_noalloc" : "sas_sparse_decode");
}

}  // namespace

extern "C" {

sas_status sas_sparse_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2], const void *K,
                             const void *V, const int64_t kv_stride[3], const void *gist_k, const void *gist_v,
                             const int64_t gist_stride[3], int32_t sel_mode, const int32_t *idx,
                             const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                             const int64_t o_stride[2], void *workspace, size_t workspace_bytes, void *stream) {
  return sparse_decode_impl(p, Q, q_stride, K, V, kv_stride, gist_k, gist_v, gist_stride, sel_mode, idx, nsel, gate,
                            kcap, scale, O, o_stride, workspace, workspace_bytes, false, stream);
}

sas_status sas_sparse_decode_noalloc(const sas_problem *p, const void *Q, const int64_t q_stride[2], const void *K,
                                     const void *V, const int64_t kv_stride[3], const void *gist_k,
                                     const void *gist_v, const int64_t gist_stride[3], int32_t sel_mode,
                                     const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                     float scale, void *O, const int64_t o_stride[2], void *stream) {
  return sparse_decode_impl(p, Q, q_stride, K, V, kv_stride, gist_k, gist_v, gist_stride, sel_mode, idx, nsel, gate,
                            kcap, scale, O, o_stride, nullptr, 0, true, stream);
}

// ---- paged K/V (one block per page, a block table per sequence) ------------------------------
static sas_status check_table(const sas_problem *p, const SeqTable &tab, const int32_t *table, int64_t table_ld,
                              const int64_t *page_stride) {
  if (!table) return fail(SAS_ERR_NULL, "block_table is NULL");
  // one page holds blk tokens of every KV head, and pages do not overlap
  if ((int64_t)(p->hkv - 1) * page_stride[1] + (int64_t)(p->block - 1) * page_stride[2] + p->head_dim >
      page_stride[0])
    return fail(SAS_ERR_SHAPE, "page stride %lld cannot hold %d tokens of %d KV heads", (long long)page_stride[0],
                p->block, p->hkv);
  int nbmax = 0;
  for (int b = 0; b < p->batch; ++b) nbmax = std::max(nbmax, cdiv(tab.len[b], p->block));
  if (table_ld < nbmax) return fail(SAS_ERR_SHAPE, "table_ld %lld < %d blocks", (long long)table_ld, nbmax);
  return SAS_OK;
}

sas_status sas_block_reps_paged(const sas_problem *p, const void *K_pages, const int64_t page_stride[3],
                                const int32_t *block_table, int64_t table_ld, float *reps,
                                const int64_t rep_stride[3], const int32_t *first_block, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!K_pages || !reps || !page_stride || !rep_stride) return fail(SAS_ERR_NULL, "K, reps or a stride array is NULL");
  if ((st = check_table(p, tab, block_table, table_ld, page_stride)) != SAS_OK) return st;
  if (!aligned16(K_pages) || !aligned16(reps) || !strides_ok(page_stride, 3, elem_bytes(p->dtype)) ||
      !strides_ok(rep_stride, 3, 4))
    return fail(SAS_ERR_SHAPE, "K / reps must be 16-byte aligned with 16-byte-multiple row strides");
  if (first_block) {
    for (int b = 0; b < p->batch; ++b) {
      const int nb = cdiv(tab.len[b], p->block);
      if (first_block[b] < 0 || first_block[b] > nb)
        return fail(SAS_ERR_SHAPE, "first_block[%d] = %d is outside [0, %d]", b, first_block[b], nb);
    }
  }
  return hip_status(launch_reps(*p, tab, K_pages, page_stride, reps, rep_stride, first_block, (hipStream_t)stream,
                                block_table, table_ld),
                    "sas_block_reps_paged");
}

sas_status sas_sparse_decode_paged(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                                   const void *K_pages, const void *V_pages, const int64_t page_stride[3],
                                   const int32_t *block_table, int64_t table_ld, int32_t sel_mode,
                                   const int32_t *idx, const int32_t *nsel, const float *gate, int32_t kcap,
                                   float scale, void *O, const int64_t o_stride[2], void *workspace,
                                   size_t workspace_bytes, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !K_pages || !V_pages || !page_stride || !idx || !nsel || !O || !o_stride)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if ((st = check_table(p, tab, block_table, table_ld, page_stride)) != SAS_OK) return st;
  if (p->dtype != SAS_BF16) return fail(SAS_ERR_UNSUPPORTED, "paged decode needs bf16 inputs");
  if (kcap < 1) return fail(SAS_ERR_SHAPE, "kcap must be >= 1");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  if (!aligned16(Q) || !aligned16(K_pages) || !aligned16(V_pages) || !aligned16(O) || !strides_ok(q_stride, 2, 2) ||
      !strides_ok(page_stride, 3, 2) || !strides_ok(o_stride, 2, 2))
    return fail(SAS_ERR_SHAPE, "Q/K/V/O must be 16-byte aligned with 16-byte-multiple row strides");
  if (sel_mode == SAS_SEL_GROUP && p->hq / p->hkv > 16)
    return fail(SAS_ERR_UNSUPPORTED, "per-group decode supports at most 16 query heads per KV head");
  int nwg = 0, cap = 0;
  if (!decode_merge_fits(*p, tab, sel_mode, kcap, 0, &nwg, &cap))
    return fail(SAS_ERR_UNSUPPORTED, "kcap %d needs %d split-K records per unit; the merge holds %d", kcap, nwg,
                cap);
  const size_t need = decode_workspace_bytes(*p, sel_mode, kcap, 0);
  if (!workspace || workspace_bytes < need)
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  return hip_status(launch_decode_bf16(*p, tab, Q, q_stride, K_pages, V_pages, page_stride, nullptr, nullptr,
                                       nullptr, sel_mode, idx, nsel, gate, kcap, resolve_scale(scale, p->head_dim),
                                       O, o_stride, (float *)workspace, (hipStream_t)stream, block_table, table_ld),
                    "sas_sparse_decode_paged");
}

sas_status sas_sparse_prefill_paged(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                                    const void *K_pages, const void *V_pages, const int64_t page_stride[3],
                                    const int32_t *block_table, int64_t table_ld, int32_t tq,
                                    const int32_t *q_start, int32_t sel_mode, const int32_t *idx,
                                    const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                                    const int64_t o_stride[3], void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!q_start) return fail(SAS_ERR_NULL, "q_start is NULL (prefill needs the first row position)");
  if ((st = check_rows(p, tq, q_start, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !K_pages || !V_pages || !page_stride || !idx || !nsel || !O || !o_stride)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if ((st = check_table(p, tab, block_table, table_ld, page_stride)) != SAS_OK) return st;
  if (p->dtype != SAS_BF16) return fail(SAS_ERR_UNSUPPORTED, "paged prefill needs bf16 inputs");
  if (kcap < 1) return fail(SAS_ERR_SHAPE, "kcap must be >= 1");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  if (!aligned16(Q) || !aligned16(K_pages) || !aligned16(V_pages) || !aligned16(O) || !strides_ok(q_stride, 3, 2) ||
      !strides_ok(page_stride, 3, 2) || !strides_ok(o_stride, 3, 2))
    return fail(SAS_ERR_SHAPE, "Q/K/V/O must be 16-byte aligned with 16-byte-multiple row strides");
  return hip_status(launch_prefill_bf16(*p, tab, Q, q_stride, K_pages, V_pages, page_stride, tq, sel_mode, idx, nsel,
                                        gate, kcap, resolve_scale(scale, p->head_dim), O, o_stride,
                                        (hipStream_t)stream, block_table, table_ld),
                    "sas_sparse_prefill_paged");
}

// ---- two-level gist selection (H-SSA) -------------------------------------------------------
// checks shared by the two entry points: bf16, group size, the opened-group list capacity
static sas_status check_hssa(const sas_problem *p, const SeqTable &tab, int32_t sel_mode, int32_t M, int32_t gcap,
                             int *maxc_out) {
  sas_status st;
  if ((st = host_lengths_only(p, "the two-level gist decode")) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (p->dtype != SAS_BF16) return fail(SAS_ERR_UNSUPPORTED, "two-level gist selection needs bf16 inputs");
  if (M < 4 || M > 64) return fail(SAS_ERR_UNSUPPORTED, "group_chunks %d outside [4, 64]", M);
  if (gcap < 1) return fail(SAS_ERR_SHAPE, "gcap must be >= 1");
  int maxc = 0;
  for (int b = 0; b < p->batch; ++b) maxc = std::max(maxc, (tab.len[b] - 1) / p->block);
  *maxc_out = maxc;
  return SAS_OK;
}

size_t sas_hssa_select_workspace(const sas_problem *p, int32_t sel_mode, int32_t group_chunks, int32_t k1) {
  if (!p || p->block < 64 || p->max_len < 1 || group_chunks < 4 || group_chunks > 64 || k1 < 0) return 0;
  return hssa_select_workspace_bytes(*p, sel_mode, group_chunks, k1);
}

sas_status sas_hssa_select_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                                  const void *gist_k, const int64_t gist_stride[3], const void *meta_k,
                                  const int64_t meta_stride[3], int32_t group_chunks, int32_t sel_mode, int32_t k1,
                                  int32_t k2, float scale, int32_t kcap, int32_t gcap, int32_t *idx, int32_t *nsel,
                                  int32_t *gidx, int32_t *gsel, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!Q || !q_stride || !gist_k || !gist_stride || !meta_k || !meta_stride || !idx || !nsel || !gidx || !gsel)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  int maxc = 0;
  if ((st = check_hssa(p, tab, sel_mode, group_chunks, gcap, &maxc)) != SAS_OK) return st;
  if (k1 < 0 || k2 < 0) return fail(SAS_ERR_SHAPE, "k1 and k2 must be >= 0");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  if (p->hq / p->hkv > 16) return fail(SAS_ERR_UNSUPPORTED, "at most 16 query heads per KV head");
  if (maxc > SELECT_DECODE_MAX_C) return fail(SAS_ERR_UNSUPPORTED, "current chunk %d > %d", maxc, SELECT_DECODE_MAX_C);
  const int nm_cap = ((p->max_len - 1) / p->block) / group_chunks;
  if (nm_cap + 1 > 512) return fail(SAS_ERR_UNSUPPORTED, "%d groups of %d chunks: at most 511", nm_cap, group_chunks);
  const int ncand = hssa_candidates_max(*p, group_chunks, k1);
  if (ncand > 2048)
    return fail(SAS_ERR_UNSUPPORTED, "(k1 + 1) * group_chunks = %d candidate chunks: at most 2048", ncand);
  const int k1u = std::min(k1, nm_cap), k2u = std::min(k2, ncand);
  if (gcap < k1u + 1) return fail(SAS_ERR_SHAPE, "gcap %d < %d opened groups", gcap, k1u + 1);
  if (kcap < k2u + 1) return fail(SAS_ERR_SHAPE, "kcap %d < %d selected chunks", kcap, k2u + 1);
  if (!aligned16(Q) || !aligned16(gist_k) || !aligned16(meta_k) || !strides_ok(q_stride, 2, 2) ||
      !strides_ok(gist_stride, 3, 2) || !strides_ok(meta_stride, 3, 2))
    return fail(SAS_ERR_SHAPE, "Q / gist / meta-gist keys must be 16-byte aligned with 16-byte-multiple row strides");
  const size_t wneed = hssa_select_workspace_bytes(*p, sel_mode, group_chunks, k1);
  if (!workspace || workspace_bytes < wneed)
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", wneed, workspace_bytes);
  if (!aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  return hip_status(launch_hssa_select(*p, tab, Q, q_stride, gist_k, gist_stride, meta_k, meta_stride, group_chunks,
                                       sel_mode, k1, k2, resolve_scale(scale, p->head_dim), kcap, gcap, idx, nsel,
                                       gidx, gsel, (float *)workspace, (hipStream_t)stream),
                    "sas_hssa_select_decode");
}

size_t sas_hssa_decode_workspace(const sas_problem *p, int32_t sel_mode, int32_t kcap, int32_t gcap,
                                 int32_t group_chunks) {
  if (!p || kcap < 1 || gcap < 1 || p->dtype != SAS_BF16 || p->block < 64 || p->max_len < 1 || group_chunks < 4 ||
      group_chunks > 64)
    return 0;
  return hssa_decode_workspace_bytes(*p, sel_mode, kcap, gcap, group_chunks);
}

sas_status sas_hssa_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2], const void *K,
                           const void *V, const int64_t kv_stride[3], const void *gist_k, const void *gist_v,
                           const int64_t gist_stride[3], const void *meta_k, const void *meta_v,
                           const int64_t meta_stride[3], int32_t group_chunks, int32_t sel_mode, const int32_t *idx,
                           const int32_t *nsel, int32_t kcap, const int32_t *gidx, int32_t gcap, float scale,
                           void *O, const int64_t o_stride[2], void *workspace, size_t workspace_bytes,
                           void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!Q || !q_stride || !K || !V || !kv_stride || !gist_k || !gist_v || !gist_stride || !meta_k || !meta_v ||
      !meta_stride || !idx || !nsel || !gidx || !O || !o_stride)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  int maxc = 0;
  if ((st = check_hssa(p, tab, sel_mode, group_chunks, gcap, &maxc)) != SAS_OK) return st;
  if (kcap < 1) return fail(SAS_ERR_SHAPE, "kcap must be >= 1");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  if (sel_mode == SAS_SEL_GROUP && p->hq / p->hkv > 16)
    return fail(SAS_ERR_UNSUPPORTED, "per-group decode supports at most 16 query heads per KV head");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(gist_k) || !aligned16(gist_v) ||
      !aligned16(meta_k) || !aligned16(meta_v) || !strides_ok(q_stride, 2, 2) || !strides_ok(kv_stride, 3, 2) ||
      !strides_ok(o_stride, 2, 2) || !strides_ok(gist_stride, 3, 2) || !strides_ok(meta_stride, 3, 2))
    return fail(SAS_ERR_SHAPE, "Q/K/V/O/gist/meta-gist must be 16-byte aligned with 16-byte-multiple row strides");
  int nwg = 0, cap = 0;
  if (!hssa_merge_fits(*p, tab, sel_mode, kcap, gcap, group_chunks, &nwg, &cap))
    return fail(SAS_ERR_UNSUPPORTED, "kcap %d + gcap %d need %d split-K records per unit; the merge holds %d", kcap,
                gcap, nwg, cap);
  const size_t need = hssa_decode_workspace_bytes(*p, sel_mode, kcap, gcap, group_chunks);
  if (!workspace || workspace_bytes < need)
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!aligned16(workspace)) return fail(SAS_ERR_SHAPE, "workspace must be 16-byte aligned");
  return hip_status(launch_hssa_decode(*p, tab, Q, q_stride, K, V, kv_stride, gist_k, gist_v, gist_stride, meta_k,
                                       meta_v, meta_stride, group_chunks, sel_mode, idx, nsel, kcap, gidx, gcap,
                                       resolve_scale(scale, p->head_dim), O, o_stride, (float *)workspace,
                                       (hipStream_t)stream),
                    "sas_hssa_decode");
}

size_t sas_sparse_prefill_backward_workspace(const sas_problem *p, int32_t tq, int32_t sel_mode, int32_t kcap,
                                             int32_t gate) {
  if (!p || tq < 1 || kcap < 1 || kcap > 32767 || p->batch < 1 || p->hq < 1 || p->hkv < 1 || p->hq % p->hkv ||
      p->block < 64 || p->max_len < 1 || (sel_mode != SAS_SEL_GROUP && sel_mode != SAS_SEL_HEAD))
    return 0;
  return bwd_plan(*p, tq, sel_mode, kcap, gate != 0).bytes;
}

sas_status sas_sparse_prefill_backward(const sas_problem *p, const void *Q, const int64_t q_stride[3], const void *K,
                                       const void *V, const int64_t kv_stride[3], int32_t tq, const int32_t *q_start,
                                       int32_t sel_mode, const int32_t *idx, const int32_t *nsel, const float *gate,
                                       int32_t kcap, float scale, const void *O, const void *dO,
                                       const int64_t o_stride[3], const float *lse, float *dQ,
                                       const int64_t dq_stride[3], float *dK,
                                       float *dV, const int64_t dkv_stride[3], float *dgate, float *dscore,
                                       const float *reps, const int64_t rep_stride[3], void *workspace,
                                       size_t workspace_bytes, void *stream) {
  SeqTable tab{};
  sas_status st;
  if ((st = check_problem(p, &tab)) != SAS_OK) return st;
  if (!q_start) return fail(SAS_ERR_NULL, "q_start is NULL (prefill needs the first row position)");
  if ((st = check_rows(p, tq, q_start, &tab)) != SAS_OK) return st;
  if ((st = check_sel(sel_mode)) != SAS_OK) return st;
  if (!Q || !q_stride || !K || !V || !kv_stride || !idx || !nsel || !O || !dO || !o_stride || !dQ || !dq_stride ||
      !dK || !dV || !dkv_stride || !workspace)
    return fail(SAS_ERR_NULL, "a required pointer is NULL");
  if (gate && (!dgate || !dscore)) return fail(SAS_ERR_NULL, "dgate and dscore are required with a gate");
  if (reps && !gate) return fail(SAS_ERR_SHAPE, "reps carry the selector's gradient, which needs a gate");
  if (reps && (!rep_stride || !aligned16(reps) || !strides_ok(rep_stride, 3, 4)))
    return fail(SAS_ERR_SHAPE, "reps must be 16-byte aligned fp32 with 16-byte-multiple strides");
  if (p->dtype != SAS_BF16) return fail(SAS_ERR_UNSUPPORTED, "the backward takes bf16 Q/K/V/O/dO");
  if (kcap < 1 || kcap > 32767) return fail(SAS_ERR_SHAPE, "kcap must be in [1, 32767]");
  if (scale < 0.f || !isfinite(scale)) return fail(SAS_ERR_SHAPE, "scale must be finite and >= 0");
  // the dK/dV kernel splits a unit's flattened (head, row) index with a 20-bit reciprocal multiply,
  // exact for indices below 128 rows x 64 heads
  if (sel_mode == SAS_SEL_GROUP && p->hq / p->hkv > BWD_MAX_GROUP)
    return fail(SAS_ERR_UNSUPPORTED, "the backward takes at most %d query heads per KV head with per-group units",
                BWD_MAX_GROUP);
  const int eb = elem_bytes(p->dtype);
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(dQ) ||
      !aligned16(dK) || !aligned16(dV) || !strides_ok(q_stride, 3, eb) || !strides_ok(kv_stride, 3, eb) ||
      !strides_ok(o_stride, 3, eb) || !strides_ok(dq_stride, 3, 4) || !strides_ok(dkv_stride, 3, 4))
    return fail(SAS_ERR_SHAPE, "inputs and gradients must be 16-byte aligned with 16-byte-multiple row strides");
  if ((int64_t)(p->max_len - 1) * kv_stride[2] * eb + (int64_t)p->head_dim * eb > 0xFFFFFFFFll)
    return fail(SAS_ERR_UNSUPPORTED, "one (sequence, KV head) K/V slab must span less than 4 GiB");
  if ((31 * q_stride[2] + p->head_dim) * eb > 0xFFFFFFFFll || (31 * o_stride[2] + p->head_dim) * eb > 0xFFFFFFFFll)
    return fail(SAS_ERR_UNSUPPORTED, "32 rows of Q or dO must span less than 4 GiB");
  const BwdPlan pl = bwd_plan(*p, tq, sel_mode, kcap, gate != nullptr);
  if (workspace_bytes < pl.bytes)
    return fail(SAS_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, pl.bytes);
  const float sc = resolve_scale(scale, p->head_dim);
  return hip_status(launch_prefill_backward(*p, tab, Q, q_stride, K, V, kv_stride, O, dO, o_stride, lse, tq, sel_mode, idx,
                                            nsel, gate, kcap, sc, dQ, dq_stride, dK, dV, dkv_stride, dgate, dscore,
                                            reps, rep_stride, workspace, (hipStream_t)stream),
                    "sas_sparse_prefill_backward");
}

}  // extern "C"
