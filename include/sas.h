/*
 * sas.h - C ABI of the MI355X (gfx950) content-selected block-sparse attention library.
 *
 * Pages cited (by title; section in brackets):
 *   [SAS]  "SAS: 通过端到端优化上下文排序的简单注意力稀疏化"
 *   [BLOG] "稀疏注意力" (blog.vegetog.com)
 *   [GSA]  "开源大模型注意力机制演进:从全注意力到门控稀疏注意力的工程实践"
 *   [SSA]  "通过Gist Token的简化稀疏注意力"
 *   [SF]   "稀疏注意力的Trade-offs：Transformer大语言模型实证研究"
 *
 * The path ([GSA] section 4 pseudo-code steps 1-3, [SAS] method, [SSA] method):
 *   sas_block_reps    one representative key per block (mean of its keys)
 *   sas_block_reps_update  the same for the blocks from a given one on (a decode loop)
 *   sas_block_reps_paged / sas_sparse_prefill_paged / sas_sparse_decode_paged  the same over a
 *                     paged KV cache
 *   sas_block_scores  score every earlier block against each selection unit's queries
 *   sas_topk_select   top-k blocks + the current block (+ block 0), optional log-gate
 *   sas_sparse_prefill / sas_sparse_decode  attention over the selected blocks only
 *   sas_hssa_select_decode / sas_hssa_decode  two-level gist selection (meta-gists) and its
 *                     attention, for decode
 *   sas_sparse_prefill_lse  sas_sparse_prefill that also keeps each row's log-sum-exp (training)
 *   sas_sparse_prefill_backward  gradients of the sparse prefill (Q, K, V, gates, scores)
 *
 * Conventions shared by every entry point
 *   - Shapes.  B sequences, Hq query heads, Hkv KV heads (Hq % Hkv == 0, G = Hq/Hkv),
 *     head dim d in {64, 128}, block size blk in {64, 128}.  Sequence b holds L_b
 *     tokens; block j covers positions [j*blk, min((j+1)*blk, L_b)); NB_b = ceil(L_b/blk).
 *   - Element strides are in elements (not bytes); the last dimension (d) is contiguous.
 *     Q and O are [B, Hq, T, d]; K and V are [B, Hkv, Lmax, d]; gist K/V [B, Hkv, NC, d].
 *   - seq_lens and q_start are HOST arrays of int32 (read during the call, not kept), except
 *     that the decode loop's entry points take seq_lens in device memory when
 *     sas_problem.seq_lens_device = 1 (see below).
 *     Every other pointer is DEVICE memory owned by the caller; the library never
 *     allocates, frees or keeps device memory, and never synchronises the stream.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before anything is launched; validation makes
 *     no HIP call, so an invalid call returns an error code and touches nothing.
 *     Launch failures return SAS_ERR_HIP.  sas_last_error() gives a thread-local text.
 *   - Selection unit ([SF] 2.1: prefill selects block to block; [SSA] method item 2:
 *     grouped or per-head expansion):
 *       decode : one unit per (sequence, selector head), the row at position L_b - 1;
 *       prefill: rows at positions q_start[b] + t, t < tq; the rows that fall in one
 *                block c form one unit per selector head.
 *     Selector head: SAS_SEL_GROUP -> KV head g (its G query heads pooled);
 *                    SAS_SEL_HEAD  -> query head h (uses KV head h / G).
 *     Unit array index: u = (b * S + s) * QB + i, S = Hkv or Hq, QB = sas_num_qblocks(tq, blk),
 *     i = c - floor(q_start[b] / blk).  Decode: QB = 1, i = 0.
 */
#ifndef SAS_H
#define SAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAS_OK = 0,
  SAS_ERR_NULL = -1,        /* a required pointer is NULL                                  */
  SAS_ERR_SHAPE = -2,       /* inconsistent sizes, strides, lengths, budget or kcap        */
  SAS_ERR_UNSUPPORTED = -3, /* valid but not built: d, blk, dtype or mode combination      */
  SAS_ERR_WORKSPACE = -4,   /* workspace smaller than the size query returns               */
  SAS_ERR_HIP = -5          /* a HIP launch failed; see sas_last_error()                   */
} sas_status;

typedef enum { SAS_F32 = 0, SAS_BF16 = 1 } sas_dtype;
typedef enum { SAS_SEL_GROUP = 0, SAS_SEL_HEAD = 1 } sas_sel_mode;
typedef enum { SAS_REPS_POOLED = 0, SAS_REPS_GIST = 1 } sas_reps_kind;

#define SAS_MAX_BATCH 64 /* sequences per call */

typedef struct sas_problem {
  int32_t batch;            /* B, 1 .. SAS_MAX_BATCH                                       */
  int32_t hq, hkv;          /* query heads, KV heads                                        */
  int32_t head_dim;         /* d                                                            */
  int32_t block;            /* blk: tokens per block (SSA: per chunk)                       */
  int32_t dtype;            /* sas_dtype of Q, K, V, O and gist K/V                         */
  int32_t max_len;          /* Lmax: token capacity of K/V (every L_b <= Lmax)              */
  const int32_t *seq_lens;  /* HOST [B]: L_b >= 1 (DEVICE [B] when seq_lens_device = 1)     */
  int32_t seq_lens_device;  /* 0: seq_lens is host memory; 1: device memory (see below)     */
} sas_problem;

/* Lengths in device memory (seq_lens_device = 1) serve a decode loop whose step is captured once in
 * a HIP graph and replayed while the lengths grow: the kernels read L_b from seq_lens when they run,
 * so nothing on the host depends on them.  The host sizes launches and checks kcap, scores_ld and
 * workspaces for the capacity max_len; a length outside [1, max_len] is clamped into it.  Taken by
 *   sas_block_reps (every block up to L_b), sas_block_reps_update (first_block must be NULL: the
 *   block holding position L_b - 1 is pooled again, which is all one appended token changes),
 *   sas_block_reps_paged, sas_select_decode, sas_sparse_decode (bf16), sas_sparse_decode_noalloc,
 *   sas_sparse_decode_paged;
 * every other entry point returns SAS_ERR_UNSUPPORTED.  kcap comes from sas_required_kcap on a
 * host problem at max_len. */

/* Budget ([SAS] method: a fixed budget of k context units per query, configurable;
 * [GSA] section 4 pseudo-code keep_ratio).  For a unit whose current block is c:
 *   candidates = blocks 0 .. c-1, minus block 0 when force_sink;
 *   k = ceil(sqrt_num * sqrt(c + count_current) / sqrt_den) if sqrt_den > 0 (integer-exact)
 *   k = k_fixed                                            else if frac_den == 0
 *   k = ceil(frac_num * (c + count_current) / frac_den)    otherwise (integer arithmetic)
 *   k is capped at the candidate count; the current block c is always added ([SAS] core
 *   insight), and block 0 when force_sink ([SF] 2.2.3, first prefix block).
 *   The square-root rule is the length-adaptive budget ([SF] 4.3.2 iso-error curve: the budget
 *   that keeps one error level goes from 1/10 of a 16K context to 1/20 of a 64K one, i.e. the kept
 *   tokens double when the length quadruples; 4.4.2: grow the budget sub-linearly with length).
 *   It is evaluated exactly: k is the smallest integer with (k sqrt_den)^2 >= sqrt_num^2 n.
 * Coverage budget ([SF] 2.3, threshold-based allocation), when coverage > 0: k is the
 *   smallest number of candidates, in (score descending, index ascending) order, whose share of
 *   the candidates' softmax mass (softmax of their scores) is >= coverage (<= 1), capped by the
 *   rule above only when k_fixed > 0, frac_den > 0 or sqrt_den > 0.  The shares are summed in fp32: where the
 *   exact share of the k-th candidate lies within ~1e-5 of coverage, k may differ by one from
 *   an exact evaluation.
 * Shared budget ([SF] 2.3, Ada-KV: top k x h over h heads), when shared_heads = 1 (per-head
 *   selection only, no coverage): the G query heads of a KV group at one query block share a
 *   budget of G times the k above.  Their candidates compete as (head, block) pairs ranked by
 *   (score descending, head ascending, block ascending); each head keeps its blocks among the
 *   first G * k pairs, plus its forced blocks, so list lengths vary between heads (kcap from
 *   sas_required_kcap covers min(G * k, candidates)). */
typedef struct sas_budget {
  int32_t k_fixed;
  int32_t frac_num, frac_den, count_current;
  int32_t force_sink;       /* 1: block 0 is always kept                                    */
  int32_t gate;             /* 1: write the log-gate over the selected set                  */
  float coverage;           /* 0: off; else in (0, 1]                                        */
  int32_t shared_heads;     /* 1: the heads of a KV group share G * k (per-head selection)     */
  int32_t sqrt_num, sqrt_den; /* square-root (length-adaptive) rule when sqrt_den > 0; each <= 65535 */
} sas_budget;

/* Number of query blocks tq consecutive positions can touch: ceil((tq-1)/blk) + 1. */
int32_t sas_num_qblocks(int32_t tq, int32_t block);

/* Smallest kcap that holds every unit's selected list for this call (>= 1), or a negative
 * sas_status for invalid arguments.  q_start: HOST [B], or NULL for decode. */
int32_t sas_required_kcap(const sas_problem *p, int32_t tq, const int32_t *q_start,
                          const sas_budget *budget);

/* A1 - block representatives ([SF] 2.1 representation heuristics: block-pooled token
 * representations; [GSA] section 4 step 1).
 *   reps[b, g, j, :] = (1/n_j) * sum of K[b, g, t, :] over the n_j present tokens of block j,
 *   for j < NB_b, in fp32 (blocks >= NB_b are left untouched).
 *   K: [B, Hkv, Lmax, d] dtype, k_stride = {batch, head, token}.
 *   reps: [B, Hkv, >= NB_b, d] fp32, rep_stride = {batch, head, block}. */
sas_status sas_block_reps(const sas_problem *p, const void *K, const int64_t k_stride[3],
                          float *reps, const int64_t rep_stride[3], void *stream);

/* A1, incremental (a decode loop that appends tokens: only the blocks that changed are pooled
 * again).  Same arguments and layout as sas_block_reps, plus
 *   first_block: HOST [B]; blocks first_block[b] .. NB_b - 1 of sequence b are recomputed
 *                (0 <= first_block[b] <= NB_b; NB_b means none).  After appending tokens to a
 *                sequence whose length was L_old, first_block[b] = floor(L_old / blk) makes reps
 *                equal, bit for bit, to a full sas_block_reps at the new length (each block is
 *                pooled by the same code in the same order).
 *   Errors: first_block NULL -> SAS_ERR_NULL; an entry outside [0, NB_b] -> SAS_ERR_SHAPE. */
sas_status sas_block_reps_update(const sas_problem *p, const void *K, const int64_t k_stride[3],
                                 float *reps, const int64_t rep_stride[3], const int32_t *first_block,
                                 void *stream);

/* A2 - block scores ([GSA] section 4 step 1; [SSA] method item 1, query against every
 * historical gist).  For unit u with current block c and query vectors q (its rows times
 * its heads):  scores[u, j] = scale * mean_q (q . r_j)   for every block j <= c that has a
 * representative, -inf for the other j <= c; entries j > c are not written.
 *   reps_kind SAS_REPS_POOLED: r = fp32 reps from sas_block_reps (every block has one).
 *   reps_kind SAS_REPS_GIST  : r = gist keys of dtype p->dtype, one per complete chunk
 *                              ([SSA] method: a gist token after each chunk); only the
 *                              chunks j < c are scored (the current chunk is attended raw).
 *   Q: [B, Hq, T, d] dtype, q_stride = {batch, head, row}; tq rows per sequence.
 *   q_start: HOST [B] first row position, or NULL for decode (tq == 1, row at L_b - 1).
 *   scale: > 0, or 0 for 1/sqrt(d).
 *   scores: [B * S * QB, scores_ld] fp32, scores_ld >= max_b NB_b.
 *   workspace: device scratch of sas_block_scores_workspace() bytes (0 for decode). */
size_t sas_block_scores_workspace(const sas_problem *p, int32_t tq, int32_t sel_mode);
sas_status sas_block_scores(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                            int32_t tq, const int32_t *q_start, const void *reps, int32_t reps_kind,
                            const int64_t rep_stride[3], int32_t sel_mode, float scale,
                            float *scores, int64_t scores_ld, void *workspace,
                            size_t workspace_bytes, void *stream);

/* A3 - top-k + forced blocks + log-gate ([SAS] core modules 2-4; [BLOG] 4.6).
 *   Keeps the k best candidates by (score descending, block index ascending), adds the
 *   current block and, with force_sink, block 0.
 *   idx [units, kcap] int32: the selected blocks in ascending order, then -1 padding;
 *   nsel [units] int32: list length (0 for unit slots no row falls in);
 *   gate [units, kcap] fp32 (required iff budget->gate, else ignored and may be NULL):
 *   g = s_j - log(sum over the selected set of exp(s)), 0 in the padding.
 *   A gate value belongs to the unit, not to a row: in prefill it comes from scores that pool all of
 *   the unit's rows, and the current block's score uses the mean of all of that block's present keys
 *   (later positions included).  Which keys a row attends stays causal; the gate value added to its
 *   logits is a unit-level quantity, so prefill and decode at the same position can differ in it.
 *   kcap must be >= sas_required_kcap(). */
sas_status sas_topk_select(const sas_problem *p, const float *scores, int64_t scores_ld,
                           int32_t tq, const int32_t *q_start, int32_t sel_mode,
                           const sas_budget *budget, int32_t kcap, int32_t *idx, int32_t *nsel,
                           float *gate, void *stream);

/* A4 - sparse prefill ([BLOG] sections 2 and 7: masked softmax attention computed block by
 * block, skipping masked blocks; [SAS] core modules 2-3: log-gate inside the softmax).
 *   O[b, h, t] = softmax_s(scale * q . k_s + gate_u(block(s))) v_s over keys s of the
 *   unit's selected blocks with s <= q_start[b] + t.
 *   Q, O: [B, Hq, T, d] (q_stride, o_stride = {batch, head, row}); K, V: kv_stride.
 *   gate: [units, kcap] or NULL for no gate.  scale: > 0 or 0 for 1/sqrt(d).
 *   bf16: the K/V rows of one (sequence, KV head) must span less than 4 GiB
 *   ((max_len - 1) * row stride + d elements), else SAS_ERR_UNSUPPORTED. */
sas_status sas_sparse_prefill(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                              const void *K, const void *V, const int64_t kv_stride[3],
                              int32_t tq, const int32_t *q_start, int32_t sel_mode,
                              const int32_t *idx, const int32_t *nsel, const float *gate,
                              int32_t kcap, float scale, void *O, const int64_t o_stride[3],
                              void *stream);

/* sas_sparse_prefill that also writes each row's log-sum-exp of its logits (natural log):
 *   lse[(b * Hq + h) * tq + t] = log sum_s exp(scale * q . k_s + gate_u(block(s))) over the row's
 *   visible keys, fp32, for the rows the call computes (others untouched).  A training step keeps it
 *   for sas_sparse_prefill_backward.  lse NULL: same as sas_sparse_prefill.  bf16 only (fp32:
 *   SAS_ERR_UNSUPPORTED when lse is given). */
sas_status sas_sparse_prefill_lse(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                                  const void *K, const void *V, const int64_t kv_stride[3], int32_t tq,
                                  const int32_t *q_start, int32_t sel_mode, const int32_t *idx,
                                  const int32_t *nsel, const float *gate, int32_t kcap, float scale, void *O,
                                  const int64_t o_stride[3], float *lse, void *stream);

/* A2 + A3 fused for decode: the scores and the selection of sas_block_scores (q_start = NULL)
 * followed by sas_topk_select, in one launch ([GSA] section 4 pseudo-code steps 1-2).  Same
 * outputs (scores rows j <= c, idx, nsel, gate).  Needs every current block c <= 2048 (e.g.
 * 131,136 tokens at blk 64; longer contexts: use the two calls) and at most 16 query heads
 * per KV head.
 *   workspace: sas_select_decode_workspace() bytes of arrival counters.  It must be zero
 *   before its first use; every call leaves it zero again.  Calls that share one workspace
 *   must not overlap in time (two streams running at once would race on the counters). */
size_t sas_select_decode_workspace(const sas_problem *p);
sas_status sas_select_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                             const void *reps, int32_t reps_kind, const int64_t rep_stride[3],
                             int32_t sel_mode, float scale, const sas_budget *budget, int32_t kcap,
                             float *scores, int64_t scores_ld, int32_t *idx, int32_t *nsel,
                             float *gate, void *workspace, size_t workspace_bytes, void *stream);

/* A5/A6 - sparse decode; one row per (sequence, query head) at position L_b - 1.
 *   Q, O: [B, Hq, d] (q_stride, o_stride = {batch, head}).
 *   Gist mode ([SSA] method items 2-3: hybrid attention) when gist_k and gist_v are both
 *   non-NULL: the key set is the raw tokens of the selected chunks plus the gist token of
 *   every complete chunk before the current one that is not selected; gist_stride =
 *   {batch, head, chunk}; the gate must be NULL in gist mode.
 *   workspace: sas_sparse_decode_workspace() bytes: per-unit arrival counters followed by
 *   the split-K partial records (bf16 path; 0 bytes for fp32).  The counters must be zero
 *   before the workspace's first use; every call leaves them zero again.  Calls that share
 *   one workspace must not overlap in time.
 *   bf16: SAS_ERR_UNSUPPORTED when kcap (plus the gist tiles) needs more split-K records per
 *   unit than the in-kernel merge can stage (with 16 heads per KV head at d 128: about 3000
 *   list entries of 64 keys; far more with fewer heads; units of one head, per-head selection,
 *   about 10,900 tiles of 64 keys). */
size_t sas_sparse_decode_workspace(const sas_problem *p, int32_t sel_mode, int32_t kcap,
                                   int32_t gist);
sas_status sas_sparse_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                             const void *K, const void *V, const int64_t kv_stride[3],
                             const void *gist_k, const void *gist_v, const int64_t gist_stride[3],
                             int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                             const float *gate, int32_t kcap, float scale, void *O,
                             const int64_t o_stride[2], void *workspace, size_t workspace_bytes,
                             void *stream);

/* sas_sparse_decode for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments without the workspace, the same
 * kernels, outputs and errors.  The split-K scratch (arrival counters and partial records) lives in a static
 * device array of the library, SAS_DECODE_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on
 * holds until the process ends; the call makes no allocation (its first call on a device looks up the
 * array's device address).  Each call clears the array's arrival counters on `stream` with a small fill
 * kernel before the attention kernel.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (two streams, two threads) race on it and must be serialised by the caller.
 *   Errors: as sas_sparse_decode; SAS_ERR_WORKSPACE when sas_sparse_decode_workspace() for the call
 *   exceeds SAS_DECODE_NOALLOC_SCRATCH_BYTES. */
#define SAS_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
sas_status sas_sparse_decode_noalloc(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                                     const void *K, const void *V, const int64_t kv_stride[3],
                                     const void *gist_k, const void *gist_v, const int64_t gist_stride[3],
                                     int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                                     const float *gate, int32_t kcap, float scale, void *O,
                                     const int64_t o_stride[2], void *stream);

/* Paged K/V ([BLOG] section 5: decode reads the KV cache; a serving cache is paged): the cache is
 * pages of one block each, [num_pages, Hkv, blk, d] (page_stride = {page, head, token}, or any
 * layout in which a page holds blk tokens of every KV head without overlapping the next), and
 * block_table: DEVICE [B, table_ld] int32 gives the page of block j of sequence b at
 * block_table[b * table_ld + j] for every j < NB_b (table_ld >= max NB_b).  The library reads
 * the table only; page indices are not checked on the host (they are device memory).
 * sas_block_reps_paged: sas_block_reps / sas_block_reps_update over a paged K (first_block: HOST
 *   [B] or NULL for every block); the reps stay [B, Hkv, NB, d] by logical block.
 * sas_sparse_decode_paged: sas_sparse_decode over paged K/V (bf16; no gist mode); same lists,
 *   workspace and errors.
 * sas_sparse_prefill_paged: sas_sparse_prefill over paged K/V (bf16); same lists and errors.
 * Paged and contiguous caches with equal contents give equal results bit for bit (the same
 * kernels; only the row addresses differ). */
sas_status sas_block_reps_paged(const sas_problem *p, const void *K_pages, const int64_t page_stride[3],
                                const int32_t *block_table, int64_t table_ld, float *reps,
                                const int64_t rep_stride[3], const int32_t *first_block,
                                void *stream);
sas_status sas_sparse_decode_paged(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                                   const void *K_pages, const void *V_pages,
                                   const int64_t page_stride[3], const int32_t *block_table,
                                   int64_t table_ld, int32_t sel_mode, const int32_t *idx,
                                   const int32_t *nsel, const float *gate, int32_t kcap,
                                   float scale, void *O, const int64_t o_stride[2],
                                   void *workspace, size_t workspace_bytes, void *stream);
sas_status sas_sparse_prefill_paged(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                                    const void *K_pages, const void *V_pages,
                                    const int64_t page_stride[3], const int32_t *block_table,
                                    int64_t table_ld, int32_t tq, const int32_t *q_start,
                                    int32_t sel_mode, const int32_t *idx, const int32_t *nsel,
                                    const float *gate, int32_t kcap, float scale, void *O,
                                    const int64_t o_stride[3], void *stream);

/* Two-level gist selection for decode ([SSA] hierarchical extension: meta-gist tokens, gists
 * of gists, make a coarse level; the ordinary gists of the chosen part are then scored and the
 * best chunks expanded).  Readings, as the page gives no more: a group is group_chunks (M)
 * consecutive chunks of blk tokens and has a meta-gist when it is complete and lies before the
 * current chunk c = floor((L_b - 1) / blk), i.e. groups i < c / M.
 *   Level 1 opens the top-k1 of those groups by meta-gist score, plus the trailing group
 *     (chunks floor(c/M) M .. c - 1), which is always open.
 *   Level 2 expands the top-k2 chunks of the open groups by gist score; the current chunk is
 *     always attended raw.  Ties go to the lower index at both levels; scores are
 *     scale * mean over the unit's heads of q . x, as in sas_block_scores.
 *   Attention (sas_hssa_decode) sees the raw tokens of the expanded chunks and of the current
 *     chunk, the gists of the open groups' chunks that were not expanded, and the meta-gists of
 *     the groups that were not opened; no gate.
 * bf16 only; 4 <= M <= 64; c <= 2048, at most 511 groups, and (k1 + 1) * M <= 2048.
 *   Q: [B, Hq, d]; gist_k: [B, Hkv, NC, d] (one per complete chunk); meta_k: [B, Hkv, NM, d].
 *   Outputs per unit u (units as in sas_select_decode):
 *     idx [units, kcap]: the expanded chunks ascending, then c; -1 padded; nsel[u] = its length
 *                        (min(k2, candidates) + 1), kcap >= that for every unit.
 *     gidx [units, gcap]: the opened groups ascending, then the trailing group floor(c/M) (which
 *                        may hold no complete chunk); -1 padded; gsel[u] = its length
 *                        (min(k1, floor(c/M)) + 1), gcap >= that.
 *   workspace: sas_hssa_select_workspace(p, sel_mode, M, k1) bytes (score rows; no state kept
 *     between calls). */
size_t sas_hssa_select_workspace(const sas_problem *p, int32_t sel_mode, int32_t group_chunks,
                                 int32_t k1);
sas_status sas_hssa_select_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                                  const void *gist_k, const int64_t gist_stride[3],
                                  const void *meta_k, const int64_t meta_stride[3],
                                  int32_t group_chunks, int32_t sel_mode, int32_t k1, int32_t k2,
                                  float scale, int32_t kcap, int32_t gcap, int32_t *idx,
                                  int32_t *nsel, int32_t *gidx, int32_t *gsel, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* Attention of the two-level gist selection (key set above), split-K over 64-key tiles like
 * sas_sparse_decode: per unit, one tile per gidx entry (that group's gists), 64 meta-gists per
 * tile, then the raw tiles of idx.  meta_v: [B, Hkv, NM, d] like meta_k.  workspace:
 * sas_hssa_decode_workspace() bytes; its arrival counters must be zero before the first call,
 * and every call leaves them zero.  Errors as sas_sparse_decode; bf16 only. */
size_t sas_hssa_decode_workspace(const sas_problem *p, int32_t sel_mode, int32_t kcap, int32_t gcap,
                                 int32_t group_chunks);
sas_status sas_hssa_decode(const sas_problem *p, const void *Q, const int64_t q_stride[2],
                           const void *K, const void *V, const int64_t kv_stride[3],
                           const void *gist_k, const void *gist_v, const int64_t gist_stride[3],
                           const void *meta_k, const void *meta_v, const int64_t meta_stride[3],
                           int32_t group_chunks, int32_t sel_mode, const int32_t *idx,
                           const int32_t *nsel, int32_t kcap, const int32_t *gidx, int32_t gcap,
                           float scale, void *O, const int64_t o_stride[2], void *workspace,
                           size_t workspace_bytes, void *stream);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char *sas_last_error(void);

/* Backward of A4 ([SAS] method, core modules 2-3: the selector score enters the logits through a
 * log-softmax over the kept set, so training reaches the scores through the gate; [BLOG] sections 2
 * and 7: the masked softmax attention that sas_sparse_prefill computes).  For the loss
 * sum(O * dO) of one sas_sparse_prefill call with the same lists, gate and scale:
 *   dQ [B, Hq, T, d] fp32 (dq_stride), dK / dV [B, Hkv, Lmax, d] fp32 (dkv_stride): every row
 *   t < tq and every key row < L_b is written (zero where no unit attends it); other rows untouched.
 *   dgate [units, kcap] fp32: gradient of each list entry's gate value (sum of dS over the
 *   block's keys over the unit's rows and heads); dscore [units, kcap] fp32: gradient of the
 *   entry's selector score through g = s - logsumexp(list scores):
 *   dscore_j = dgate_j - exp(g_j) * sum_j' dgate_j'.  Padding entries get 0.  Both are required
 *   iff gate != NULL (without a gate they are not written and may be NULL).
 *   O: the forward output (bf16, o_stride); dO: its gradient (bf16, same strides).
 *   lse: the forward's row log-sum-exp from sas_sparse_prefill_lse ([B, Hq, tq] fp32), or NULL to
 *   recompute it (one more pass over each unit's list).
 *   reps (with a gate; fp32 [B, Hkv, >= NB_b, d], rep_stride as in sas_block_reps): the block
 *   representatives the selection scored, or NULL.  Given, the gradient continues through the
 *   selector ([SAS] method: trained end to end through the gate): the scores are
 *   s_j = scale * qbar . r_j of the unit's mean query vector qbar and the block means r_j, so each of
 *   the unit's query vectors gets scale * sum_j dscore_j r_j / (its vector count) added to dQ, and
 *   each present key of block j gets scale * sum over the units keeping j of dscore_j qbar, divided
 *   by the block's key count, added to dK (a fixed-order sum per block over the units that keep it,
 *   so it is deterministic).  Lists stay fixed.  The gradient follows the forward as defined: a unit's
 *   score pools all of its rows and the current block's mean covers all of that block's present keys,
 *   so a row's loss also reaches, through its unit's gate value, the unit's other rows' queries and
 *   the current block's keys after the row (see sas_topk_select).
 *   Q, K, V, idx, nsel, gate, kcap, scale: as given to sas_sparse_prefill (bf16 only).
 *   kcap <= 32767.  workspace: sas_sparse_prefill_backward_workspace(p, tq, sel_mode, kcap, gate
 *   != NULL) bytes of device scratch (no initial contents needed; it grows with the batch, the rows,
 *   the block count and, with a gate, the block count times the units per KV head).
 *   Arithmetic: P and dS are rounded to bf16 as matrix operands, with fp32 accumulation; dQ, dgate
 *   and dscore are deterministic; dK and dV are too, except in blocks whose selecting units hold
 *   more than 32768 (row, head) pairs in all, or number more than 256: their unit list is cut into
 *   several work items whose partial sums meet in fp32 atomic adds.
 *   Errors: as sas_sparse_prefill; SAS_ERR_UNSUPPORTED for fp32, for per-group units with more than 64
 *   query heads per KV head and for token strides of Q or dO at which 32 rows span 4 GiB or more;
 *   SAS_ERR_WORKSPACE when too small; SAS_ERR_SHAPE for reps without a gate. */
size_t sas_sparse_prefill_backward_workspace(const sas_problem *p, int32_t tq, int32_t sel_mode, int32_t kcap,
                                             int32_t gate);
sas_status sas_sparse_prefill_backward(const sas_problem *p, const void *Q, const int64_t q_stride[3],
                                       const void *K, const void *V, const int64_t kv_stride[3], int32_t tq,
                                       const int32_t *q_start, int32_t sel_mode, const int32_t *idx,
                                       const int32_t *nsel, const float *gate, int32_t kcap, float scale,
                                       const void *O, const void *dO, const int64_t o_stride[3],
                                       const float *lse, float *dQ,
                                       const int64_t dq_stride[3], float *dK, float *dV,
                                       const int64_t dkv_stride[3], float *dgate, float *dscore,
                                       const float *reps, const int64_t rep_stride[3], void *workspace,
                                       size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SAS_H */
