/*
 * cpattn.h -- C ABI of the per-rank attention of load-balanced context
 * parallelism, for AMD Instinct MI355X (gfx950).
 *
 * What is computed. The context-parallel multimodal page
 * (xuesongtap.github.io/2026/03/22/context-parallel-multimodal) describes
 * how a CP group of size P shares one long causal sequence:
 *   - section 1.1: the sequence is cut into 2P chunks and rank r keeps
 *     chunks r and 2P-1-r (head-tail pairing), so every rank gets the same
 *     causal work;
 *   - sections 2 and 4.1: an image-token prefix is never split; every rank
 *     keeps all of it and only the text is cut into chunks;
 *   - section 5.3: packed samples are delimited by cu_seqlens and are
 *     balanced sample by sample.
 * Each rank then attends its rows causally to the key/value blocks of all
 * P ring steps and combines the per-step partial results by their
 * log-sum-exp (Ring Attention, Liu et al., ICLR 2024, the page's [2]).
 * On one GPU every step's K/V block is read in place from HBM.
 *
 * Conventions shared by every entry point.
 *   - Layout "THD": q is [seq_len, heads, head_dim]; k and v are
 *     [seq_len, kv_heads, head_dim]; all contiguous, head_dim fastest.
 *   - Rank-local rows: for each sample in cu_seqlens order, the image rows
 *     (whole prefix), then text chunk r, then text chunk 2P-1-r. A sample's
 *     text of length T is padded at its end to 2P*c rows, c = ceil(T/2P);
 *     pad rows carry index -1, output 0 and lse -inf.
 *   - Mask: causal with an inclusive diagonal over [image, text] inside a
 *     sample; samples never see each other. Scale 1/sqrt(head_dim); query
 *     head h reads KV head h / (heads / kv_heads).
 *   - cu_seqlens: int32[n_samples + 1], 0 = cu[0] < cu[1] < ... <
 *     cu[n_samples] = seq_len, over real tokens. NULL means one sample
 *     [0, seq_len) and requires n_samples == 1.
 *   - n_img: int32[n_samples], image-prefix length of each sample,
 *     0 <= n_img[s] <= cu[s+1] - cu[s]. NULL means no image prefix.
 *   - Host pointers are read during the call only; the library keeps no
 *     caller pointer. Its only state is a ring of four pinned host staging
 *     buffers per host thread for the plan upload (each hipHostMalloc'd on
 *     first use, grown when a larger plan comes, kept until the process
 *     ends); a call waits for the upload made four calls earlier from the
 *     same buffer before rewriting it, so the host can run up to four calls
 *     ahead of the device. Calls from different threads, or on different
 *     streams, may run concurrently. Apart from the static scratch of
 *     cp_attn_rank_fwd_noalloc, the library holds no device memory.
 *   - Errors: every argument is checked before anything is written or
 *     launched; on error nothing is written and a negative status is
 *     returned. No C++ exception crosses this boundary.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t cp_status;

enum {
  CP_OK = 0,
  CP_EINVAL = -1,       /* malformed argument (sizes, ranks, cu_seqlens, NULL) */
  CP_ENOSPC = -2,       /* caller buffer (index capacity, workspace) too small */
  CP_EUNSUPPORTED = -3, /* valid but not supported (dtype, head_dim, sizes)   */
  CP_EHIP = -4          /* a HIP runtime call failed                          */
};

enum { CP_DTYPE_F32 = 0, CP_DTYPE_BF16 = 1 };

/* Largest cp_size accepted (per-row step masks are 32-bit). */
#define CP_MAX_CP_SIZE 32

/*
 * How the text of a sample is split over the CP group (the *_ex entry
 * points). Both view the padded text as 2P chunks of c = ceil(T/2P).
 *   CP_SPLIT_HEAD_TAIL: rank r holds chunks r and 2P-1-r (the context-
 *     parallel multimodal page, section 1.1: equal causal work per rank).
 *   CP_SPLIT_CONTIGUOUS: rank r holds chunks 2r and 2r+1, i.e. the r-th
 *     contiguous P-th of the text -- the plain split that section 1.1
 *     describes as unbalanced under a causal mask (later ranks do more).
 * The entry points without the suffix use CP_SPLIT_HEAD_TAIL.
 */
enum { CP_SPLIT_HEAD_TAIL = 0, CP_SPLIT_CONTIGUOUS = 1 };

/*
 * How the ring steps of a rank's rows are laid over workgroups (the
 * schedule argument of cp_attn_rank_workspace_size_ex and
 * cp_attn_rank_fwd_ex). Both give the same rows up to floating-point
 * rounding order (the log-sum-exp merge is an exact refactoring of the
 * softmax, Ring Attention's blockwise combination).
 *   CP_SCHED_ROW_TILE: one workgroup takes every ring step of a row tile
 *     and carries one online softmax across them, walking the union of the
 *     steps' key ranges in key order (the ranges are disjoint, so this is
 *     the same set of keys); no per-step partial is written. bf16 with
 *     head_dim 128 only.
 *   CP_SCHED_PER_STEP: one workgroup per (row tile, ring step); each writes
 *     its step's partial output and log-sum-exp into the workspace, and a
 *     second pass merges them. The only schedule of fp32 and head_dim 64.
 *   CP_SCHED_AUTO: ROW_TILE where it exists and the grid has at least 512
 *     workgroups (two per compute unit of a 256-CU MI355X), else PER_STEP.
 * The entry points without the suffix use CP_SCHED_AUTO. ROW_TILE for a
 * dtype/head_dim that has no such kernel returns CP_EUNSUPPORTED.
 */
enum { CP_SCHED_AUTO = 0, CP_SCHED_ROW_TILE = 1, CP_SCHED_PER_STEP = 2 };

/*
 * cp_partition_index -- rows of one CP rank (host only, integer, exact).
 *
 * Page section 1.1 (chunks [cp_rank, 2*cp_size-cp_rank-1]), section 4.1
 * (image prefix kept whole), section 5.3 (per-sample split).
 *
 * index: host int32[capacity]; receives the global token id of every
 *   rank-local row (-1 for pad rows). May be NULL to query the row count.
 * n_rows: host, receives the number of rank-local rows R.
 * cu_rows_local: host int32[n_samples + 1] or NULL; receives the sample
 *   boundaries in rank-local row order.
 * Returns CP_ENOSPC (writing nothing) if index != NULL and capacity < R.
 */
cp_status cp_partition_index(int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                             int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                             int32_t *index, int64_t capacity, int64_t *n_rows,
                             int32_t *cu_rows_local);

/*
 * cp_pair_counts -- unmasked (query, key) pairs per head on one rank
 * (host only, exact). A row at position p of its sample sees p + 1 keys.
 * pairs_real sums over real rows; pairs_padded also counts every pad row
 * as a token at its padded text offset, which head-tail pairing equalises
 * across ranks exactly (page section 1.1). Either output may be NULL.
 */
cp_status cp_pair_counts(int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                         int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                         int64_t *pairs_padded, int64_t *pairs_real);

/*
 * cp_attn_rank_workspace_size -- bytes of device workspace that
 * cp_attn_rank_fwd needs for these arguments (host only). The workspace
 * holds the uploaded plan and, where the ring steps are merged in a
 * separate pass (fp32, head_dim 64, small bf16 grids), the per-step partial
 * outputs fp32 [P, R, heads, head_dim] and log-sum-exps [P, heads, R].
 */
cp_status cp_attn_rank_workspace_size(int64_t seq_len, const int32_t *n_img,
                                      const int32_t *cu_seqlens, int32_t n_samples,
                                      int32_t cp_size, int32_t cp_rank, int32_t heads,
                                      int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                      size_t *bytes);

/*
 * cp_attn_rank_plan_stats -- diagnostics of the work list cp_attn_rank_fwd
 * builds for these arguments (host only, integer, exact).
 *
 * n_tiles: row tiles; n_entries: (row tile, ring step) work entries;
 * kv_tiles: key tiles walked per head group, summed over entries;
 * covered_pairs: (query, key) pairs per head that the entries' key spans
 *   expose under the causal mask -- equal to pairs_real of cp_pair_counts
 *   when every visible pair is scheduled exactly once;
 * step_pairs: host int64[cp_size] or NULL; the same count split by ring
 *   step (step s reads the keys of source rank (cp_rank - s) mod cp_size).
 * Any output may be NULL.
 */
cp_status cp_attn_rank_plan_stats(int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                                  int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                                  int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                  int64_t *n_tiles, int64_t *n_entries, int64_t *kv_tiles,
                                  int64_t *covered_pairs, int64_t *step_pairs);

/*
 * cp_attn_rank_fwd -- forward attention of one CP rank's rows.
 *
 * Steps, all enqueued on `stream` (no host synchronisation):
 *   1. plan on the host (partition, per-step key spans, work list) and
 *      upload it into the workspace;
 *   2. gather the rank's query rows from q (page section 1.1, index_select):
 *      fused into step 3's query loads -- a row tile is a run of
 *      consecutive global ids, read in place from q;
 *   3. for every ring step s = 0..P-1 (source rank j = (r - s) mod P; the
 *      image prefix and the rank's own chunks at s = 0, chunks j and
 *      2P-1-j at s > 0), blockwise causal attention of the rank's rows to
 *      that step's keys, each step giving a partial output normalised by
 *      its own softmax sum, and that sum's log-sum-exp;
 *   4. merge the partials of each row by their log-sum-exp (Ring
 *      Attention's combination of blockwise results).
 * With bf16 and head_dim 128, steps 3 and 4 run in one kernel: a workgroup
 * takes all ring steps of a row tile, walks the union of their key ranges
 * in key order and merges every key block into one running output by the
 * online-softmax (log-sum-exp) update, so no partial leaves its registers;
 * the result equals the per-step partials merged by log-sum-exp up to
 * rounding order. Other dtypes, head_dim 64 and small grids write per-step partials
 * for all rows and merge them in a separate pass (cp_lse_merge's kernel).
 *
 * q, k, v: device, dtype CP_DTYPE_BF16 or CP_DTYPE_F32, THD layout.
 * out: device [R, heads, head_dim] in dtype; lse: device fp32 [heads, R],
 *   natural log. R is the row count from cp_partition_index.
 * workspace: device, at least cp_attn_rank_workspace_size bytes, 256-byte
 *   aligned; its contents on entry are ignored.
 * stream: a hipStream_t (NULL = the null stream).
 * head_dim must be 64 or 128; heads % kv_heads == 0; cp_size <= 32;
 * seq_len < 2^31. Results are deterministic: no floating-point atomics,
 * fixed merge order.
 */
cp_status cp_attn_rank_fwd(const void *q, const void *k, const void *v, int32_t dtype,
                           int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                           int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t heads,
                           int32_t kv_heads, int32_t head_dim, void *out, float *lse,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * cp_attn_rank_fwd_timed -- cp_attn_rank_fwd that also records six
 * caller-created hipEvent_t on `stream` at its stage boundaries:
 * events[0] before the plan upload, [1] after it, [2] and [3] right after
 * [1] (the Q gather is done by the attention kernels as they load Q, and V
 * is read in its own layout, so those two stages are empty), [4] after the
 * attention, [5] after the merge (right after [4] where the attention
 * kernel merges the ring steps itself). A caller can then
 * time one stage with hipEventElapsedTime, without a profiler. events may
 * be NULL (then this is exactly cp_attn_rank_fwd), and so may any entry:
 * that boundary is then not recorded (each record costs a few microseconds
 * on the stream). The library does not keep the events.
 */
cp_status cp_attn_rank_fwd_timed(const void *q, const void *k, const void *v, int32_t dtype,
                                 int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                                 int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                                 int32_t heads, int32_t kv_heads, int32_t head_dim, void *out,
                                 float *lse, void *workspace, size_t workspace_bytes,
                                 void *stream, void *const *events);

/*
 * cp_attn_rank_fwd_noalloc -- cp_attn_rank_fwd for callers that cannot
 * allocate device memory or hand over a workspace: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as cp_attn_rank_fwd, without the
 * workspace. Its scratch (the uploaded plan; on the fp32 and head_dim-64
 * paths also the per-step partials) is a static device array of
 * CP_NOALLOC_SCRATCH_BYTES per GPU, held from the library's first use on
 * that GPU until the process ends. A problem whose scratch would exceed it
 * returns CP_ENOSPC before any device work. bf16 with head_dim 128 always
 * takes the row-tile schedule (CP_SCHED_ROW_TILE: no partials), so there
 * the limit is the plan alone: 8 bytes per rank-local row plus about 50 per
 * (row tile, ring step), e.g. about a million rank rows at P = 8 with 64-row
 * tiles. The exact need is what cp_attn_rank_workspace_size_ex returns for
 * CP_SPLIT_HEAD_TAIL with that schedule (CP_SCHED_AUTO on the other paths).
 *
 * It calls no hipMalloc, hipHostMalloc or hipFree: the plan is copied from
 * ordinary host memory, so the call returns only after that copy has run,
 * i.e. after `stream` has finished the work queued on it before this call
 * (the kernels themselves are enqueued asynchronously). Every call on one
 * GPU uses the same array and overwrites it: calls that overlap on one GPU
 * (other streams, other host threads) race; calls on one stream are
 * ordered. Nothing in the array needs to start at zero.
 */
#define CP_NOALLOC_SCRATCH_BYTES (16u << 20)
cp_status cp_attn_rank_fwd_noalloc(const void *q, const void *k, const void *v, int32_t dtype,
                                   int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                                   int32_t n_samples, int32_t cp_size, int32_t cp_rank,
                                   int32_t heads, int32_t kv_heads, int32_t head_dim, void *out,
                                   float *lse, void *stream);

/*
 * cp_gather_rows -- the chunk-index gather alone (page section 1.1,
 * index_select on the sequence dimension): dst[i, :] = src[index[i], :]
 * for index[i] >= 0 and 0 for index[i] == -1.
 *
 * src: device [src_rows, row_elems]; dst: device [n_rows, row_elems];
 * index: device int32[n_rows], each -1 or in [0, src_rows) (not checked on
 * the device: the caller guarantees it). row_elems * element size must be
 * a multiple of 16 bytes; src, dst 16-byte aligned.
 */
cp_status cp_gather_rows(const void *src, int32_t dtype, int64_t src_rows, int64_t row_elems,
                         const int32_t *index, int64_t n_rows, void *dst, void *stream);

/*
 * cp_lse_merge -- the log-sum-exp merge alone (Ring Attention's combination
 * of blockwise partial results).
 *
 * part_out: device fp32 [n_steps, n_rows, heads, head_dim], each partial
 *   already normalised by its own softmax sum; part_lse: device fp32
 *   [n_steps, heads, n_rows]; step_mask: device uint32[n_rows], bit s set
 *   when row has a partial from step s (other steps are not read).
 * For each (row, head): m = max_s lse_s, w_s = exp(lse_s - m),
 *   out = sum_s w_s * part_s / sum_s w_s, lse = m + ln(sum_s w_s);
 *   steps are taken in increasing s. A row with mask 0 gets out 0, lse -inf.
 * out: device [n_rows, heads, head_dim] in dtype; lse: device fp32
 *   [heads, n_rows]. n_steps <= 32, head_dim 64 or 128.
 */
cp_status cp_lse_merge(const float *part_out, const float *part_lse, const uint32_t *step_mask,
                       int32_t n_steps, int64_t n_rows, int32_t heads, int32_t head_dim,
                       int32_t dtype, void *out, float *lse, void *stream);

/*
 * The same operations with an explicit split (CP_SPLIT_*) and, for the
 * workspace size and the forward, an explicit schedule (CP_SCHED_*). An
 * unknown split or schedule returns CP_EUNSUPPORTED and writes nothing.
 * Everything else -- arguments, layouts, errors -- is as for the entry
 * point without the suffix; cp_attn_rank_fwd_ex also takes the optional six
 * events of cp_attn_rank_fwd_timed (NULL: none). A workspace sized for one
 * (split, schedule) is valid only for that pair.
 */
cp_status cp_partition_index_ex(int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                                int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                                int32_t *index, int64_t capacity, int64_t *n_rows,
                                int32_t *cu_rows_local);
cp_status cp_pair_counts_ex(int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                            int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                            int64_t *pairs_padded, int64_t *pairs_real);
cp_status cp_attn_rank_workspace_size_ex(int64_t seq_len, const int32_t *n_img,
                                         const int32_t *cu_seqlens, int32_t n_samples,
                                         int32_t cp_size, int32_t cp_rank, int32_t split,
                                         int32_t schedule, int32_t heads, int32_t kv_heads, int32_t head_dim,
                                         int32_t dtype, size_t *bytes);
cp_status cp_attn_rank_plan_stats_ex(int64_t seq_len, const int32_t *n_img,
                                     const int32_t *cu_seqlens, int32_t n_samples, int32_t cp_size,
                                     int32_t cp_rank, int32_t split, int32_t heads,
                                     int32_t kv_heads, int32_t head_dim, int32_t dtype,
                                     int64_t *n_tiles, int64_t *n_entries, int64_t *kv_tiles,
                                     int64_t *covered_pairs, int64_t *step_pairs);
cp_status cp_attn_rank_fwd_ex(const void *q, const void *k, const void *v, int32_t dtype,
                              int64_t seq_len, const int32_t *n_img, const int32_t *cu_seqlens,
                              int32_t n_samples, int32_t cp_size, int32_t cp_rank, int32_t split,
                              int32_t schedule, int32_t heads, int32_t kv_heads, int32_t head_dim,
                              void *out, float *lse, void *workspace, size_t workspace_bytes,
                              void *stream, void *const *events);

/*
 * cp_attn_rank_bwd -- gradients of one CP rank's attention share.
 *
 * For a loss whose gradient w.r.t. the rank's forward output is dout, the
 * softmax-attention chain rule over the same rows and ring-step keys as
 * cp_attn_rank_fwd: with P = exp(S - lse) (S = q k^T / sqrt(head_dim),
 * lse the forward's), Delta = rowsum(dout * out):
 *   dv = P^T dout;  ds = P * (dout v^T - Delta);
 *   dq = ds k / sqrt(head_dim);  dk = ds^T q / sqrt(head_dim).
 * Ring Attention's backward passes the same blockwise steps around the
 * ring in reverse; on one GPU every step's K/V is in HBM and the gradient
 * of a key simply sums over the rank's rows.
 *
 * q, k, v: as for cp_attn_rank_fwd (device, THD); out, lse: that call's
 * outputs for the same arguments; dout: device [R, heads, head_dim] in
 * dtype. split: CP_SPLIT_*.
 * dq: device fp32 [R, heads, head_dim] (rank-local rows; pad rows 0).
 * dk, dv: device fp32 [seq_len, kv_heads, head_dim]: every key's gradient
 *   from this rank's rows, summed over the query heads of its KV head (0
 *   for keys no row of the rank sees). Summing dk, dv over all ranks of a
 *   CP group, and scattering each rank's dq back by its index, gives the
 *   gradients of the whole sequence (the reverse ring / all-reduce).
 * workspace: device, cp_attn_rank_bwd_workspace_size bytes, 256-byte
 *   aligned. dtype and head_dim as for cp_attn_rank_fwd: bf16 with
 *   head_dim 128 runs on MFMA (P and dS rounded to bf16 for the products);
 *   fp32 inputs and head_dim 64 run fp32 FMA kernels (P and dS in fp32).
 *   Deterministic (no atomics).
 */
cp_status cp_attn_rank_bwd_workspace_size(int64_t seq_len, const int32_t *n_img,
                                          const int32_t *cu_seqlens, int32_t n_samples,
                                          int32_t cp_size, int32_t cp_rank, int32_t split,
                                          int32_t heads, int32_t kv_heads, int32_t head_dim,
                                          int32_t dtype, size_t *bytes);
cp_status cp_attn_rank_bwd(const void *q, const void *k, const void *v, const void *out,
                           const float *lse, const void *dout, int32_t dtype, int64_t seq_len,
                           const int32_t *n_img, const int32_t *cu_seqlens, int32_t n_samples,
                           int32_t cp_size, int32_t cp_rank, int32_t split, int32_t heads,
                           int32_t kv_heads, int32_t head_dim, float *dq, float *dk, float *dv,
                           void *workspace, size_t workspace_bytes, void *stream);

/* Static English text for a status code. */
const char *cp_status_string(cp_status s);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
