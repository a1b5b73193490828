/*
 * libkvsel -- attention-score token selection on AMD Instinct MI355X (gfx950).
 *
 * The four calls below are the data-parallel hot path of Token-Selective
 * Propagation (FastKV) and of StructKV's pivot-layer pruning:
 *
 *   kvsel_window_score     window softmax over all keys, summed over the
 *                          window rows and the query heads of each GQA group
 *   kvsel_accumulate_stats cross-layer running score, head sum, and the
 *                          per-layer entropy / sparsity / variance
 *   kvsel_topk             top-k plus the window, for either budget
 *   kvsel_gather           compaction of K/V rows and hidden rows
 *
 * with variants: the score from given normalisers (_lse) or with every
 * window row's entropy (_entropy), both budgets at once (kvsel_topk2),
 * several gathers at once (_multi) or into a paged cache (_paged), and the
 * host-side pivot picks (kvsel_pivot_layer, kvsel_pivot_layer_sparsity).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Device pointers point to HIP device memory owned by the caller; the
 *    library never allocates or frees device memory.  Scratch memory is a
 *    caller-provided workspace whose size the matching *_workspace() query
 *    returns (0 means none is needed; ws may then be NULL).
 *  - Host pointers (cu_seqlens, per-sequence budgets) are read during the
 *    call only.  Launch metadata derived from them travels in kernel
 *    arguments, so nothing is copied host->device and nothing is read back.
 *  - Every call enqueues asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream) and returns without synchronising.  Device-side
 *    faults surface at the caller's next synchronisation.
 *  - Every call returns a kvsel_status.  All arguments are validated on the
 *    host before anything is enqueued; a non-OK status means nothing was
 *    enqueued (KVSEL_ELAUNCH excepted: a HIP launch failed, earlier launches
 *    of the same call may have been enqueued).
 *  - Device pointers must be 16-byte aligned.  Device data (values,
 *    indices) is not validated except where stated.
 *  - The library holds no state and is re-entrant; calls on different
 *    streams are independent.  Results are deterministic: no floating-point
 *    atomics are used, every reduction has a fixed order.
 *
 * Packed variable-length batches
 * ------------------------------
 *  A batch of B sequences is packed along the token axis: sequence b owns
 *  rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of every [T, ...] tensor, with
 *  T = cu_seqlens[B].  Positions returned by kvsel_topk are sequence-local.
 */
#ifndef KVSEL_H
#define KVSEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvsel_status {
  KVSEL_OK = 0,
  KVSEL_EINVAL = 1,        /* an argument is invalid (null, misaligned, inconsistent) */
  KVSEL_EUNSUPPORTED = 2,  /* valid but not supported by this build (e.g. head dim) */
  KVSEL_EWORKSPACE = 3,    /* workspace missing or smaller than the query returned */
  KVSEL_ELAUNCH = 4        /* the HIP runtime refused a launch */
} kvsel_status;

/* Packed batch description.  cu_seqlens is a HOST array of batch+1 int32:
 * cu_seqlens[0] == 0, non-decreasing.  batch >= 1. */
typedef struct kvsel_varlen {
  int32_t batch;
  const int32_t* cu_seqlens;
} kvsel_varlen;

/* Human-readable name of a status code (static storage). */
const char* kvsel_status_string(int status);

/* ABI version of this header, bumped on any incompatible change. */
#define KVSEL_ABI_VERSION 1
int kvsel_abi_version(void);

/* Number of selected positions per (row, sequence) for a budget of k tokens
 * with a window of w: min(n, max(k, 0) + w).  The total over the batch,
 * L = sum_b min(n_b, k_b + w), is the length of each output row of
 * kvsel_topk and the number of output rows of kvsel_gather.  Returns -1 on
 * invalid arguments. */
int64_t kvsel_selected_length(const kvsel_varlen* v, const int32_t* k_host, int32_t w);

/*
 * kvsel_window_score -- steps 1 and 2 of token selection.
 *
 * FastKV summary page, section 2A (Token-Selective Propagation): at the TSP
 * layer each token's importance comes from the attention paid to it by a
 * window of the most recent tokens.  FastKV abstract: compression is GQA
 * aware, one decision per KV head.  For sequence b (length n), query head h
 * in KV group g = h / (h_q / h_kv) and window row i (position n - w + i):
 *
 *    P[b,h,i,j] = softmax_j( scale * <q_win[b,i,h,:], k[off_b + j, g, :]> ),
 *                 over the causally visible keys j <= n - w + i
 *    score[g, off_b + j] = sum_{h in group g} sum_{i < w} P[b,h,i,j]
 *
 * Arguments
 *   v        packed batch; every n_b >= w.
 *   q_win    device, bf16 [B, w, h_q, d]: queries of the last w positions.
 *   k        device, bf16 [T, h_kv, d]: the layer's keys.
 *   h_q, h_kv  query and KV head counts; h_q % h_kv == 0.
 *   d        head dimension: 64 or 128 (else KVSEL_EUNSUPPORTED).
 *   w        window length, >= 1.
 *   scale    softmax scale (usually 1/sqrt(d)); finite and > 0.
 *   score    device, fp32 [h_kv, T], written (every element).
 *   lse      device, fp32 [B, h_q, w] natural-log normaliser of each
 *            softmax row, or NULL.
 *   ws       device workspace of kvsel_window_score_workspace() bytes.
 * Returns KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_EWORKSPACE or
 * KVSEL_ELAUNCH.  The workspace query returns 0 for invalid arguments.
 */
size_t kvsel_window_score_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv,
                                    int32_t d, int32_t w);
int kvsel_window_score(const kvsel_varlen* v, const void* q_win, const void* k,
                       int32_t h_q, int32_t h_kv, int32_t d, int32_t w, float scale,
                       float* score, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_window_score_stats -- steps 1 and 2 with the head sum, the running
 * accumulation and the statistics of kvsel_accumulate_stats folded in.
 *
 * FastKV summary page, section 2A (one propagated set per sequence, scored
 * by the sum over KV heads) and StructKV summary page, sections 2A-2B (the
 * score accumulated over layers; entropy, sparsity and variance per layer).
 * The result is that of
 *
 *   kvsel_window_score(v, q_win, k, h_q, h_kv, d, w, scale, score, lse, ...)
 *   kvsel_accumulate_stats(v, score, h_kv, w, h_q / h_kv, c_in, c_out, tok, stats, ...)
 *
 * -- score, lse, c_out and tok bit for bit; stats up to the rounding of
 * its sums, which are added in another order -- but the second pass over
 * the keys does the accumulate call's work on the score it has just formed,
 * so the score is not read back and no further kernel runs.
 *
 * Arguments as for kvsel_window_score, plus those of kvsel_accumulate_stats
 * (each of c_out, tok, stats may be NULL; c_out may alias c_in; with all
 * three NULL this is kvsel_window_score).  ws is a device workspace of
 * kvsel_window_score_stats_workspace() bytes.  Returns KVSEL_OK,
 * KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_EWORKSPACE or KVSEL_ELAUNCH.  The
 * workspace query returns 0 for invalid arguments.
 */
size_t kvsel_window_score_stats_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv, int32_t d,
                                          int32_t w);
int kvsel_window_score_stats(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                             int32_t h_kv, int32_t d, int32_t w, float scale, float* score, float* lse,
                             const float* c_in, float* c_out, float* tok, float* stats, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * kvsel_window_score_noalloc -- kvsel_window_score without a workspace
 * argument and without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP stream
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * kernels and results as kvsel_window_score (bit for bit); the per-chunk
 * partials go to a fixed scratch array of KVSEL_NOALLOC_SCRATCH_BYTES
 * (4 MiB) that the library holds in device memory on every GPU it runs on,
 * until the process ends.  The call itself allocates nothing (no hipMalloc,
 * no allocating library routine); the caller still provides score (and lse).
 *
 * Limit: the partials take kvsel_window_score_workspace() bytes, which must
 * not exceed KVSEL_NOALLOC_SCRATCH_BYTES -- at most 4096 (work units x KV
 * heads) per launch group, e.g. sequences of up to about 2.5M keys at 8 KV
 * heads; larger inputs return KVSEL_EWORKSPACE before anything is enqueued.
 * Arguments and other statuses as for kvsel_window_score (KVSEL_ELAUNCH
 * also when the scratch's device address cannot be looked up).
 *
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (each call writes every partial it reads, so nothing has
 * to be cleared): calls that overlap on one GPU -- on different streams, or
 * from different host threads -- race and give undefined results.
 * Serialise them.
 */
#define KVSEL_NOALLOC_SCRATCH_BYTES 4194304
int kvsel_window_score_noalloc(const kvsel_varlen* v, const void* q_win, const void* k,
                               int32_t h_q, int32_t h_kv, int32_t d, int32_t w, float scale,
                               float* score, float* lse, void* stream);

/*
 * kvsel_window_score_lse -- steps 1 and 2 with the softmax normalisers given.
 *
 * FastKV summary page, section 2A: the window's attention at the TSP layer
 * is part of that layer's own prefill attention, which computes every
 * row's softmax over all keys and with it each row's log-sum-exp.  Given
 * those normalisers the score needs one pass over K instead of two.
 *
 *   score[g, off_b + j] = sum_{h in g} sum_{i < w} exp(scale * <q_win[b,i,h,:], k[off_b+j,g,:]>
 *                                                      - lse_in[b, h, i])
 * over the causally visible keys, i.e. kvsel_window_score's result when
 * lse_in is the normaliser that call returns in `lse` (up to its rounding).
 *
 * Arguments as for kvsel_window_score, plus
 *   lse_in   device fp32 [B, h_q, w]: natural-log normaliser of each window
 *            row, log sum_j exp(scale * <q, k_j>) over its visible keys.
 * No workspace.  Returns KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED or
 * KVSEL_ELAUNCH.
 */
int kvsel_window_score_lse(const kvsel_varlen* v, const void* q_win, const void* k, int32_t h_q,
                           int32_t h_kv, int32_t d, int32_t w, float scale, const float* lse_in,
                           float* score, void* stream);

/*
 * kvsel_window_score_entropy -- steps 1 and 2 plus the entropy of every
 * window row.
 *
 * StructKV summary page, section 2B: the pivot layer is found by watching
 * the attention entropy layer by layer.  Read at the level of the softmax
 * rows, each window row's entropy is
 *
 *    H[b,h,i] = - sum_j P[b,h,i,j] ln P[b,h,i,j]     (nats; 0 ln 0 = 0)
 *
 * over its visible keys, with P as in kvsel_window_score.  The first pass
 * over the keys, which finds every row's normaliser, also keeps
 * tt = sum_j 2^(x_j - m) (x_j - m) beside its running max m and sum l (x the
 * logit in log2 units), so the entropy costs no extra pass over K:
 * H = ln2 * (log2 l - tt / l), both terms non-negative.
 *
 * Arguments as for kvsel_window_score, plus
 *   row_ent  device fp32 [B, h_q, w]: H of every window row, written.
 *   mean_ent device fp32 [B]: per sequence, the mean of H over all h_q * w
 *            rows, or NULL.
 *   ws       device workspace of kvsel_window_score_entropy_workspace()
 *            bytes (kvsel_window_score's plus the per-chunk row sums).
 * Returns KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED, KVSEL_EWORKSPACE or
 * KVSEL_ELAUNCH.  The workspace query returns 0 for invalid arguments.
 */
size_t kvsel_window_score_entropy_workspace(const kvsel_varlen* v, int32_t h_q, int32_t h_kv,
                                            int32_t d, int32_t w);
int kvsel_window_score_entropy(const kvsel_varlen* v, const void* q_win, const void* k,
                               int32_t h_q, int32_t h_kv, int32_t d, int32_t w, float scale,
                               float* score, float* lse, float* row_ent, float* mean_ent,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_accumulate_stats -- the StructKV part of step 2, and the head sum.
 *
 * StructKV summary page, section 2A: a global in-degree score adds each
 * token's attention contributions from the input layer to the pivot layer;
 * section 2B: per-layer attention entropy, sparsity and variance are
 * monitored to find the pivot.  FastKV section 2A: the propagated set is one
 * set per sequence, so its score is the sum over KV heads.
 *
 *   x[g, t]   = (c_in ? c_in[g, t] : 0) + score[g, t]
 *   c_out     = x                      (if non-NULL; may alias c_in)
 *   tok[t]    = sum_g x[g, t]          (if non-NULL; g ascending)
 *   stats[b]  = {entropy, sparsity, variance}   (if non-NULL)
 * where for sequence b (length n) and KV head g the window's attention
 * distribution is p_j = score[g, off_b + j] / (w * group) (its exact total,
 * since each of the w*group softmax rows sums to one), and
 *   entropy  = -sum_j p_j ln p_j,
 *   sparsity = #{ j : p_j < 1/n } / n   (decided exactly: score*n < w*group),
 *   variance = mean_j (p_j - 1/n)^2,
 * each averaged over the h_kv heads.  The stats use this layer's score, not
 * the accumulated x.
 *
 * Arguments
 *   score   device fp32 [h_kv, T];  c_in, c_out device fp32 [h_kv, T] or NULL;
 *   tok     device fp32 [T] or NULL; stats device fp32 [B, 3] or NULL.
 *   w, group  window length and query heads per KV head, both >= 1; every
 *           sequence holds the window (1 <= w <= n_b), as in the score call
 *           that made `score`.  A sequence shorter than w (n_b = 0
 *           included, which has no distribution) returns KVSEL_EINVAL.
 *   ws      device workspace of kvsel_accumulate_stats_workspace() bytes
 *           (needed only when stats != NULL).
 */
size_t kvsel_accumulate_stats_workspace(const kvsel_varlen* v, int32_t h_kv);
int kvsel_accumulate_stats(const kvsel_varlen* v, const float* score, int32_t h_kv,
                           int32_t w, int32_t group, const float* c_in, float* c_out,
                           float* tok, float* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_topk -- step 3: top-k plus the window, for one budget.
 *
 * FastKV summary page, section 2A: only the selected subset travels on,
 * together with the window tokens; section 2B: the TSP rate and the KV
 * retention rate are independent budgets (StructKV section 2C: R_struct and
 * R_KV), so the caller runs this once per budget (per-KV-head rows for the
 * cache, the head-sum row for the propagated sequence).
 *
 * For each row r and sequence b (length n, budget k_host[b]):
 * candidates are positions 0 .. n-w-1; the min(k, n-w) largest values are
 * kept, equal values going to the lower position; the kept positions are
 * written in ascending order, followed by the window n-w .. n-1.  Row r's
 * output for sequence b has min(n, k + w) entries and starts at
 * sum_{b' < b} min(n_b', k_b' + w).  The selection is exact on the fp32
 * values (-0 is treated as +0); NaN keys give an unspecified selection.
 *
 * Arguments
 *   keys    device fp32 [rows, T]; row stride T.
 *   rows    >= 1.
 *   w       window, 1 <= w <= every n_b.
 *   k_host  HOST int32 [B] budgets in tokens (window excluded), >= 0.
 *   idx     device int32 [rows, L], L = kvsel_selected_length(v, k_host, w).
 *   ws      device workspace of kvsel_topk_workspace(v, rows, w) bytes (it
 *           does not depend on the budgets).
 * Sequences longer than 8 * 2^20 + w return KVSEL_EUNSUPPORTED.
 */
size_t kvsel_topk_workspace(const kvsel_varlen* v, int32_t rows, int32_t w);
int kvsel_topk(const kvsel_varlen* v, const float* keys, int32_t rows, int32_t w,
               const int32_t* k_host, int32_t* idx, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_topk2 -- step 3 for both decoupled budgets in the same launches.
 *
 * FastKV summary page, section 2B (and StructKV section 2C): the KV
 * retention budget and the propagation budget are chosen independently
 * from the same scores, one per KV head and one on the head sum.  This call
 * is exactly kvsel_topk(v, keys_a, rows_a, w, k_a, idx_a, ...) followed by
 * kvsel_topk(v, keys_b, rows_b, w, k_b, idx_b, ...), with both selections'
 * latency chains in the same launches (one launch when every row is short
 * or the sequences many, two otherwise; the result does not depend on it).
 *
 * Arguments as for kvsel_topk, per set: keys_a device fp32 [rows_a, T],
 * k_a HOST int32 [B], idx_a device int32 [rows_a, L_a]; likewise for b.
 * rows_b may be 0 (then keys_b, k_b and idx_b are ignored).  w is shared.
 *   ws   device workspace of kvsel_topk2_workspace(v, rows_a, rows_b, w)
 *        bytes (it does not depend on the budgets).
 */
size_t kvsel_topk2_workspace(const kvsel_varlen* v, int32_t rows_a, int32_t rows_b, int32_t w);
int kvsel_topk2(const kvsel_varlen* v, int32_t w, const float* keys_a, int32_t rows_a,
                const int32_t* k_a, int32_t* idx_a, const float* keys_b, int32_t rows_b,
                const int32_t* k_b, int32_t* idx_b, void* ws, size_t ws_bytes, void* stream);

/*
 * kvsel_gather -- step 4: compact rows by the selected positions.
 *
 * FastKV summary page, section 2A/2B: the propagated tokens' hidden rows
 * form the shortened sequence for the later layers; the retained K/V
 * entries of each KV head form the compressed cache.  Pure copy, bit-exact.
 *
 *   dst[s, h, :] = src[off_b + idx[h or 0, s], h, :]
 * for every output row s of sequence b (the layout kvsel_topk writes).
 *
 * Arguments
 *   src        device [T, heads, row_bytes] bytes (e.g. bf16 K: heads=h_kv,
 *              row_bytes=2*d; hidden: heads=1, row_bytes=2*D).
 *   heads      >= 1.   row_bytes  > 0 and a multiple of 16.
 *   idx        device int32 [idx_rows, L]; idx_per_head = 1 uses row h for
 *              head h (idx_rows = heads), 0 uses row 0 for every head.
 *   k_host, w  the budgets and window the indices were selected with
 *              (they fix L and the per-sequence segments).
 *   dst        device [L, heads, row_bytes].
 * An index outside [0, n_b) leaves that output row zero-filled.
 */
int kvsel_gather(const kvsel_varlen* v, const void* src, int32_t heads, int32_t row_bytes,
                 const int32_t* idx, int32_t idx_per_head, const int32_t* k_host, int32_t w,
                 void* dst, void* stream);

/*
 * kvsel_gather_multi -- step 4 for several tensors in one launch.
 *
 * FastKV summary page, section 2B: the retained K and V entries share one
 * index set per KV head, and the propagated hidden rows use the other
 * budget's; this call does up to KVSEL_GATHER_MAX_JOBS such gathers over
 * the same packed batch in one launch (the work-groups are shared out in
 * proportion to each job's bytes).  Job j is exactly
 *   kvsel_gather(v, src, heads, row_bytes, idx, idx_per_head, k_host, w, dst)
 * with job j's fields.  Every pointer rule of kvsel_gather applies per job;
 * jobs must not write overlapping memory.
 */
#define KVSEL_GATHER_MAX_JOBS 4
typedef struct kvsel_gather_job {
  const void* src;            /* device [T, heads, row_bytes] */
  void* dst;                  /* device [L, heads, row_bytes] */
  const int32_t* idx;         /* device int32 [heads or 1, L] */
  const int32_t* k_host;      /* HOST int32 [B] budgets */
  int32_t heads;
  int32_t row_bytes;
  int32_t idx_per_head;
  int32_t reserved;           /* 0 */
} kvsel_gather_job;
int kvsel_gather_multi(const kvsel_varlen* v, int32_t w, int32_t n_jobs, const kvsel_gather_job* jobs,
                       void* stream);

/*
 * kvsel_gather_paged -- step 4 written straight into a paged KV cache.
 *
 * FastKV summary page, section 2B: the KV-retention budget decides what
 * the cache keeps for decoding.  A decode cache is usually held in
 * fixed-size blocks mapped per sequence by a block table; this call
 * writes the kept rows there directly instead of into a flat array.
 *
 * Job j is kvsel_gather_multi's job j (jobs[j].dst must be NULL) with the
 * destination pages[j]: selected row s (sequence-local, 0 <= s < L_b) of
 * sequence b, head h goes to
 *    cache[block_table[b * max_blocks + s / block_size], s % block_size, h, :]
 * cache      device [num_blocks, block_size, heads, row_bytes], 16-byte aligned.
 * block_table device int32 [B, max_blocks], 4-byte aligned; every sequence
 *            needs max_blocks * block_size >= L_b (else KVSEL_EINVAL).
 *            Entries are device data: a block number outside
 *            [0, num_blocks) (e.g. -1 for an unmapped block) makes the rows
 *            that map to it be skipped, never written out of bounds.
 * Slots no selected row maps to keep their contents.  An out-of-range
 * index gives a zero row, as in kvsel_gather.  Jobs must not write the
 * same cache slots.  Returns KVSEL_OK, KVSEL_EINVAL, KVSEL_EUNSUPPORTED or
 * KVSEL_ELAUNCH.
 */
typedef struct kvsel_paged_cache {
  void* cache;                /* device [num_blocks, block_size, heads, row_bytes] */
  const int32_t* block_table; /* device int32 [B, max_blocks] */
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_blocks;
  int32_t reserved;           /* 0 */
} kvsel_paged_cache;
int kvsel_gather_paged(const kvsel_varlen* v, int32_t w, int32_t n_jobs, const kvsel_gather_job* jobs,
                       const kvsel_paged_cache* pages, void* stream);

/*
 * kvsel_pivot_layer -- StructKV pivot pick (host, tiny).
 *
 * StructKV summary page, section 2B: the pivot is where attention entropy
 * drops sharply.  Returns the layer l >= 1 with the largest drop
 * entropy[l-1] - entropy[l] (the smallest such l on ties), 0 when layers is
 * 1, and -1 on invalid arguments (NULL, layers < 1, a non-finite value).
 * entropy is a HOST array read with the given element stride.
 */
int32_t kvsel_pivot_layer(const float* entropy, int32_t layers, int32_t stride);

/*
 * kvsel_pivot_layer_sparsity -- StructKV pivot pick with both signs of the
 * transition (host, tiny).
 *
 * StructKV summary page, section 2B: at the pivot the entropy falls sharply
 * and the sparsity rises.  Among the layers l >= 1 whose sparsity rose
 * (sparsity[l] > sparsity[l-1]), returns the one with the largest entropy
 * drop entropy[l-1] - entropy[l], the smallest such l on ties.  If no
 * layer's sparsity rose, returns kvsel_pivot_layer(entropy, ...).  0 when
 * layers is 1; -1 on invalid arguments (NULL, layers < 1, stride < 1, a
 * non-finite value).  Both arrays are HOST arrays read with the given
 * element stride (e.g. the entropy and sparsity columns of per-layer
 * kvsel_accumulate_stats results).
 */
int32_t kvsel_pivot_layer_sparsity(const float* entropy, const float* sparsity, int32_t layers,
                                   int32_t stride);

/*
 * kvsel_probe_read -- streaming-read probe (a measurement aid, not a step of
 * the selection path; no page defines it).
 *
 * Reads `heads` interleaved row sets of a device buffer: row r of head h is
 * the row_bytes bytes at src + r * stride_bytes + h * row_bytes, for r in
 * [0, rows).  wgs_per_head work-groups of 256 threads split each head's rows
 * into equal runs; each writes the XOR of what it read to out[h * wgs_per_head
 * + x] (device, uint32, heads * wgs_per_head entries), so no load can be
 * dropped.  Used to measure the reference rates the kernels are priced
 * against: a plain read (heads = 1, row_bytes = stride_bytes), a read in the
 * key cache's [T, h_kv, d] layout one head at a time (row_bytes = 2d,
 * stride_bytes = h_kv * 2d), and a re-read of a buffer small enough for the
 * last-level cache.
 *
 * src and out are device pointers, 16-byte aligned.  row_bytes is a power of
 * two >= 16; stride_bytes is a multiple of 16 and >= heads * row_bytes;
 * rows >= 1; 1 <= heads <= 65535; wgs_per_head >= 1.  Otherwise
 * KVSEL_EINVAL and nothing is enqueued.  Asynchronous on `stream`.
 */
int kvsel_probe_read(const void* src, int64_t rows, int32_t heads, int32_t row_bytes,
                     int64_t stride_bytes, int32_t wgs_per_head, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVSEL_H */
