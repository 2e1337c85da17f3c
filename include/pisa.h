/*
 * pisa.h -- C ABI of libpisa.so: PISA pyramid Top-K block selection and block-sparse attention
 * for AMD MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   "Block Sparse Attention with Log-Linear Complexity" (ai-papers-daily digest), section
 *   方法关键点 (method key points): keys are cut into leaf blocks of C tokens and mean-pooled upward
 *   with merge factor 2 into an O(log N) pyramid; each query walks coarse-to-fine from the root,
 *   scores at most g*K candidates per level, keeps the Top-K and expands only their children; leaf
 *   candidates are scored by the exact LogSumExp (LSE) over their raw keys, intermediate candidates
 *   by the LSE over their children's mean keys; the query heads that share a KV head share one
 *   selection, whose score is the sum of their per-head LSEs (section 工作参考价值, third bullet).
 *   Attention then runs over the selected leaf blocks only ("PISA：log-linear 复杂度的金字塔稀疏
 *   注意力" explainer, 核心方法 §7). The decode step keeps a cached mean pyramid, updates only the
 *   new token's ancestor path and runs every level in one kernel (digest, 工作参考价值 second
 *   bullet). bsa_select is the flat block selection of ordinary block-sparse attention that scores
 *   every (query, block) pair (digest, 动机).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers (HIP device memory), contiguous, 16-byte aligned.
 *     host_lens is a HOST pointer. `stream` is a hipStream_t (NULL = the default stream).
 *   - Layouts (head-major): Q and O are [B, Hq, N, d]; K and V are [B, Hkv, N, d]. Query heads
 *     r*G .. r*G+G-1 (G = Hq/Hkv) share KV head r. A "unit" is (b, r, i): one KV head at one
 *     query position; its G query heads share one selection.
 *   - Element type of Q, K, V, O is pisa_shape.dtype (IEEE fp32 or bfloat16). Pyramids and LSEs
 *     are fp32. Leaf indices are int32.
 *   - Causal: a node is eligible for query i iff its first token is <= i; leaf scores and
 *     attention mask tokens t > i.
 *   - Selections are ascending leaf indices padded with -1 to K. Top-K order is score descending,
 *     then node index ascending (ties go to the lower index).
 *   - Ownership: the caller allocates every buffer, including the workspace (sized by
 *     pisa_workspace_size). The library never allocates, frees or synchronises; every call only
 *     enqueues work on `stream` and returns. Inputs are read-only; outputs are fully overwritten.
 *   - Errors: a negative pisa_status. Arguments are validated before anything is enqueued, so an
 *     error leaves every output untouched. A failed launch returns PISA_EHIP. pisa_last_error()
 *     gives a thread-local message for the last non-OK return. Calls are reentrant.
 */
#ifndef PISA_H_
#define PISA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PISA_OK = 0,
  PISA_EINVAL = -1,       /* bad argument: null pointer, negative size, inconsistent shape */
  PISA_EUNSUPPORTED = -2, /* valid but not supported by these kernels (see pisa_shape limits) */
  PISA_EWORKSPACE = -3,   /* workspace missing or smaller than pisa_workspace_size() */
  PISA_EHIP = -4          /* a HIP launch failed */
} pisa_status;

typedef enum { PISA_FP32 = 0, PISA_BF16 = 1 } pisa_dtype;

/* Operation codes for pisa_workspace_size. */
enum { PISA_OP_SELECT = 1, PISA_OP_ATTN = 2, PISA_OP_DECODE = 3, PISA_OP_BSA = 4, PISA_OP_ATTN_BWD = 5, PISA_OP_TRACE = 6 };

/* Problem shape, passed by pointer to every call.
 * Limits of these kernels (PISA_EUNSUPPORTED otherwise): head_dim in {64, 128}; block C in
 * {32, 64}; 1 <= top_k <= 32; branch (merge factor g) == 2; causal == 1 (the walk's eligibility and
 * every score take the tokens t <= i of position i only); G = Hq/Hkv in {1, 2, 4, 8, 16};
 * q_tile in {1, 2, 4, 8, 16} with q_tile*G <= 16 (q_tile > 1 groups q_tile units that share a
 * candidate block into one matrix tile; q_tile == 1 walks each unit to its leaves directly);
 * units B*Hkv*seq_len < 2^27. */
typedef struct {
  int32_t batch;      /* B */
  int32_t seq_len;    /* N: tokens (prefill), or the cache capacity Nmax (decode)          */
  int32_t n_q_heads;  /* Hq                                                                */
  int32_t n_kv_heads; /* Hkv, divides Hq                                                   */
  int32_t head_dim;   /* d                                                                 */
  int32_t block;      /* C: tokens per leaf block                                          */
  int32_t top_k;      /* K: nodes kept per level                                           */
  int32_t branch;     /* g: merge factor of the pyramid                                    */
  int32_t causal;     /* 1: position i sees tokens t <= i (the only mode)                   */
  int32_t q_tile;     /* units per matrix tile in the leaf stage (see above)               */
  float scale;        /* score scale s; 0 means 1/sqrt(d)                                  */
  int32_t dtype;      /* pisa_dtype of Q, K, V, O                                          */
} pisa_shape;

/* Pyramid layout for a shape (host only, enqueues nothing; each output pointer may be NULL). Level l has n_l = ceil(n_{l-1}/2)
 * nodes, n_0 = ceil(seq_len / C), up to a single root; levels are stored leaf-first, so node
 * (l, j) of head (b, r) is row ((b*Hkv + r) * nodes_per_head + level_offset[l] + j) of a
 * [B*Hkv*nodes_per_head, d] fp32 array. n_levels counts the root. level_offset has room for 32
 * entries. */
pisa_status pisa_pyramid_layout(const pisa_shape* shape, int32_t* n_levels, int64_t* level_offset,
                                int64_t* nodes_per_head);

/* Workspace bytes needed by an operation (host only). 0 is a valid answer. */
pisa_status pisa_workspace_size(const pisa_shape* shape, int32_t op, size_t* bytes);

/* Mean-pooled key pyramid (digest 方法关键点, pyramid bullet; explainer 核心方法 §1).
 *   k         [B, Hkv, N, d] keys (dtype).
 *   host_lens NULL: every sequence holds N tokens. Else a host array of B lengths (0 <= len <= N,
 *             B <= 256): tokens at positions >= len are ignored (a decode cache holding len tokens).
 *   pyr_mean  out, fp32 pyramid (pisa_pyramid_layout): node mean = mean of the keys present in the
 *             node's span; nodes holding no token get 0.
 *   pyr_sum   out, nullable, same layout: per-node key sums, needed by pisa_decode_step. */
pisa_status pisa_build_pyramid(const pisa_shape* shape, const void* k, const int32_t* host_lens, float* pyr_mean,
                               float* pyr_sum, void* stream);

/* Pyramid Top-K selection with LSE scoring (digest 方法关键点, pyramid / scoring / complexity
 * bullets; abstract). For each unit (b, r, i): walk from the root; at level l the candidates are the
 * eligible children of the nodes kept at level l+1; a level with more than K candidates scores each
 * candidate c as sum over the group's heads h of LSE over c's eligible children c' of
 * s * q_{h,i} . mean(c') (levels >= 1), or of s * q_{h,i} . k_t over the leaf's tokens t <= i (leaf
 * level), and keeps the Top-K; a level with at most K candidates keeps them all.
 *   q        [B, Hq, N, d]; k [B, Hkv, N, d]; pyr_mean from pisa_build_pyramid (host_lens NULL).
 *   sel      out int32 [B, Hkv, N, K]: selected leaves, ascending, -1 padded.
 *   sel_lse  out, nullable, fp32 [B, Hq, N, K]: per-head leaf LSE of each selected leaf
 *            (-inf where sel is -1).
 *   ws       workspace of at least pisa_workspace_size(shape, PISA_OP_SELECT) bytes. */
pisa_status pisa_select(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean, int32_t* sel,
                        float* sel_lse, void* ws, size_t ws_bytes, void* stream);

/* pisa_select for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, kernels and results as pisa_select,
 * but the workspace is a scratch array of pisa_select_noalloc_max_bytes() bytes (64 MiB) that the
 * library holds in every GPU's memory from its first use on that GPU until the process ends; the call
 * itself allocates and frees nothing. The scratch of the current device (hipGetDevice) is used, so
 * `stream` must belong to that device. Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (other streams, other threads) race and give undefined results; calls on
 * one stream are ordered and safe. Returns PISA_EUNSUPPORTED, before anything is enqueued, when
 * pisa_workspace_size(shape, PISA_OP_SELECT) exceeds the scratch (for example 64K tokens x 8 KV heads
 * with K = 16; 16K tokens x 2 KV heads with 16 query heads fits). */
pisa_status pisa_select_noalloc(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean,
                                int32_t* sel, float* sel_lse, void* stream);
size_t pisa_select_noalloc_max_bytes(void);

/* The traceable selection path (explainer 亮点 5: which nodes the walk kept at every level can be read
 * back): pisa_select's walk for a list of units, returning the kept nodes of every level, so that a
 * unit's whole path can be inspected or checked level by level against another implementation. It
 * runs the one-unit-per-wave walk and leaf stage of pisa_select with q_tile 1 (shape->q_tile is ignored;
 * pisa_select gives the same selection at every q_tile), so its kept sets are pisa_select's.
 *   units    int64 [n_units]: unit indices u = (b * Hkv + r) * N + i, in any order, repeats allowed; an
 *            index outside [0, B * Hkv * N) gives rows of -1 (it is not an error).
 *   trace    out int32 [n_units, n_levels, K] (n_levels from pisa_pyramid_layout): row (t, l) holds the
 *            nodes of level l kept for unit units[t], ascending, -1 padded; a level with at most K
 *            eligible nodes (every level above the walk's first scored one) lists all of them; row
 *            (t, 0), the leaves, equals the unit's row of pisa_select's sel.
 *   ws       workspace of at least pisa_workspace_size(shape, PISA_OP_TRACE) bytes (the bf16 routing
 *            planes; none for fp32).
 * n_units = 0 enqueues nothing (units and trace may then be NULL); n_units < 0 is PISA_EINVAL. */
pisa_status pisa_select_trace(const pisa_shape* shape, const void* q, const void* k, const float* pyr_mean,
                              const int64_t* units, int64_t n_units, int32_t* trace, void* ws, size_t ws_bytes,
                              void* stream);

/* pisa_sparse_attn and pisa_sparse_attn_backward process the batch in chunks of consecutive (sequence,
 * KV head) slices, the fewest whose workspace fits 16 GiB (at least one slice each), so their
 * pisa_workspace_size is that of one chunk, not of the whole batch. The environment variable
 * PISA_ATTN_CHUNK_MIB, if set to a smaller positive number of MiB, lowers the budget; it is read at every
 * call, so keep it unchanged between the workspace query and the call. Results do not depend on the
 * chunking. */

/* Block-sparse attention over the selected leaves (explainer 核心方法 §7, last step). For each
 * (b, h, i): O = sum over t in T of softmax_t(s * q_{h,i} . k_t) v_t, T = the tokens t <= i of the
 * leaves in sel[b, h/G, i, :]; the softmax normalises over T only.
 *   sel      int32 [B, Hkv, N, K] as written by pisa_select (or bsa_select): each row ascending
 *            leaves j with j*C <= i, -1 padded, at least one entry.
 *   o        out [B, Hq, N, d] (dtype). o_lse out, nullable, fp32 [B, Hq, N]: LSE over T. */
pisa_status pisa_sparse_attn(const pisa_shape* shape, const void* q, const void* k, const void* v, const int32_t* sel,
                             void* o, float* o_lse, void* ws, size_t ws_bytes, void* stream);

/* Backward of pisa_sparse_attn (digest 工作参考价值 fourth bullet: the gradients pass only through the
 * selected attention; the selection itself gets no gradient). For each (b, h, i) with T = the tokens
 * t <= i of the leaves in sel[b, h/G, i, :], p_t = exp(s q . k_t - o_lse), dp_t = dO . v_t,
 * D = dO . o, ds_t = p_t (dp_t - D):
 *   d_q[b, h, i] = s sum_t ds_t k_t;  d_k[b, r, t] = s sum ds_t q;  d_v[b, r, t] = sum p_t dO
 * (the last two summed over every query head of KV head r and every query that attends t).
 *   sel, o, o_lse: the selection and the outputs of the forward call (o_lse is required here).
 *   d_o [B, Hq, N, d]: the gradient of o. d_q [B, Hq, N, d], d_k and d_v [B, Hkv, N, d]: out.
 *   bfloat16 inputs and outputs only (fp32 accumulation); PISA_EUNSUPPORTED for fp32.
 *   ws: pisa_workspace_size(shape, PISA_OP_ATTN_BWD) bytes. d_k and d_v add the pairs of a leaf in the
 *   order in which the pairs were bucketed (by atomic counters), so their last bits may differ from run
 *   to run. */
pisa_status pisa_sparse_attn_backward(const pisa_shape* shape, const void* q, const void* k, const void* v,
                                      const int32_t* sel, const void* o, const float* o_lse, const void* d_o,
                                      void* d_q, void* d_k, void* d_v, void* ws, size_t ws_bytes, void* stream);

/* One fused decode step (digest 工作参考价值 second bullet; 方法关键点 Kernel bullet). For every
 * sequence b with p = host_lens[b] tokens cached (shape.seq_len = capacity Nmax, p < Nmax): append
 * k_new/v_new at position p; add k_new to the sum of each ancestor of leaf p/C in pyr_sum and
 * refresh those nodes' means in pyr_mean; then run the pisa_select walk and pisa_sparse_attn for
 * query position i = p over the p+1 cached tokens. One kernel launch does all of it. The caller
 * advances host_lens afterwards.
 *   q_new [B, Hq, d]; k_new, v_new [B, Hkv, d]; k_cache, v_cache [B, Hkv, Nmax, d] (updated);
 *   pyr_sum, pyr_mean: the decode pyramid (layout of shape), initialised by pisa_build_pyramid with
 *   pyr_sum set and host_lens = the cached lengths; o out [B, Hq, d]; sel_out out, nullable, int32
 *   [B, Hkv, K].
 *   ws: pisa_workspace_size(shape, PISA_OP_DECODE) bytes, 16-byte aligned, all zero before its first
 *   decode step (for example from hipMemset once). It holds per-unit arrival counters that every step
 *   leaves at zero again, so one zeroed workspace serves every later step of the same shape; other
 *   calls must not write it in between, and steps that share it must not overlap in time (one
 *   workspace per stream). PISA_EWORKSPACE when it is missing or too small. */
pisa_status pisa_decode_step(const pisa_shape* shape, const int32_t* host_lens, const void* q_new, const void* k_new,
                             const void* v_new, void* k_cache, void* v_cache, float* pyr_sum, float* pyr_mean, void* o,
                             int32_t* sel_out, void* ws, size_t ws_bytes, void* stream);

/* Flat block selection of ordinary block-sparse attention, for comparison (digest 动机: every
 * (query, key block) pair is scored, O(N^2/C)). Per unit, each eligible leaf j gets
 * B(j) = sum over the group's heads of s * q_{h,i} . mean(leaf j), and the Top-K leaves are kept.
 * The leaf means are pooled inside the call (in the workspace).
 *   sel out int32 [B, Hkv, N, K] ascending, -1 padded. */
pisa_status bsa_select(const pisa_shape* shape, const void* q, const void* k, int32_t* sel, void* ws, size_t ws_bytes,
                       void* stream);

/* Selection quality (digest 关键实验: block selections are compared by Recall@K and by the attention
 * mass ratio). A dense causal pass that scores every leaf, not a bounded candidate set, at chosen
 * query positions, and the measures computed from it.
 *
 * pisa_flat_leaf_lse: for every (b, query head h, position index x) with i = positions[x]:
 *   leaf_lse out fp32 [B, Hq, n_pos, n0] (n0 = ceil(N / C)): per leaf j, the exact LSE over the leaf's
 *            tokens t <= i of s * q_{h,i} . k_t, -inf for leaves after i (the same per-leaf arithmetic
 *            as pisa_select's leaf stage);
 *   row_lse  out fp32 [B, Hq, n_pos]: the LSE of the whole causal row (every t <= i).
 *   positions: device int32 [n_pos], each in [0, N); a position outside gives NaN rows.
 * Work is O(n_pos * i * d * Hq) MFMA flops: use it on samples of positions at long N.
 *
 * pisa_selection_quality: per unit (b, r, x), from the outputs of pisa_flat_leaf_lse:
 *   flat_sel out int32 [B, Hkv, n_pos, K]: the flat exact Top-K, the K eligible leaves with the largest
 *            head-summed leaf LSE (score descending, then lower index), ascending, -1 padded;
 *   recall   out fp32 [B, Hkv, n_pos]: |sel[b, r, i] & flat_sel| / min(K, eligible leaves);
 *   mass     out fp32 [B, Hq, n_pos]: per head, sum over the leaves j of sel[b, r, i] of
 *            exp(leaf_lse[j] - row_lse), the share of full causal attention's softmax mass inside the
 *            selected blocks.
 *   sel: int32 [B, Hkv, N, K] as written by pisa_select or bsa_select. At most 16384 leaves. */
pisa_status pisa_flat_leaf_lse(const pisa_shape* shape, const void* q, const void* k, const int32_t* positions,
                               int32_t n_pos, float* leaf_lse, float* row_lse, void* stream);
pisa_status pisa_selection_quality(const pisa_shape* shape, const float* leaf_lse, const float* row_lse,
                                   const int32_t* positions, int32_t n_pos, const int32_t* sel, int32_t* flat_sel,
                                   float* recall, float* mass, void* stream);

/* Selection variants: the ablations and options that the pages name beside the method. Not the fast
 * path: the walk scores node summaries with fp32 dot products, one wave per unit, to measure how the
 * options change the selection.
 *
 * pisa_build_pyramid_pooled: a pyramid (pisa_pyramid_layout) whose node summary is the mean, the sum or
 * the element-wise max of the raw keys in the node's span (explainer 核心方法 §1: mean, sum or max
 * pooling). variance, nullable (mean or sum pooling only): the per-dimension population variance of
 * those keys, in the same layout.
 *
 * pisa_select_variant: the pisa_select walk with these options (sel out int32 [B, Hkv, N, K]):
 *   score  PISA_SCORE_LSE: LSE over the eligible children's summaries, exact LSE over raw keys at the
 *          leaves (the method; with mean pooling and the fixed budget, the selection pisa_select makes);
 *          PISA_SCORE_MEAN: s * q . the node's own summary (digest 方法关键点, scoring bullet: the
 *          PISA-1 ablation); PISA_SCORE_MEAN_VAR: that plus (s^2 / 2) * sum_d q_d^2 var_d (PISA-2: mean
 *          plus variance; needs variance); heads summed at every level.
 *   budget PISA_BUDGET_FIXED: K nodes kept at every level; PISA_BUDGET_HALVING: K_l = min(n_l, K 2^l),
 *          half as many at each finer level (explainer 核心方法 §7 and 工程落地), K leaves in the end.
 *   max_level  -1: the walk starts at the root; else it starts from every eligible node of level
 *          min(max_level, root) (a truncated pool chain, explainer 工程落地 ⑥).
 * Candidate lists are held in on-chip memory: the starting level and twice the kept nodes of every level
 * must not exceed 2048 nodes (PISA_EUNSUPPORTED otherwise). summary/variance come from
 * pisa_build_pyramid_pooled (or pisa_build_pyramid, which is mean pooling). */
typedef enum { PISA_POOL_MEAN = 0, PISA_POOL_SUM = 1, PISA_POOL_MAX = 2 } pisa_pool;
typedef enum { PISA_SCORE_LSE = 0, PISA_SCORE_MEAN = 1, PISA_SCORE_MEAN_VAR = 2 } pisa_score;
typedef enum { PISA_BUDGET_FIXED = 0, PISA_BUDGET_HALVING = 1 } pisa_budget;
typedef struct {
  int32_t score;     /* pisa_score */
  int32_t budget;    /* pisa_budget */
  int32_t max_level; /* -1, or the highest pyramid level the walk starts from */
} pisa_variant;
pisa_status pisa_build_pyramid_pooled(const pisa_shape* shape, const void* k, int32_t pool, float* summary,
                                      float* variance, void* stream);
pisa_status pisa_select_variant(const pisa_shape* shape, const pisa_variant* variant, const void* q, const void* k,
                                const float* summary, const float* variance, int32_t* sel, void* stream);

/* A message for a status value (any int; values that are not a pisa_status get a generic message). */
const char* pisa_status_string(int32_t status);
const char* pisa_last_error(void);

/* Stage timing for profiling, off by default. While enabled (per calling thread), every call
 * records a pair of HIP events on its stream around each of its kernel launches (a launcher that
 * issues several small kernels, such as the regroup, is one stage). pisa_stage_times() waits for
 * the recorded events, adds each stage's elapsed time to a per-name total and count, forgets the
 * events and writes up to `cap` entries: names (NUL-terminated, at most 31 characters),
 * total milliseconds and launch counts. It returns the number of distinct stage names (which may
 * exceed cap), or a negative pisa_status (PISA_EINVAL for cap < 0). pisa_stage_timing(0) also discards the totals. Event
 * creation happens here, so do not enable it under stream capture. */
pisa_status pisa_stage_timing(int32_t enable);
int32_t pisa_stage_times(char (*names)[32], double* total_ms, int32_t* count, int32_t cap);

#ifdef __cplusplus
}
#endif
#endif /* PISA_H_ */
