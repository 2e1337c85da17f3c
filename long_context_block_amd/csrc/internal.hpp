// Internal launcher declarations shared by the C ABI (api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace pisa {

constexpr int kMaxLensBatch = 256;

// Per-sequence token counts, passed by value in the kernel arguments.
struct LensArg {
  int has;  // 0: every sequence holds N tokens
  int hkv;  // KV heads (to map a (b, r) row to b)
  int len[kMaxLensBatch];
};

struct PyrDims {
  int BH;  // B * Hkv
  int N;   // tokens per sequence (or capacity)
  int C;
  int D;
  Levels lv;
};

struct SelDims {
  int B, Hq, Hkv, G, N, D, C, K, q_tile;
  int chunk_log2;  // pairs are bucketed per position chunk of 2^chunk_log2 units (>= 10)
  float scale;
  bool bf16;
  Levels lv;
};

hipError_t launch_pool(const void* k, bool bf16, const PyrDims& pd, LensArg lens, int max_level, float* mean,
                       float* sum, hipStream_t st);
hipError_t launch_split_hilo(const float* mean, long long rows, int D, uint16_t* hilo, hipStream_t st);

// Selection. `nodes` is the bf16 hi/lo pyramid (bf16 inputs) or the fp32 means (fp32 inputs).
hipError_t launch_route(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                        const int* hexp, bool fused, int* kept, int* sel, float* sel_lse, hipStream_t st);
// The walk of launch_route (fused) for a list of units, writing every level's kept nodes to trace
// [n_units, n_levels, K] (level 0: the selection); a unit index outside [0, U) gives rows of -1.
hipError_t launch_route_trace(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                              const int* hexp, const long long* units, long long n_units, int* trace,
                              hipStream_t st);
// Routing with 16 / G units per wave (bf16 inputs, G in {4, 8, 16}, K <= 32); same kept sets as
// launch_route. Writes the kept level-1 nodes [U, K].
bool route_group_supported(const SelDims& sd);
hipError_t launch_route_group(const SelDims& sd, const void* q, const void* hilo, const float* norms, const int* hexp,
                              int* kept, hipStream_t st);
// Routing planes of a bf16 pyramid: per KV head an exponent hexp (max |mean| 2^hexp in [2^14, 2^15)),
// per row the fp16 hi/lo planes of 2^hexp mean and the hi-plane score bound (unscaled units).
// part_max: 64 floats of scratch per KV head.
hipError_t launch_route_planes(const float* mean, long long heads, const Levels& lv, int D, float* part_max,
                               int* hexp, uint16_t* hilo, float* bound, hipStream_t st);

// Bucket (unit, slot) pairs by node: node lists [U, K] (-1 = none) -> pairs sorted by
// (b*Hkv + r, node), packed as (unit << 5) | slot. counts/offsets have n_buckets (+1) entries. With
// ranks_to_positions, ranks[u * K + slot] ends as the pair's index in the sorted list.
hipError_t launch_regroup(const int* nodes, long long U, int K, int N, int buckets_per_head, int n_heads,
                          int chunk_log2, int* counts, int* offsets, int* ranks, bool ranks_to_positions,
                          uint32_t* pairs, hipStream_t st);

hipError_t launch_leaf_lse(const SelDims& sd, const void* q, const void* k, const int* kept, const uint32_t* pairs,
                           const int* total, float* leaf_lse, hipStream_t st);
hipError_t launch_finalize(const SelDims& sd, const int* kept, const float* leaf_lse, int* sel, float* sel_lse,
                           hipStream_t st);

// Attention over selected leaves. The partial rows of sorted pair x are part[(x G + h) D ..] and
// part_lse[x G + h]; pos[u K + slot] is the sorted index of the pair (u, slot).
hipError_t launch_attn_leaf(const SelDims& sd, const void* q, const void* k, const void* v, const int* sel,
                            const uint32_t* pairs, const int* total, void* part, float* part_lse, hipStream_t st);
hipError_t launch_attn_merge(const SelDims& sd, const int* sel, const int* pos, const void* part,
                             const float* part_lse, void* o, float* o_lse, hipStream_t st);

// Backward of the sparse attention (bf16): pairs/total/pos/offsets from launch_regroup over sel (to
// positions); dsum [B Hq N], dk_acc and dv_acc = dk_acc + B Hkv N D (fp32 accumulators), kv_part
// attn_backward_kv_part_bytes(sd) of per-task dK/dV slots, part [pairs, G, D] (bf16).
hipError_t launch_attn_backward(const SelDims& sd, const void* q, const void* k, const void* v, const int* sel,
                                const void* o, const float* o_lse, const void* d_o, const uint32_t* pairs,
                                const int* total, const int* pos, const int* offsets, float* dsum, float* dk_acc,
                                float* dv_acc, float* kv_part, void* part, void* d_q, void* d_k, void* d_v,
                                hipStream_t st);
size_t attn_backward_kv_part_bytes(const SelDims& sd);

// Flat block selection.
hipError_t launch_bsa(const SelDims& sd, const void* q, const float* leaf_mean, const uint16_t* leaf_hilo, int* sel,
                      hipStream_t st);

// Selection quality: every leaf's exact per-head LSE and each row's LSE at the given positions, then
// per unit the flat exact Top-K, the recall of `sel` against it and its share of the softmax mass.
hipError_t launch_flat_leaf_lse(const SelDims& sd, const void* q, const void* k, const int* pos, int n_pos,
                                float* leaf_lse, float* row_lse, hipStream_t st);
hipError_t launch_quality(const SelDims& sd, const float* leaf_lse, const float* row_lse, const int* pos, int n_pos,
                          const int* sel, int* flat_sel, float* recall, float* mass, hipStream_t st);

// Selection variants: a pyramid of pooled summaries (pool 0 mean, 1 sum, 2 max; variance nullable),
// and the walk under a scoring rule (0 LSE, 1 mean, 2 mean + variance), a budget (0 fixed, 1 halving)
// from the starting level `start` (at most the root). Candidate lists live in LDS: at most
// kVariantLdsCand candidates per level.
constexpr int kVariantLdsCand = 2048;
hipError_t launch_pool_pooled(const void* k, bool bf16, const PyrDims& pd, int pool, float* summary, float* variance,
                              hipStream_t st);
hipError_t launch_variant(const SelDims& sd, int score, int budget, int start, const void* q, const void* k,
                          const float* summary, const float* variance, int* sel, hipStream_t st);

// Decode step.
struct DecodeArgs {
  int B, Hq, Hkv, G, Nmax, D, C, K;
  float scale;
  bool bf16;
  Levels lv;
  LensArg lens;
  int* ticket;      // [B*Hkv] arrival counters, zero before the step (the step leaves them zero)
  float* part_o;    // [B*Hkv, 2K, G, D]
  float* part_lse;  // [B*Hkv, 2K, G]
};
// Work-groups per decode unit for top-k K (the candidate leaves, 2K, one per wave).
int decode_splits(int K);
hipError_t launch_decode(const DecodeArgs& da, const void* q_new, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, float* pyr_sum, float* pyr_mean, void* o, int* sel_out, hipStream_t st);

}  // namespace pisa
