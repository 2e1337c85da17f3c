// Pyramid Top-K selection with LogSumExp scoring.
//
// "Block Sparse Attention with Log-Linear Complexity" digest, 方法关键点:
//   pyramid bullet  -- the walk starts at the coarsest level with one candidate, scores the bounded
//                      candidate set of each level, keeps the Top-K and expands only their children;
//   scoring bullet  -- leaves by the exact LSE over their raw keys, intermediate nodes by the LSE over
//                      their children's mean keys;
//   complexity      -- at most g*K candidates per query per level;
//   Kernel bullet   -- prefill in two stages: intermediate-level routing without materialising QK,
//                      then queries that share a leaf key block are grouped into tiles so the key
//                      tile is loaded once (Qtile); GQA heads of one KV head share the selection.
//
// route_kernel: one wave per unit (b, r, i). The G query heads are the 16 matrix columns (zero past
// G). At a scored level the <= 2K candidates' <= 4K children are the matrix rows; their fp32 means
// enter as bf16 hi + lo planes (two MFMA passes, since q is exact in bf16) or as fp32 (fp32 MFMA).
// Each lane then holds both children of two candidates for one head, so the per-head LSE over the
// children is lane-local; a 16-lane butterfly sums the heads. Top-K is a rank count over the
// candidate lanes (score desc, index asc) followed by a stable lane compaction.
//
// With q_tile == 1 the wave goes on to the leaves itself (the unit-major leaf stage). With
// q_tile > 1 it writes its kept level-1 nodes; regroup buckets the (unit, kept node) pairs by node;
// leaf_lse_kernel loads each bucket's 2C x d key tile into registers once and runs tiles of q_tile
// units x G heads against it; finalize_kernel does the leaf Top-K. Both leaf paths run the same
// per-column arithmetic and sum the heads in the same order, so their outputs agree bit for bit.
#include "common.hpp"
#include "internal.hpp"
#include "pair_runs.hpp"
#include "walk_tiles.hpp"

namespace pisa {

template <typename T>
struct RouteParams {
  const T* q;
  const T* k;
  const void* nodes;
  const float* norms;  // hi-plane score bound per pyramid row (bf16 inputs)
  const int* hexp;     // per KV head: the routing planes hold 2^hexp mean (bf16 inputs)
  int B, Hq, Hkv, G, N, K, upw;
  float scale;
  Levels lv;
  int* kept;      // [U, K] (tiled path)
  int* sel;       // [U, K] (fused path)
  float* sel_lse; // [B, Hq, N, K] or null (fused path)
  // traced walk: the units to walk, and per unit and level its kept nodes [n_units, n_levels, K]
  const long long* units;
  long long n_units;
  int* trace;
};

// Top-K of the leaf candidates and the outputs. Lane c < n_cand is candidate c = 2*slot + bit
// (leaf 2*kept[slot] + bit); ell(c, h) gives its per-head LSE. The heads are summed in index order.
// sc: this lane's head-summed score (used when n_cand > K).
template <typename F>
__device__ __forceinline__ void leaf_topk_write_sc(int n_cand, int leaf_c, float sc, int G, int K, long long u,
                                                   long long qrow0, long long qstride, F ell, int* sel,
                                                   float* sel_lse, uint32_t* keys) {
  const int lane = lane_id();
  bool keep = lane < n_cand;
  if (n_cand > K) keep = topk_keep(sc, n_cand, K, keys);
  int nsel;
  const int leaf_sel = compact_lanes(keep, leaf_c, &nsel);
  const int c_sel = compact_lanes(keep, lane, &nsel);
  if (lane < K) {
    sel[u * K + lane] = lane < nsel ? leaf_sel : -1;
    if (sel_lse) {
      for (int h = 0; h < G; ++h) sel_lse[(qrow0 + h * qstride) * K + lane] = lane < nsel ? ell(c_sel, h) : kNegInf;
    }
  }
}

template <typename F>
__device__ __forceinline__ void leaf_topk_write(int n_cand, int leaf_c, int G, int K, long long u, long long qrow0,
                                                long long qstride, F ell, int* sel, float* sel_lse, uint32_t* keys) {
  float sc = 0.f;
  if (n_cand > K && lane_id() < n_cand)
    for (int h = 0; h < G; ++h) sc += ell(lane_id(), h);
  leaf_topk_write_sc(n_cand, leaf_c, sc, G, K, u, qrow0, qstride, ell, sel, sel_lse, keys);
}

// TRACE (with FUSED): the units come from p.units, and every level's kept nodes, the leaves' included,
// go to p.trace instead of sel; the arithmetic is the same.
template <typename T, int D, int C, bool FUSED, int KM, bool TRACE = false>
__global__ __launch_bounds__(256, FUSED ? 2 : 4) void route_kernel(RouteParams<T> p) {
  static_assert(!TRACE || FUSED, "the traced walk includes the leaf stage");
  constexpr int kLog2C = C == 64 ? 6 : 5;
  __shared__ float s_ell[FUSED ? 4 : 1][64][17];
  __shared__ __align__(16) float s_sc[4][64];
  __shared__ __align__(16) uint32_t s_key[4][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long U = (long long)p.B * p.Hkv * p.N;
  const int lb = xcd_logical_block(gridDim.x);
  const long long first = ((long long)lb * 4 + wave) * p.upw;
  for (int it = 0; it < p.upw; ++it) {
    long long u = first + it;
    long long trow = 0;  // TRACE: this unit's first trace row (level 0)
    if constexpr (TRACE) {
      if (u >= p.n_units) break;
      trow = u * p.lv.n_levels;
      u = p.units[u];
      if (u < 0 || u >= U) {  // not a unit of this shape: every level reads -1
        for (int x = lane; x < p.lv.n_levels * p.K; x += 64) p.trace[trow * p.K + x] = -1;
        continue;
      }
    } else {
      if (u >= U) break;
    }
    const long long bh = u / p.N;
    const long long i = u % p.N;
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    Frag<T> qf[D / 32];
    const bool hv = r16 < p.G;
    const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
    const T* qrow = p.q + (qrow0 + (long long)(hv ? r16 : 0) * p.N) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (hv)
        qf[s].load(qrow + 32 * s);
      else
        qf[s].zero();
    }
    int kept;
    int nk;
    auto trace_hook = [&](int l, int kept_l, int nk_l) {
      if constexpr (TRACE) {
        if (lane < p.K) p.trace[(trow + l) * p.K + lane] = lane < nk_l ? kept_l : -1;
      }
    };
    if constexpr (sizeof(T) == 2) {
      RoutePlanes<D> rows;
      rows.base = (const uint16_t*)p.nodes + bh * p.lv.rnodes * 2 * D;
      // sum over the group's heads of |q_h| (lane r16 = head holds its d/4 elements per lane group)
      float sq = 0.f;
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = qf[s].get(e);
          sq += x * x;
        }
      const float sq_all = colgroup_sum(sq);  // every lane takes part in the exchange
      const float qn = row_sum16(hv ? sqrtf(sq_all) : 0.f);
      const float* norms = p.norms + bh * p.lv.rnodes;
      Frag<uint16_t> qh[D / 32];
      const int te = route_q_f16<D>(qf, qh);
      const float col_scale = ldexpf(p.scale, -(te + p.hexp[bh]));
      nk = walk_to_level1<T, D, KM>(
          p.lv, kLog2C, p.K, (int)i, &kept,
          [&](int lc, int cn, int n_cand, int e_child) {
            return select_level_refine<D, KM>(rows, norms, (int)p.lv.roff[lc], qh, qn, cn, n_cand, e_child, p.G,
                                              p.scale, col_scale, p.K, s_sc[wave], s_key[wave]);
          },
          trace_hook);
    } else {
      NodeRows<T, D> rows;
      rows.base = (const float*)p.nodes + bh * p.lv.nodes * D;
      nk = walk_to_level1<T, D, KM>(
          p.lv, kLog2C, p.K, (int)i, &kept,
          [&](int lc, int cn, int n_cand, int e_child) {
            score_candidates<T, D, KM>(rows, (int)p.lv.off[lc], qf, cn, n_cand, e_child, p.G, p.scale, s_sc[wave]);
            return topk_keep_lds(s_sc[wave], n_cand, p.K, s_key[wave]);
          },
          trace_hook);
    }
    if constexpr (!FUSED) {
      if (lane < p.K) p.kept[u * p.K + lane] = lane < nk ? kept : -1;
    } else {
      int n_cand = 2 * nk;
      {
        const int lastp = readlane(kept, nk - 1);
        if ((2LL * lastp + 1) * C > i) --n_cand;
      }
      const int par = __shfl(kept, lane >> 1);
      const int leaf_c = 2 * par + (lane & 1);
      if (n_cand > p.K || p.sel_lse) {
        const T* kbh = p.k + bh * (long long)p.N * D;
        for (int slot = 0; slot < nk; ++slot) {
          const long long pn = readlane(kept, slot);
          Frag<T> kf[C / 8][D / 32];
          load_leaf_pair<T, D, C>(kbh, 2 * pn * C, p.N, kf);
          float l0, l1;
          leaf_pair_lse<T, D, C>(kf, qf, 2 * pn * C, i, p.scale, l0, l1);
          if (grp == 0 && hv) {
            s_ell[FUSED ? wave : 0][2 * slot][r16] = l0;
            s_ell[FUSED ? wave : 0][2 * slot + 1][r16] = l1;
          }
        }
        __threadfence_block();
      }
      leaf_topk_write(
          n_cand, leaf_c, p.G, p.K, TRACE ? trow : u, qrow0, p.N,
          [&](int c, int h) { return s_ell[FUSED ? wave : 0][c][h]; }, TRACE ? p.trace : p.sel,
          TRACE ? nullptr : p.sel_lse, s_key[wave]);
      __threadfence_block();
    }
  }
}

// bf16 routing with the upper pyramid levels in LDS. One work-group of 16 waves per CU and KV head
// slice: the hi plane of pyramid rows [lds_first, nodes) of KV head bh (<= kRouteLdsBytes) is staged
// into LDS once, then the waves walk units of that head (groups of kRouteUnits consecutive positions,
// spread round-robin over the head's work-groups). Child rows of those levels are read from LDS; the
// two largest levels and all lo rows come from global memory (L2). Same arithmetic as route_kernel.
constexpr int kRouteLdsBytes = 128 * 1024;
constexpr int kRouteUnits = 4;

// waves per work-group: 16 for up to 4 candidate tiles, 8 (256 registers each) for 8 tiles (K > 16), so that
// the larger walk state does not spill
template <int KM>
constexpr int route_lds_waves() {
  return KM <= 4 ? 16 : 8;
}

template <int D, int C, int KM>
__global__ __launch_bounds__(route_lds_waves<KM>() * 64) void route_lds_kernel(RouteParams<uint16_t> p, int lds_first,
                                                                                int wg_per_head) {
  constexpr int kLog2C = C == 64 ? 6 : 5;
  constexpr int NW = route_lds_waves<KM>();
  __shared__ __align__(16) uint16_t s_hi[kRouteLdsBytes / 2];
  __shared__ float s_bound[kRouteLdsBytes / 128];  // one per staged row (rows of >= 64 values)
  __shared__ __align__(16) float s_sc[NW][64];
  __shared__ __align__(16) uint32_t s_key[NW][64];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH, w = blockIdx.x / BH;  // consecutive work-groups: different heads
  LdsHiRows<D> rows;
  rows.base = (const uint16_t*)p.nodes + (long long)bh * p.lv.rnodes * 2 * D;
  const float* norms = p.norms + (long long)bh * p.lv.rnodes;
  rows.lds = s_hi;
  rows.lds_bound = s_bound;
  rows.first = lds_first;
  stage_hi_rows<D>(rows.base, norms, lds_first, (int)(p.lv.rnodes - lds_first), s_hi, s_bound);
  __syncthreads();
  const int hexp = p.hexp[bh];
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const bool hv = r16 < p.G;
  const int groups = (p.N + kRouteUnits - 1) / kRouteUnits;
  for (int gi = w * NW + wave; gi < groups; gi += wg_per_head * NW) {
    for (int it = 0; it < kRouteUnits; ++it) {
      const int i = gi * kRouteUnits + it;
      if (i >= p.N) break;
      const long long u = (long long)bh * p.N + i;
      Frag<uint16_t> qf[D / 32];
      const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
      const uint16_t* qrow = p.q + (qrow0 + (long long)(hv ? r16 : 0) * p.N) * D + 8 * grp;
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) {
        if (hv)
          qf[s2].load(qrow + 32 * s2);
        else
          qf[s2].zero();
      }
      float sq = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = qf[s2].get(e);
          sq += x * x;
        }
      const float sq_all = colgroup_sum(sq);  // every lane takes part in the exchange
      const float qn = row_sum16(hv ? sqrtf(sq_all) : 0.f);
      Frag<uint16_t> qh[D / 32];
      const int te = route_q_f16<D>(qf, qh);
      const float col_scale = ldexpf(p.scale, -(te + hexp));
      int kept;
      const int nk =
          walk_to_level1<uint16_t, D, KM>(p.lv, kLog2C, p.K, i, &kept, [&](int lc, int cn, int n_cand, int e_child) {
            return select_level_refine<D, KM>(rows, norms, (int)p.lv.roff[lc], qh, qn, cn, n_cand, e_child, p.G,
                                              p.scale, col_scale, p.K, s_sc[wave], s_key[wave]);
          });
      if (lane < p.K) p.kept[u * p.K + lane] = lane < nk ? kept : -1;
    }
  }
}

template <typename T>
struct LeafParams {
  const T* q;
  const T* k;
  const int* kept;
  const uint32_t* pairs;
  const int* total;
  int B, Hq, Hkv, G, N, K, q_tile, tasks, chunk_log2;
  float scale;
  float* leaf_lse;  // [U, K, 2, G]
};

constexpr int kLeafTask = 256;  // pairs per wave task

// One tile of q_tile pairs x G heads (16 columns): the column's query fragments and its pair.
template <typename T, int D>
struct LeafTile {
  Frag<T> qf[D / 32];
  long long u;
  int slot;
  bool valid;
};

// The tiled leaf stage: wave task t covers pairs [256 t, 256 t + 256) of the bucket-sorted list. For
// each run of one bucket (same KV head and level-1 node) the key tile is loaded once into registers
// and tiles of q_tile units x G heads are scored against it; the query fragments of the tile two
// ahead are in flight while a tile runs.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void leaf_lse_kernel(LeafParams<T> p) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int task = xcd_logical_block(gridDim.x) * 4 + wave;
  const long long total = *p.total;
  const long long pos0 = (long long)task * kLeafTask;
  if (task >= p.tasks || pos0 >= total) return;
  PairRun run;
  run.base = pos0;
  run.end = pos0 + kLeafTask < total ? pos0 + kLeafTask : total;
  const long long nch = ((long long)p.N + (1LL << p.chunk_log2) - 1) >> p.chunk_log2;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const long long x = pos0 + 64 * w + lane;
    run.pr[w] = x < run.end ? p.pairs[x] : 0u;
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const long long x = pos0 + 64 * w + lane;
    const long long u = run.pr[w] >> 5;
    run.key[w] = x < run.end ? ((u / p.N) * nch + ((u % p.N) >> p.chunk_log2)) * (1LL << 32) +
                                   p.kept[u * p.K + (run.pr[w] & 31)]
                             : -1;
  }
  const int h = r16 % p.G;
  const int cols = p.q_tile * p.G;
  long long pos = pos0;
  while (pos < run.end) {
    const uint32_t pr0 = run.pair(pos);
    const long long u0 = readlane((int)(pr0 >> 5), 0);
    const long long bh = u0 / p.N;
    const int node = p.kept[u0 * p.K + (readlane((int)pr0, 0) & 31)];
    const long long seg = run.run_end(pos, (bh * nch + ((u0 % p.N) >> p.chunk_log2)) * (1LL << 32) + node);
    const T* kbh = p.k + bh * (long long)p.N * D;
    const long long t0 = 2LL * node * C;
    Frag<T> kf[C / 8][D / 32];
    load_leaf_pair<T, D, C>(kbh, t0, p.N, kf);
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    const T* qhead = p.q + (((long long)b * p.Hq + (long long)r * p.G + h) * p.N) * D + 8 * grp;
    const long long ubase = bh * p.N;
    auto fetch = [&](LeafTile<T, D>& t, long long tp) {
      const long long pi = tp + r16 / p.G;
      t.valid = r16 < cols && pi < seg;
      const uint32_t pc = run.pair(t.valid ? pi : pos);
      t.u = pc >> 5;
      t.slot = pc & 31;
      const T* qrow = qhead + (t.u - ubase) * D;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        if (t.valid)
          t.qf[s].load(qrow + 32 * s);
        else
          t.qf[s].zero();
      }
    };
    auto score = [&](const LeafTile<T, D>& t) {
      float l0, l1;
      leaf_pair_lse<T, D, C>(kf, t.qf, t0, t.valid ? t.u - ubase : -1, p.scale, l0, l1);
      if (grp == 0 && t.valid) {
        float* dst = p.leaf_lse + ((t.u * p.K + t.slot) * 2) * p.G + h;
        dst[0] = l0;
        dst[p.G] = l1;
      }
    };
    const long long step = p.q_tile;
    const long long ntiles = (seg - pos + step - 1) / step;
    // ring of R tiles: the query fragments of tile t+R are requested as tile t finishes
    // (bf16 tiles are small enough for R = 4 without spilling; fp32 keeps R = 2)
    constexpr int R = sizeof(T) == 2 ? 4 : 2;
    LeafTile<T, D> X[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < ntiles) fetch(X[r], pos + r * step);
    for (long long t = 0; t < ntiles; t += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (t + r < ntiles) {
          score(X[r]);
          if (t + r + R < ntiles) fetch(X[r], pos + (t + r + R) * step);
        }
      }
    }
    pos = seg;
  }
}

// bf16, work-group cooperative leaf stage: a work-group task is kLeafWgTask consecutive sorted pairs;
// for each run (one KV head and level-1 node) the 256 threads stage the node's two leaves (2C keys)
// into LDS, then the four waves take the run's tiles of q_tile units x G heads round-robin, reading
// every K fragment from LDS. The per-column arithmetic (fragment values, MFMA order, LSE code) is the
// unit-major leaf stage's, so both give the same bits. Four work-groups share a CU (at most 128
// registers per lane and 40 KiB of LDS each: 512-pair tasks, 16-bit run offsets), so that many waves
// cover the query gathers' latency, each with one register set of queries in flight. The bound names
// three work-groups per CU: under it the compiler keeps two key-fragment reads from LDS in flight
// ahead of the MFMAs (under a bound of four it waits for each read) and still ends at 124 registers,
// so four work-groups fit all the same.
constexpr int kLeafWgTask = 512;

template <int D, int C>
__global__ __launch_bounds__(256, 3) void leaf_lse_wg_kernel(LeafParams<uint16_t> p) {
  __shared__ __align__(16) uint16_t s_k[2 * C][D];
  __shared__ uint32_t s_pair[kLeafWgTask];
  __shared__ long long s_key[kLeafWgTask];
  __shared__ uint16_t s_run[kLeafWgTask + 1];
  __shared__ int s_wcount[4];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long total = *p.total;
  const long long base = (long long)xcd_logical_block(gridDim.x) * kLeafWgTask;
  if (base >= total) return;  // whole work-group
  const int n = (int)(total - base < kLeafWgTask ? total - base : kLeafWgTask);
  const long long nch = ((long long)p.N + (1LL << p.chunk_log2) - 1) >> p.chunk_log2;
  const int nrun = stage_pair_runs<kLeafWgTask>(
      p.pairs, base, n,
      [&](uint32_t pr) {
        const long long u = pr >> 5;
        const unsigned bh = (unsigned)u / (unsigned)p.N, i = (unsigned)u - bh * (unsigned)p.N;  // u < 2^27
        return ((long long)bh * nch + (i >> p.chunk_log2)) * (1LL << 32) + p.kept[u * p.K + (pr & 31)];
      },
      s_pair, s_key, s_run, s_wcount);
  const int h = r16 % p.G;
  const int cols = p.q_tile * p.G;
  for (int r = 0; r < nrun; ++r) {
    const int a = s_run[r], b = s_run[r + 1];
    const long long u0 = s_pair[a] >> 5;
    const long long bh = u0 / p.N;
    const int node = (int)(s_key[a] & 0xffffffffLL);
    const long long t0 = 2LL * node * C;
    const uint16_t* kbh = p.k + bh * (long long)p.N * D;
    stage_leaf_pair_wg<D, C>(kbh, t0, p.N, s_k);
    __syncthreads();
    const int bi = (int)(bh / p.Hkv), ri = (int)(bh % p.Hkv);
    // quad-coalesced query loads: lane 4 r + c reads chunks 4 s + c of column r's query row (64
    // contiguous bytes per quad and k step); quad_rows_to_mfma() moves them to the MFMA layout
    const int qr = quad_row(), hq = qr % p.G;
    const uint16_t* qhead =
        p.q + (((long long)bi * p.Hq + (long long)ri * p.G + hq) * p.N) * D + 8 * quad_chunk();
    const long long ubase = bh * p.N;
    const int ntiles = (b - a + p.q_tile - 1) / p.q_tile;
    // A column past the run, past the tile's q_tile units, or past the wave's last tile repeats the
    // run's first pair: it computes that pair's values again and stores the same bits to the same place.
    // pc: the pair of this lane's column (r16).
    auto fetch = [&](int t, Frag<uint16_t> (&qf)[D / 32], uint32_t& pc) {
      int xl = a + t * p.q_tile + qr / p.G;
      xl = (t < ntiles && qr < cols && xl < b) ? xl : a;
      const uint16_t* qrow = qhead + ((long long)(s_pair[xl] >> 5) - ubase) * D;
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) qf[s2].load(qrow + 32 * s2);
      int x = a + t * p.q_tile + r16 / p.G;
      x = (t < ntiles && r16 < cols && x < b) ? x : a;
      pc = s_pair[x];
    };
    struct Out {
      float l0, l1;
      uint32_t pc;
    };
    auto score = [&](Frag<uint16_t> (&qf)[D / 32], uint32_t pc, Out& out) {
      out.pc = pc;
      quad_rows_to_mfma(qf);
      leaf_pair_lse_k<uint16_t, D, C, true>([&](int m, int s2) { return leaf_k_frag_wg<D>(s_k, m, s2); }, qf, t0,
                                      (long long)(pc >> 5) - ubase, p.scale, out.l0, out.l1);
    };
    auto store = [&](const Out& out) {
      // the column's 4 lanes hold the same values
      float* dst = p.leaf_lse + ((long long)(out.pc >> 5) * p.K + (out.pc & 31)) * 2 * p.G + h;
      dst[0] = out.l0;
      dst[p.G] = out.l1;
    };
    if (wave < ntiles) {
      // the queries of this wave's next tile (t + 4) are requested as soon as tile t has read its own
      Frag<uint16_t> qa[D / 32];
      uint32_t pa;
      fetch(wave, qa, pa);
      opaque_frags(qa);
      for (int t = wave; t < ntiles; t += 4) {
        Out out;
        score(qa, pa, out);
        fetch(t + 4, qa, pa);
        store(out);
      }
    }
    __syncthreads();  // every wave is done with this node's keys before they are restaged
  }
}

template <typename T>
struct FinParams {
  const int* kept;
  const float* leaf_lse;
  int B, Hq, Hkv, G, N, K, C, upw;
  int* sel;
  float* sel_lse;
};

// A wave finalizes kFinUnits consecutive units. Every unit's kept slots and its candidates' head-summed
// leaf LSEs are requested before any Top-K, so the wave waits for memory once. Candidate lanes past a
// unit's count read values that the Top-K ignores.
constexpr int kFinUnits = 4;

__global__ __launch_bounds__(256) void finalize_kernel(FinParams<float> p) {
  __shared__ __align__(16) uint32_t s_key[4][64];
  // unit indices fit in 32 bits (packed pairs hold them in 27), and every index here is wave-uniform
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const unsigned U = (unsigned)p.B * p.Hkv * p.N;
  const unsigned first = ((unsigned)xcd_logical_block(gridDim.x) * 4 + wave) * kFinUnits;
  const int slot = lane >> 1;
  const bool cand_lane = slot < p.K;
  int kp[kFinUnits];
  float sc[kFinUnits];
#pragma unroll
  for (int it = 0; it < kFinUnits; ++it) {
    const unsigned u = first + it < U ? first + it : U - 1;
    kp[it] = cand_lane ? p.kept[(long long)u * p.K + slot] : -1;
    const float* ll = p.leaf_lse + ((long long)u * p.K * 2 + (cand_lane ? lane : 0)) * p.G;
    float x = 0.f;  // heads in index order
    if ((p.G & 3) == 0) {
      // 16-byte loads (the rows are 16-byte aligned): a lane quad reads 64 contiguous bytes
      for (int h = 0; h < p.G; h += 4) {
        const float4 v = *reinterpret_cast<const float4*>(ll + h);
        x += v.x;
        x += v.y;
        x += v.z;
        x += v.w;
      }
    } else {
      for (int h = 0; h < p.G; ++h) x += ll[h];
    }
    sc[it] = x;
  }
#pragma unroll
  for (int it = 0; it < kFinUnits; ++it) {
    const unsigned u = first + it;
    if (u >= U) break;
    const unsigned bh = u / (unsigned)p.N, i = u - bh * (unsigned)p.N;
    const int b = (int)(bh / (unsigned)p.Hkv), r = (int)(bh - (unsigned)b * p.Hkv);
    const int leaf_c = 2 * kp[it] + (lane & 1);
    const bool valid = kp[it] >= 0 && (long long)leaf_c * p.C <= (long long)i;
    const int n_cand = __popcll(__ballot(valid));
    const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
    const float* ll = p.leaf_lse + u * p.K * 2 * p.G;
    leaf_topk_write_sc(
        n_cand, leaf_c, sc[it], p.G, p.K, u, qrow0, p.N, [&](int c, int h) { return ll[c * p.G + h]; }, p.sel,
        p.sel_lse, s_key[wave]);
  }
}

// K <= 16: a unit has at most 32 leaf candidates, so each half-wave finalizes its own unit (lanes
// 32 half + c hold candidate c of unit 2 it + half): ranking, compaction and stores run for two units at
// once. Same keys, same ranking rule and the same head order as finalize_kernel, so the same outputs.
__global__ __launch_bounds__(256) void finalize_half_kernel(FinParams<float> p) {
  __shared__ __align__(16) uint32_t s_key[4][64];
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5, cl = lane & 31;
  const unsigned U = (unsigned)p.B * p.Hkv * p.N;
  const unsigned first = ((unsigned)xcd_logical_block(gridDim.x) * 4 + wave) * kFinUnits;
  const int slot = cl >> 1;
  const bool cand_lane = slot < p.K;
  constexpr int NP = kFinUnits / 2;  // passes of two units
  int kp[NP];
  float sc[NP];
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const unsigned u0 = first + 2 * it + half;
    const unsigned u = u0 < U ? u0 : U - 1;
    kp[it] = cand_lane ? p.kept[(long long)u * p.K + slot] : -1;
    const float* ll = p.leaf_lse + ((long long)u * p.K * 2 + (cand_lane ? cl : 0)) * p.G;
    float x = 0.f;  // heads in index order
    if ((p.G & 3) == 0) {
      for (int h = 0; h < p.G; h += 4) {
        const float4 v = *reinterpret_cast<const float4*>(ll + h);
        x += v.x;
        x += v.y;
        x += v.z;
        x += v.w;
      }
    } else {
      for (int h = 0; h < p.G; ++h) x += ll[h];
    }
    sc[it] = x;
  }
  uint32_t* keys = s_key[wave] + 32 * half;
  const unsigned long long hmask = 0xffffffffull << (32 * half);
#pragma unroll
  for (int it = 0; it < NP; ++it) {
    const unsigned u = first + 2 * it + half;
    const bool live = u < U;  // both halves run every step; a dead half stores nothing
    const unsigned uu = live ? u : U - 1;
    const unsigned bh = uu / (unsigned)p.N, i = uu - bh * (unsigned)p.N;
    const int b = (int)(bh / (unsigned)p.Hkv), r = (int)(bh - (unsigned)b * p.Hkv);
    const int leaf_c = 2 * kp[it] + (cl & 1);
    const bool valid = kp[it] >= 0 && (long long)leaf_c * p.C <= (long long)i;
    const int n_cand = __popcll(__ballot(valid) & hmask);  // valid candidates are a prefix
    // Top-K by key (score descending, index ascending; keyed relative to the unit's first candidate, as
    // topk_keep does); slots past the candidates hold 0
    const float r0 = readlane(sc[it], 0), r1 = readlane(sc[it], 32);
    const float hr = half ? r1 : r0;
    const float ref = __builtin_isfinite(hr) ? hr : 0.f;
    const uint32_t mine = cl < n_cand ? topk_key(sc[it] - ref, cl) : 0u;
    keys[cl] = mine;
    __threadfence_block();
    bool keep = cl < n_cand;
    if (n_cand > p.K) {
      int rank = 0;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + c);
        rank += (v.x > mine) + (v.y > mine) + (v.z > mine) + (v.w > mine);
      }
      keep = keep && rank < p.K;
    }
    __threadfence_block();  // the next unit rewrites the keys
    // stable compaction within the half
    const unsigned m = (unsigned)((__ballot(keep) & hmask) >> (32 * half));
    const int below = __popc(m & ((1u << cl) - 1u));
    const int nsel = __popc(m);
    const int dst = 32 * half + (keep ? below : nsel + (cl - below));
    const int leaf_sel = __builtin_amdgcn_ds_permute(dst << 2, leaf_c);
    const int c_sel = __builtin_amdgcn_ds_permute(dst << 2, cl);
    if (live && cl < p.K) {
      p.sel[(long long)u * p.K + cl] = cl < nsel ? leaf_sel : -1;
      if (p.sel_lse) {
        const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
        const float* ll = p.leaf_lse + (long long)u * p.K * 2 * p.G;
        for (int h = 0; h < p.G; ++h)
          p.sel_lse[(qrow0 + (long long)h * p.N) * p.K + cl] = cl < nsel ? ll[c_sel * p.G + h] : kNegInf;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------ regroup
// Counting sort of (unit, slot) pairs by (KV head, node). Work-group = a run of units of one KV head;
// ranks are taken in LDS, then each non-empty bucket reserves its range with one global atomic.
__global__ __launch_bounds__(256) void fill_zero_kernel(int* x, long long n) {
  for (long long j = (long long)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += (long long)gridDim.x * blockDim.x)
    x[j] = 0;
}

constexpr int kRegroupUnits = 1024;

__global__ __launch_bounds__(1024) void hist_kernel(const int* __restrict__ nodes, int K, int N, int nb, int chunks,
                                                   int chunk_log2, int use_lds, int* __restrict__ counts,
                                                   int* __restrict__ ranks) {
  extern __shared__ int lc[];  // nb local counts, then nb bases
  const int bh = blockIdx.x / chunks, ch = blockIdx.x % chunks;
  const long long i0 = (long long)ch * kRegroupUnits;
  const long long u0 = (long long)bh * N + i0;
  const long long u1 = (long long)bh * N + (i0 + kRegroupUnits < N ? i0 + kRegroupUnits : N);
  const long long n_pairs = (u1 - u0) * K;
  const long long p0 = u0 * K;
  // every unit of this work-group lies in one position chunk (chunk_log2 >= log2 kRegroupUnits)
  const int nch = (int)(((long long)N + (1LL << chunk_log2) - 1) >> chunk_log2);
  const long long bucket0 = ((long long)bh * nch + (i0 >> chunk_log2)) * nb;
  if (!use_lds) {
    for (long long x = threadIdx.x; x < n_pairs; x += blockDim.x) {
      const int nd = nodes[p0 + x];
      if (nd >= 0 && nd < nb) ranks[p0 + x] = atomicAdd(&counts[bucket0 + nd], 1);
    }
    return;
  }
  for (int j = threadIdx.x; j < nb; j += blockDim.x) lc[j] = 0;
  __syncthreads();
  for (long long x = threadIdx.x; x < n_pairs; x += blockDim.x) {
    const int nd = nodes[p0 + x];
    if (nd >= 0 && nd < nb) ranks[p0 + x] = atomicAdd(&lc[nd], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int c = lc[j];
    lc[nb + j] = c ? atomicAdd(&counts[bucket0 + j], c) : 0;
  }
  __syncthreads();
  for (long long x = threadIdx.x; x < n_pairs; x += blockDim.x) {
    const int nd = nodes[p0 + x];
    if (nd >= 0 && nd < nb) ranks[p0 + x] += lc[nb + nd];
  }
}

// Exclusive scan of n counts into offsets[0..n] (one work-group of 1024 threads; counts and offsets
// 16-byte aligned). Tiles of 4096 counts: each thread reads 4 consecutive counts of the tile as one 16-byte
// load (the next tile's load is in flight meanwhile), the waves scan their threads' sums by lane
// shuffles, the wave totals meet in LDS, and the tile's total carries into the next tile.
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts, long long n, int* __restrict__ offsets) {
  constexpr int kTile = 4096;
  __shared__ int s_wave[16];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  auto load4 = [&](long long j) {
    if (j + 3 < n) return *reinterpret_cast<const int4*>(counts + j);
    return make_int4(j < n ? counts[j] : 0, j + 1 < n ? counts[j + 1] : 0, j + 2 < n ? counts[j + 2] : 0, 0);
  };
  long long carry = 0;  // the counts of the tiles before this one
  int4 c = load4(4LL * tid);
  for (long long t0 = 0; t0 < n; t0 += kTile) {
    const long long j = t0 + 4LL * tid;
    const int4 nx = t0 + kTile < n ? load4(j + kTile) : make_int4(0, 0, 0, 0);
    const int own = c.x + c.y + c.z + c.w;
    int x = own;  // inclusive scan over the wave's lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int v = s_wave[w];
      before += w < wave ? v : 0;
      total += v;
    }
    const int e0 = (int)carry + before + x - own;  // offset of this thread's first count
    const int4 o4 = make_int4(e0, e0 + c.x, e0 + c.x + c.y, e0 + c.x + c.y + c.z);
    if (j + 3 < n) {
      *reinterpret_cast<int4*>(offsets + j) = o4;
    } else {
      if (j < n) offsets[j] = o4.x;
      if (j + 1 < n) offsets[j + 1] = o4.y;
      if (j + 2 < n) offsets[j + 2] = o4.z;
    }
    carry += total;
    c = nx;
    __syncthreads();  // s_wave is rewritten by the next tile
  }
  if (tid == 0) offsets[n] = (int)carry;
}

// With to_positions, ranks[x] is replaced by the pair's index in the sorted list (its row in the
// leaf-major attention's partial outputs); entries that are not attended get 0, an index that exists,
// so a reader that trusts a malformed selection still stays inside the partial buffer.
__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ nodes, long long n_pairs, int K, int N,
                                                      int nb, int chunk_log2, const int* __restrict__ offsets,
                                                      int* __restrict__ ranks, int to_positions,
                                                      uint32_t* __restrict__ pairs) {
  const int nch = (int)(((long long)N + (1LL << chunk_log2) - 1) >> chunk_log2);
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n_pairs; x += (long long)gridDim.x * blockDim.x) {
    const int nd = nodes[x];
    if (nd < 0 || nd >= nb) {  // out-of-range entries are not attended
      if (to_positions) ranks[x] = 0;
      continue;
    }
    // pair indices fit in 32 bits (a packed pair holds its unit in 27), so the divisions are 32-bit
    const unsigned u = (unsigned)x / (unsigned)K;
    const int slot = (int)((unsigned)x - u * (unsigned)K);
    const unsigned bh = u / (unsigned)N, i = u - bh * (unsigned)N;
    const int at = offsets[((long long)bh * nch + (i >> chunk_log2)) * nb + nd] + ranks[x];
    pairs[at] = (uint32_t)((u << 5) | (unsigned)slot);
    if (to_positions) ranks[x] = at;
  }
}

hipError_t launch_regroup(const int* nodes, long long U, int K, int N, int nb, int n_heads, int chunk_log2,
                          int* counts, int* offsets, int* ranks, bool ranks_to_positions, uint32_t* pairs,
                          hipStream_t st) {
  const int nch = (int)(((long long)N + (1LL << chunk_log2) - 1) >> chunk_log2);
  const long long NB = (long long)nb * nch * n_heads;
  long long zb = (NB + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(zb < 4096 ? zb : 4096)), dim3(256), 0, st, counts, NB);
  const int chunks = (N + kRegroupUnits - 1) / kRegroupUnits;
  const int use_lds = nb <= 8192;  // 2*nb ints of LDS, at most 64 KiB
  const size_t lds = use_lds ? (size_t)nb * 2 * sizeof(int) : 0;
  hipLaunchKernelGGL(hist_kernel, dim3(n_heads * chunks), dim3(1024), lds, st, nodes, K, N, nb, chunks, chunk_log2,
                     use_lds, counts, ranks);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, NB, offsets);
  const long long n_pairs = U * K;
  long long sb = (n_pairs + 255) / 256;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)(sb < 65536 ? sb : 65536)), dim3(256), 0, st, nodes, n_pairs, K, N,
                     nb, chunk_log2, offsets, ranks, ranks_to_positions ? 1 : 0, pairs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ launchers
template <typename T, int D, int C, bool FUSED>
static hipError_t route_t(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                          const int* hexp, int* kept, int* sel, float* sel_lse, hipStream_t st) {
  RouteParams<T> p;
  p.hexp = hexp;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.nodes = nodes;
  p.norms = norms;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.scale = sd.scale;
  p.lv = sd.lv;
  p.kept = kept;
  p.sel = sel;
  p.sel_lse = sel_lse;
  p.units = nullptr;
  p.n_units = 0;
  p.trace = nullptr;
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  if constexpr (sizeof(T) == 2 && !FUSED) {
    // LDS-resident upper levels: the smallest level whose rows up to the root fit in kRouteLdsBytes
    int lcut = 0;
    while (lcut < sd.lv.n_levels - 1 && (sd.lv.rnodes - sd.lv.roff[lcut]) * D * 2 > kRouteLdsBytes) ++lcut;
    const int lds_first = (int)sd.lv.roff[lcut];
    const int BH = sd.B * sd.Hkv;
    const long long groups = (sd.N + kRouteUnits - 1) / kRouteUnits;
    long long wph = 256 / BH;  // about one work-group per CU
    if (wph < 1) wph = 1;
    if (sd.K <= 16) {
      constexpr int NW = route_lds_waves<4>();
      if (wph > (groups + NW - 1) / NW) wph = (groups + NW - 1) / NW;
      hipLaunchKernelGGL((route_lds_kernel<D, C, 4>), dim3((unsigned)(BH * wph)), dim3(NW * 64), 0, st, p, lds_first,
                         (int)wph);
    } else {
      constexpr int NW = route_lds_waves<8>();
      if (wph > (groups + NW - 1) / NW) wph = (groups + NW - 1) / NW;
      hipLaunchKernelGGL((route_lds_kernel<D, C, 8>), dim3((unsigned)(BH * wph)), dim3(NW * 64), 0, st, p, lds_first,
                         (int)wph);
    }
    return hipGetLastError();
  }
  else {
    p.upw = 4;
    const long long waves = (U + p.upw - 1) / p.upw;
    const long long blocks = (waves + 3) / 4;
    if (sd.K <= 16)
      hipLaunchKernelGGL((route_kernel<T, D, C, FUSED, 4>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    else
      hipLaunchKernelGGL((route_kernel<T, D, C, FUSED, 8>), dim3((unsigned)blocks), dim3(256), 0, st, p);
    return hipGetLastError();
  }
}

template <typename T, bool FUSED>
static hipError_t route_dc(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                           const int* hexp, int* kept, int* sel, float* sel_lse, hipStream_t st) {
  if (sd.D == 128) {
    if (sd.C == 64) return route_t<T, 128, 64, FUSED>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
    return route_t<T, 128, 32, FUSED>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
  }
  if (sd.C == 64) return route_t<T, 64, 64, FUSED>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
  return route_t<T, 64, 32, FUSED>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
}

// The traced walk: one wave per listed unit, route_kernel's fused walk and leaf stage.
template <typename T, int D, int C>
static hipError_t route_trace_t(const SelDims& sd, const void* q, const void* k, const void* nodes,
                                const float* norms, const int* hexp, const long long* units, long long n_units,
                                int* trace, hipStream_t st) {
  RouteParams<T> p;
  p.hexp = hexp;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.nodes = nodes;
  p.norms = norms;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.scale = sd.scale;
  p.lv = sd.lv;
  p.kept = nullptr;
  p.sel = nullptr;
  p.sel_lse = nullptr;
  p.units = units;
  p.n_units = n_units;
  p.trace = trace;
  p.upw = 1;
  const long long blocks = (n_units + 3) / 4;
  if (sd.K <= 16)
    hipLaunchKernelGGL((route_kernel<T, D, C, true, 4, true>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((route_kernel<T, D, C, true, 8, true>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t route_trace_dc(const SelDims& sd, const void* q, const void* k, const void* nodes,
                                 const float* norms, const int* hexp, const long long* units, long long n_units,
                                 int* trace, hipStream_t st) {
  if (sd.D == 128) {
    if (sd.C == 64) return route_trace_t<T, 128, 64>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
    return route_trace_t<T, 128, 32>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
  }
  if (sd.C == 64) return route_trace_t<T, 64, 64>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
  return route_trace_t<T, 64, 32>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
}

hipError_t launch_route_trace(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                              const int* hexp, const long long* units, long long n_units, int* trace,
                              hipStream_t st) {
  if (n_units == 0) return hipSuccess;
  if (sd.bf16) return route_trace_dc<uint16_t>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
  return route_trace_dc<float>(sd, q, k, nodes, norms, hexp, units, n_units, trace, st);
}

hipError_t launch_route(const SelDims& sd, const void* q, const void* k, const void* nodes, const float* norms,
                        const int* hexp, bool fused, int* kept, int* sel, float* sel_lse, hipStream_t st) {
  if (sd.bf16)
    return fused ? route_dc<uint16_t, true>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st)
                 : route_dc<uint16_t, false>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
  return fused ? route_dc<float, true>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st)
               : route_dc<float, false>(sd, q, k, nodes, norms, hexp, kept, sel, sel_lse, st);
}

template <typename T, int D, int C>
static hipError_t leaf_t(const SelDims& sd, const void* q, const void* k, const int* kept, const uint32_t* pairs,
                         const int* total, float* leaf_lse, hipStream_t st) {
  LeafParams<T> p;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.kept = kept;
  p.pairs = pairs;
  p.total = total;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.q_tile = sd.q_tile;
  p.chunk_log2 = sd.chunk_log2;
  p.scale = sd.scale;
  p.leaf_lse = leaf_lse;
  const long long max_pairs = (long long)sd.B * sd.Hkv * sd.N * sd.K;
  if constexpr (sizeof(T) == 2) {
    const long long wg = (max_pairs + kLeafWgTask - 1) / kLeafWgTask;
    p.tasks = (int)wg;
    hipLaunchKernelGGL((leaf_lse_wg_kernel<D, C>), dim3((unsigned)wg), dim3(256), 0, st, p);
  } else {
    const long long tasks = (max_pairs + kLeafTask - 1) / kLeafTask;
    p.tasks = (int)tasks;
    const long long blocks = (tasks + 3) / 4;
    hipLaunchKernelGGL((leaf_lse_kernel<T, D, C>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_leaf_lse(const SelDims& sd, const void* q, const void* k, const int* kept, const uint32_t* pairs,
                           const int* total, float* leaf_lse, hipStream_t st) {
  if (sd.bf16) {
    if (sd.D == 128)
      return sd.C == 64 ? leaf_t<uint16_t, 128, 64>(sd, q, k, kept, pairs, total, leaf_lse, st)
                        : leaf_t<uint16_t, 128, 32>(sd, q, k, kept, pairs, total, leaf_lse, st);
    return sd.C == 64 ? leaf_t<uint16_t, 64, 64>(sd, q, k, kept, pairs, total, leaf_lse, st)
                      : leaf_t<uint16_t, 64, 32>(sd, q, k, kept, pairs, total, leaf_lse, st);
  }
  if (sd.D == 128)
    return sd.C == 64 ? leaf_t<float, 128, 64>(sd, q, k, kept, pairs, total, leaf_lse, st)
                      : leaf_t<float, 128, 32>(sd, q, k, kept, pairs, total, leaf_lse, st);
  return sd.C == 64 ? leaf_t<float, 64, 64>(sd, q, k, kept, pairs, total, leaf_lse, st)
                    : leaf_t<float, 64, 32>(sd, q, k, kept, pairs, total, leaf_lse, st);
}

hipError_t launch_finalize(const SelDims& sd, const int* kept, const float* leaf_lse, int* sel, float* sel_lse,
                           hipStream_t st) {
  FinParams<float> p;
  p.kept = kept;
  p.leaf_lse = leaf_lse;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.C = sd.C;
  p.upw = kFinUnits;
  p.sel = sel;
  p.sel_lse = sel_lse;
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  const long long waves = (U + kFinUnits - 1) / kFinUnits;
  if (sd.K <= 16)
    hipLaunchKernelGGL(finalize_half_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace pisa
