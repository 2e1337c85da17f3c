// Device tiles of the pyramid walk and the leaf LSE, shared by the prefill selection kernels and the
// fused decode step (see select.hip for the method citations).
#pragma once
#include "common.hpp"

namespace pisa {

template <typename T, int D>
struct NodeRows;

// bf16 path: row r at base + r*2D holds hi[D] then lo[D]; one row fragment = hi and lo halves.
template <int D>
struct NodeRows<uint16_t, D> {
  const uint16_t* base;
  __device__ __forceinline__ int index(int level_off, int child, int) const { return level_off + child; }
  struct Row {
    Frag<uint16_t> hi[D / 32], lo[D / 32];
  };
  __device__ __forceinline__ void load(Row& f, int row, int grp) const {
    const uint16_t* p = base + (unsigned)row * (2 * D) + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      f.hi[s].load(p + 32 * s);
      f.lo[s].load(p + D + 32 * s);
    }
  }
  __device__ __forceinline__ void dot(f32x4& acc, const Row& f, const Frag<uint16_t> (&qf)[D / 32]) const {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      mma(acc, f.hi[s], qf[s]);
      mma(acc, f.lo[s], qf[s]);
    }
  }
};

// fp16 routing planes of one KV head (hi = rne(2^hexp mean), lo = rne(2^hexp mean - hi)), addressed by
// routing row (Levels::roff) in the quad-interleaved layout of route_plane_chunk.
template <int D>
struct RoutePlanes {
  const uint16_t* base;  // the KV head's planes
  // hi plane of routing row R (the first pass of the routing walk)
  __device__ __forceinline__ void load_hi(Frag<uint16_t> (&hi)[D / 32], int R, int grp) const {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) hi[s].load(route_plane_chunk(base, R, 0, 4 * s + grp, D));
  }
  // the row's hi-plane score bound
  __device__ __forceinline__ float bound(const float* norms, int R) const { return norms[R]; }
  // lo plane of routing row R, zero where !need. R must be a valid row either way: the load is
  // unconditional and its value dropped afterwards, because a load under a lane condition makes the
  // compiler wait for it before issuing the next one.
  // lo plane of routing row R as read (for rows whose sums are discarded when not needed)
  __device__ __forceinline__ void load_lo_any(Frag<uint16_t> (&lo)[D / 32], int R, int grp) const {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) lo[s].load(route_plane_chunk(base, R, 1, 4 * s + grp, D));
  }
  __device__ __forceinline__ void load_lo(Frag<uint16_t> (&lo)[D / 32], int R, int grp, bool need) const {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      Frag<uint16_t> v;
      v.load(route_plane_chunk(base, R, 1, 4 * s + grp, D));
      lo[s].u = need ? v.u : make_uint4(0u, 0u, 0u, 0u);
    }
  }
};

// The column's query (bf16 fragments qf) in fp16 scaled by 2^te, max |q| 2^te in [2^14, 2^15) over the
// column (zero columns: te = 0): exact, since a bf16 value keeps its 8 significant bits in fp16 in that
// range (values under 2^-14 after scaling, 2^-28 of the largest, may round: the routing bound's
// accumulation slack covers them). Returns te.
template <int D>
__device__ __forceinline__ int route_q_f16(const Frag<uint16_t> (&qf)[D / 32], Frag<uint16_t> (&qh)[D / 32]) {
  float mx = 0.f;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(qf[s].get(e)));
  const int te = f16_range_exp(colgroup_max(mx));
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)f32_to_f16_bits(ldexpf(qf[s].get(2 * e), te)) |
             ((uint32_t)f32_to_f16_bits(ldexpf(qf[s].get(2 * e + 1), te)) << 16);
    qh[s].u = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return te;
}

// Fragments of local LDS row r (layout below): chunk 4 s + grp sits at chunk (4 s + grp) ^ (r mod D/8),
// i.e. at element (r D + 8 (grp ^ (r mod D/8))) ^ 32 s, since 4 s only flips chunk bits that r D and
// grp do not touch: one address per row, then a constant XOR per k step.
template <int D>
__device__ __forceinline__ void lds_hi_row(Frag<uint16_t> (&hi)[D / 32], const uint16_t* lds, int r, int grp) {
  // byte offsets: one XOR per k step
  const unsigned b0 = 2u * (unsigned)(r * D + 8 * (grp ^ (r & (D / 8 - 1))));
  const char* base = reinterpret_cast<const char*>(lds);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) hi[s].u = *reinterpret_cast<const uint4*>(base + (b0 ^ (64u * s)));
}

// Routing walk with the hi plane of the upper pyramid rows (node >= first) resident in LDS: local row
// r = node - first holds D hi values, 16-byte chunk c stored at chunk c ^ (r mod D/8), so the 4
// consecutive rows of one kept node (its grandchildren) fall on distinct chunk columns. Lower rows and
// every lo plane are read from global memory.
template <int D>
struct LdsHiRows : RoutePlanes<D> {
  const uint16_t* lds;
  const float* lds_bound;  // the same rows' hi-plane bounds
  int first;
  __device__ __forceinline__ float bound(const float* norms, int node) const {
    return node >= first ? lds_bound[node - first] : norms[node];
  }
  __device__ __forceinline__ void load_hi(Frag<uint16_t> (&hi)[D / 32], int node, int grp) const {
    if (node >= first) {
      lds_hi_row<D>(hi, lds, node - first, grp);
    } else {
      RoutePlanes<D>::load_hi(hi, node, grp);
    }
  }
};

// Level-uniform row access. All rows of one pyramid level are either LDS-resident or not, so the choice
// is made once per level (a scalar branch) and each path issues plain LDS or plain global loads that can
// be in flight together; a per-lane choice compiles to flat loads, each waited for before its MFMA.
template <int D>
struct GlobalHiLoader {
  const RoutePlanes<D>* rows;
  __device__ __forceinline__ void load_hi(Frag<uint16_t> (&hi)[D / 32], int node, int grp) const {
    rows->load_hi(hi, node, grp);
  }
  __device__ __forceinline__ float bound(const float* norms, int node) const { return norms[node]; }
};
template <int D>
struct LdsHiLoader {
  const uint16_t* lds;
  const float* lds_bound;
  int first;
  __device__ __forceinline__ void load_hi(Frag<uint16_t> (&hi)[D / 32], int node, int grp) const {
    lds_hi_row<D>(hi, lds, node - first, grp);
  }
  __device__ __forceinline__ float bound(const float*, int node) const { return lds_bound[node - first]; }
};
// f(loader) for the level whose rows start at level_off (wave-uniform)
template <int D, class F>
__device__ __forceinline__ void for_level_rows(const RoutePlanes<D>& rows, int, F&& f) {
  f(GlobalHiLoader<D>{&rows});
}
template <int D, class F>
__device__ __forceinline__ void for_level_rows(const LdsHiRows<D>& rows, int level_off, F&& f) {
  if (__builtin_amdgcn_readfirstlane(level_off) >= rows.first)
    f(LdsHiLoader<D>{rows.lds, rows.lds_bound, rows.first});
  else
    f(GlobalHiLoader<D>{&rows});
}

// Cooperative copy of the hi planes of routing rows [first, first + n) into lds (layout above) and of
// their bounds into lds_bound. Consecutive threads read consecutive 16-byte pieces of a row group.
template <int D>
__device__ __forceinline__ void stage_hi_rows(const uint16_t* base, const float* norms, int first, int n,
                                              uint16_t* lds, float* lds_bound) {
  constexpr int CHR = D / 8;
  for (int x = threadIdx.x; x < n; x += blockDim.x) lds_bound[x] = norms[first + x];
  const int a0 = first >> 2, a1 = (first + n + 3) >> 2;  // row groups touched
  for (int x = threadIdx.x; x < (a1 - a0) * 4 * CHR; x += blockDim.x) {
    const int R = 4 * (a0 + x / (4 * CHR)) + (x & 3), c = (x >> 2) % CHR;
    const int r = R - first;
    if (r >= 0 && r < n)
      *reinterpret_cast<uint4*>(lds + r * D + 8 * (c ^ (r & (CHR - 1)))) =
          *reinterpret_cast<const uint4*>(route_plane_chunk(base, R, 0, c, D));
  }
}

// fp32 path: row r at base + r*D.
template <int D>
struct NodeRows<float, D> {
  const float* base;
  __device__ __forceinline__ int index(int level_off, int child, int) const { return level_off + child; }
  struct Row {
    Frag<float> m[D / 32];
  };
  __device__ __forceinline__ void load(Row& f, int row, int grp) const {
    const float* p = base + (unsigned)row * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) f.m[s].load(p + 32 * s);
  }
  __device__ __forceinline__ void dot(f32x4& acc, const Row& f, const Frag<float> (&qf)[D / 32]) const {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) mma(acc, f.m[s], qf[s]);
  }
};

// Scores of the candidates c in [0, n_cand) (node index cn in lane c, ascending) at a level l >= 1:
// sum over heads of the LSE over the eligible children (level l-1) of scale * q . mean(child). Child
// nodes below e_child are eligible (first token <= i); since the candidates are the children of an
// ascending kept list, only the last candidate can miss its second child. KM = M-tiles for 2K
// candidates (2 rows each). The scores land in s_sc[c] (LDS).
template <typename T, int D, int KM, class Rows = NodeRows<T, D>>
__device__ void score_candidates(const Rows& rows, int level_off, const Frag<T> (&qf)[D / 32], int cn,
                                 int n_cand, int e_child, int G, float scale, float* s_sc) {
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  const int MT = (2 * n_cand + 15) >> 4;
  const bool last_two = 2 * readlane(cn, n_cand - 1) + 1 < e_child;  // last candidate has both children
  const int n_full = last_two ? n_cand : n_cand - 1;                 // candidates with two eligible children
  int child[KM];
#pragma unroll
  for (int m = 0; m < KM; ++m) {
    const int row = 16 * m + r16;
    const int cidx = row >> 1;
    const int cnode = __shfl(cn, cidx & 63);
    const bool valid = cidx < n_cand && ((row & 1) == 0 || cidx < n_full);
    child[m] = valid ? 2 * cnode + (row & 1) : 0;
  }
  constexpr int MB = 2;  // M-tiles whose loads are in flight together
#pragma unroll
  for (int m0 = 0; m0 < KM; m0 += MB) {
    if (m0 < MT) {
      typename NodeRows<T, D>::Row f[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) rows.load(f[mb], rows.index(level_off, child[m0 + mb], 16 * (m0 + mb) + r16), grp);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int m = m0 + mb;
        if (m < MT) {
          f32x4 acc = zero4();
          rows.dot(acc, f[mb], qf);
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int c = 8 * m + 2 * grp + a;
            const float x0 = scale * acc[2 * a], x1 = scale * acc[2 * a + 1];
            float l = c < n_full ? lse2(x0, x1) : x0;
            l = row_sum16(r16 < G ? l : 0.f);
            if (r16 == 0) s_sc[c] = l;
          }
        }
      }
    }
  }
  __threadfence_block();
}

// One scored level for bf16 inputs, in two passes over the <= 4K child rows of the fp16 routing planes
// (hi = rne(2^hexp mean), lo = rne(2^hexp mean - hi)). Pass 1 uses the hi plane only; a candidate's
// score then lies within E_c = scale * sum_h |q_h| * max over its children of the row bound b
// (b >= |q . lo| / |q| plus the accumulation slack, in unscaled units) of its hi+lo score (LSE is
// 1-Lipschitz in the max norm, per head). With the Top-K of the hi scores as the "in" group, a
// candidate is decided by pass 1 when its interval cannot cross the boundary (an "in" candidate whose
// lower end is above every "out" upper end, or an "out" candidate whose upper end is below every "in"
// lower end); the rest get the lo plane added (pass 2) and compete by their hi+lo scores for the
// remaining places. The kept set is the one the hi+lo scores of every candidate give, while only the
// lo rows of undecided candidates are read. Returns this lane's keep flag.
// qf: the column's query in fp16 scaled by 2^te (route_q_f16); col_scale = scale 2^-(te + hexp) returns
// the dot products with the scaled planes to scale * q . mean.
template <int D, int KM, class Rows>
__device__ bool select_level_refine(const Rows& rows, const float* norms, int level_off,
                                    const Frag<uint16_t> (&qf)[D / 32], float qnorm_sum, int cn, int n_cand,
                                    int e_child, int G, float scale, float col_scale, int K, float* s_sc,
                                    uint32_t* keys) {
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  n_cand = __builtin_amdgcn_readfirstlane(n_cand);
  const int MT = (2 * n_cand + 15) >> 4;
  const bool last_two = 2 * readlane(cn, n_cand - 1) + 1 < e_child;
  const int n_full = last_two ? n_cand : n_cand - 1;
  int child[KM];
  bool valid[KM];
#pragma unroll
  for (int m = 0; m < KM; ++m) {
    const int row = 16 * m + r16;
    const int cidx = row >> 1;
    const int cnode = __shfl(cn, cidx & 63);
    valid[m] = cidx < n_cand && ((row & 1) == 0 || cidx < n_full);
    child[m] = valid[m] ? 2 * cnode + (row & 1) : 0;
  }
  // pass 1: hi plane, after the candidates' child-row bounds are requested
  f32x4 acc[KM];
  float nb0 = 0.f, nb1 = 0.f;
  for_level_rows(rows, level_off, [&](const auto& ld) {
    if (lane < n_cand) {
      nb0 = ld.bound(norms, level_off + 2 * cn);
      nb1 = lane < n_full ? ld.bound(norms, level_off + 2 * cn + 1) : 0.f;
    }
    // every M-tile is loaded (invalid rows read row level_off; tiles past MT are never scored), so no
    // branch separates the tiles' loads
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      Frag<uint16_t> hi[D / 32];
      ld.load_hi(hi, level_off + child[m], grp);
      acc[m] = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mma_f16(acc[m], hi[s], qf[s]);
    }
  });
  auto cand_scores = [&](int m, unsigned long long only) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int c = 8 * m + 2 * grp + a;
      const float x0 = col_scale * acc[m][2 * a], x1 = col_scale * acc[m][2 * a + 1];
      float l = c < n_full ? lse2(x0, x1) : x0;
      l = row_sum16(r16 < G ? l : 0.f);
      if (r16 == 0 && ((only >> (c & 63)) & 1ull)) s_sc[c] = l;
    }
  };
#pragma unroll
  for (int m = 0; m < KM; ++m)
    if (m < MT) cand_scores(m, ~0ull);
  const float e = lane < n_cand ? scale * qnorm_sum * fmaxf(nb0, nb1) : 0.f;
  __threadfence_block();
  const float sh = lane < n_cand ? s_sc[lane] : kNegInf;
  // both passes key relative to the first candidate's hi score (the routing kernels that walk several
  // units per wave use the same reference)
  const float ref = topk_ref(sh);
  const bool in = topk_keep_ref(sh, n_cand, K, keys, ref);
  const float lo_b = sh - e, hi_b = sh + e;
  const float u_out = wave_max(!in && lane < n_cand ? hi_b : kNegInf);
  const float l_in = wave_min(in ? lo_b : -kNegInf);
  const bool refine = lane < n_cand && ((in && lo_b <= u_out) || (!in && hi_b >= l_in));
  const unsigned long long rmask = __ballot(refine);
  if (rmask == 0ull) return in;
  // pass 2: lo plane of the undecided candidates' rows
#pragma unroll
  for (int m = 0; m < KM; ++m) {
    const unsigned long long tile = (rmask >> (8 * m)) & 0xffull;
    if (m < MT && tile) {
      const int cidx = (16 * m + r16) >> 1;
      const bool need = valid[m] && ((rmask >> cidx) & 1ull);
      Frag<uint16_t> lo[D / 32];
      rows.load_lo(lo, level_off + (need ? child[m] : 0), grp, need);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) mma_f16(acc[m], lo[s], qf[s]);
      cand_scores(m, rmask);
    }
  }
  __threadfence_block();
  const float key = refine ? s_sc[lane < n_cand ? lane : 0] : (in ? -kNegInf : kNegInf);
  return topk_keep_ref(key, n_cand, K, keys, ref);
}

// Walk from the root to level 1 for query position i. Level l has e_l = (i >> (log2 C + l)) + 1
// eligible nodes; levels with e_l <= K keep all of them, so the walk starts below the highest level
// with more than K. level_select(child level, candidate node, n_cand, eligible children) scores one
// level. Returns the number of kept level-1 nodes; lane c < n holds the c-th (ascending).
// A pyramid of one leaf has the virtual level-1 node 0.
// level_hook(l, kept, nk), if given, sees every level l >= 1 once, from the top: lane c < nk holds
// the c-th kept node of level l (ascending); where a level has at most K eligible nodes, all of them.
template <typename T, int D, int KM, class LevelSelect, class LevelHook>
__device__ int walk_to_level1(const Levels& lv, int log2c, int K, int i, int* kept_out, LevelSelect&& level_select,
                              LevelHook&& level_hook) {
  const int lane = lane_id();
  const int L = lv.n_levels - 1;
  int lstar = 0;
  for (int l = L; l >= 1; --l) {
    if ((i >> (log2c + l)) + 1 > K) {
      lstar = l;
      break;
    }
  }
  for (int l = L; l > lstar; --l) {  // levels with at most K eligible nodes keep them all
    const int n_l = (i >> (log2c + l)) + 1;
    level_hook(l, lane < n_l ? lane : -1, n_l);
  }
  int nk, kept;
  if (lstar == 0) {
    nk = (i >> (log2c + 1)) + 1;
    *kept_out = lane < nk ? lane : -1;
    return nk;
  }
  nk = (i >> (log2c + lstar + 1)) + 1;
  kept = lane < nk ? lane : -1;
  for (int l = lstar; l >= 1; --l) {
    const int e_l = (i >> (log2c + l)) + 1;
    const int par = __shfl(kept, lane >> 1);
    const int cn = 2 * par + (lane & 1);
    int n_cand = 2 * nk;
    if (readlane(cn, n_cand - 1) >= e_l) --n_cand;
    if (n_cand <= K) {
      kept = lane < n_cand ? cn : -1;
      nk = n_cand;
      level_hook(l, kept, nk);
      continue;
    }
    const bool keep = level_select(l - 1, cn, n_cand, (i >> (log2c + l - 1)) + 1);
    int cnt;
    const int nxt = compact_lanes(keep, cn, &cnt);
    kept = lane < cnt ? nxt : -1;
    nk = cnt;
    level_hook(l, kept, nk);
  }
  *kept_out = kept;
  return nk;
}

template <typename T, int D, int KM, class LevelSelect>
__device__ int walk_to_level1(const Levels& lv, int log2c, int K, int i, int* kept_out, LevelSelect&& level_select) {
  return walk_to_level1<T, D, KM>(lv, log2c, K, i, kept_out, level_select, [](int, int, int) {});
}

// Key tile of leaves 2p and 2p+1: rows = tokens t0 .. t0+2C-1 of one KV head. Rows past N repeat token
// N - 1: those tokens are later than every query, so the causal mask drops them before any use (the
// loads stay unconditional, so all of them are in flight together).
template <typename T, int D, int C>
__device__ __forceinline__ void load_leaf_pair(const T* kbh, long long t0, int N, Frag<T> (&kf)[C / 8][D / 32]) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
  for (int m = 0; m < C / 8; ++m) {
    long long t = t0 + 16 * m + r16;
    t = t < N ? t : N - 1;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) kf[m][s].load(kbh + t * D + 32 * s + 8 * grp);
  }
}

// Per-column LSEs of the two leaves from the accumulated tile dot products (acc[m]: tokens t0 + 16 m +
// (0..15)), masking tokens after icol in place.
template <typename T, int C>
__device__ __forceinline__ void leaf_pair_lse_acc(f32x4 (&acc)[C / 8], long long t0, long long icol, float scale,
                                                  float& lse0, float& lse1) {
  constexpr int ML = C / 16;  // M-tiles per leaf
  const int grp = lane_id() >> 4;
  // causal mask on offsets within the tile: token t0 + o is visible iff o <= icol - t0
  const long long lim64 = icol - t0;
  const int lim = lim64 < 0 ? -1 : (lim64 > 2 * C ? 2 * C : (int)lim64);
  // bf16: every column sees all 2C tokens (the usual case away from the diagonal): no mask (same
  // values). The mask is applied in place, so both cases score the same registers.
  bool all_visible = false;
  if constexpr (sizeof(T) == 2) all_visible = __all(lim >= 2 * C - 1);
  if (!all_visible) {
#pragma unroll
    for (int m = 0; m < 2 * ML; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int o = 16 * m + 4 * grp + j;
        if (o > lim) acc[m][j] = kNegInf;
      }
  }
#pragma unroll
  for (int bit = 0; bit < 2; ++bit) {
    float x[ML * 4];
#pragma unroll
    for (int mm = 0; mm < ML; ++mm)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[mm * 4 + j] = acc[bit * ML + mm][j];
    const float l = column_lse<ML * 4>(x, scale);
    if (bit == 0)
      lse0 = l;
    else
      lse1 = l;
  }
}

// Per-column LSE over leaf 2p (lse0) and leaf 2p+1 (lse1) of scale * q_col . k_t for t <= icol.
// kfrag(m, s) returns the A-fragment of tokens t0 + 16 m + (0..15), k step s.
// kPhased: a scheduling fence after each k step, so that LDS-sourced fragments of one step at a time
// are live (the arithmetic is unchanged).
template <typename T, int D, int C, bool kPhased = false, typename KFrag>
__device__ __forceinline__ void leaf_pair_lse_k(KFrag kfrag, const Frag<T> (&qf)[D / 32], long long t0,
                                                long long icol, float scale, float& lse0, float& lse1) {
  constexpr int MT = C / 8;
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = zero4();
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
#pragma unroll
    for (int m = 0; m < MT; ++m) mma(acc[m], kfrag(m, s), qf[s]);
    if constexpr (kPhased) __builtin_amdgcn_sched_barrier(0);
  }
  leaf_pair_lse_acc<T, C>(acc, t0, icol, scale, lse0, lse1);
}

template <typename T, int D, int C>
__device__ __forceinline__ void leaf_pair_lse(const Frag<T> (&kf)[C / 8][D / 32], const Frag<T> (&qf)[D / 32],
                                              long long t0, long long icol, float scale, float& lse0, float& lse1) {
  leaf_pair_lse_k<T, D, C>([&](int m, int s) -> const Frag<T>& { return kf[m][s]; }, qf, t0, icol, scale, lse0,
                           lse1);
}

// ---- work-group shared bf16 key tile of a leaf pair (2C x D rows in LDS)
// 16-byte chunk c of row t is stored at chunk c ^ (t mod D/8): the 16 consecutive rows that one
// A-fragment read touches then fall on distinct chunk columns (no bank conflicts).
template <int D>
__device__ __forceinline__ int leaf_kswz(int t) {
  return t & (D / 8 - 1);
}

// Cooperative staging by 256 threads of tokens t0 .. t0 + 2C - 1 (past N: token N - 1, which the
// causal mask drops for every query).
template <int D, int C>
__device__ __forceinline__ void stage_leaf_pair_wg(const uint16_t* kbh, long long t0, long long N,
                                                   uint16_t (*sk)[D]) {
  constexpr int CHR = D / 8, NCH = 2 * C * CHR, IT = NCH / 256;
  static_assert(NCH % 256 == 0, "tile shape");
  const int tid = threadIdx.x;
  uint4 kk[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    long long tt = t0 + t;
    tt = tt < N ? tt : N - 1;
    kk[it] = *reinterpret_cast<const uint4*>(kbh + tt * D + 8 * c);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    *reinterpret_cast<uint4*>(&sk[t][8 * (c ^ leaf_kswz<D>(t))]) = kk[it];
  }
}

template <int D>
__device__ __forceinline__ Frag<uint16_t> leaf_k_frag_wg(const uint16_t (*sk)[D], int m, int s) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
  const int t = 16 * m + r16;
  Frag<uint16_t> f;
  f.u = *reinterpret_cast<const uint4*>(&sk[t][8 * ((4 * s + grp) ^ leaf_kswz<D>(t))]);
  return f;
}

}  // namespace pisa
