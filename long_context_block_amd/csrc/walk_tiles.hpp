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
// Child rows staged in LDS in MFMA-row order (row 2c + bit = child bit of candidate c): bf16 hi/lo
// planes, or fp32 rows. `index` maps (level offset, child node, MFMA row) to the row to read.
template <typename T, int D>
struct StagedRows;

template <int D>
struct StagedRows<uint16_t, D> : NodeRows<uint16_t, D> {
  __device__ __forceinline__ int index(int, int, int local_row) const { return local_row; }
};

template <int D>
struct StagedRows<float, D> : NodeRows<float, D> {
  __device__ __forceinline__ int index(int, int, int local_row) const { return local_row; }
};

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

// Walk from the root to level 1 for query position i. Level l has e_l = (i >> (log2 C + l)) + 1
// eligible nodes; levels with e_l <= K keep all of them, so the walk starts below the highest level
// with more than K. Returns the number of kept level-1 nodes; lane c < n holds the c-th (ascending).
// A pyramid of one leaf has the virtual level-1 node 0.
template <typename T, int D, int KM>
__device__ int walk_to_level1(const NodeRows<T, D>& rows, const Levels& lv, const Frag<T> (&qf)[D / 32], int log2c,
                              int K, int G, float scale, int i, int* kept_out, float* s_sc) {
  const int lane = lane_id();
  const int L = lv.n_levels - 1;
  int lstar = 0;
  for (int l = L; l >= 1; --l) {
    if ((i >> (log2c + l)) + 1 > K) {
      lstar = l;
      break;
    }
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
      continue;
    }
    score_candidates<T, D, KM>(rows, (int)lv.off[l - 1], qf, cn, n_cand, (i >> (log2c + l - 1)) + 1, G, scale, s_sc);
    const bool keep = topk_keep_lds(s_sc, n_cand, K);
    __threadfence_block();
    int cnt;
    const int nxt = compact_lanes(keep, cn, &cnt);
    kept = lane < cnt ? nxt : -1;
    nk = cnt;
  }
  *kept_out = kept;
  return nk;
}

// Key tile of leaves 2p and 2p+1: rows = tokens t0 .. t0+2C-1 of one KV head (zero past N).
template <typename T, int D, int C>
__device__ __forceinline__ void load_leaf_pair(const T* kbh, long long t0, int N, Frag<T> (&kf)[C / 8][D / 32]) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
  for (int m = 0; m < C / 8; ++m) {
    const long long t = t0 + 16 * m + r16;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (t < N)
        kf[m][s].load(kbh + t * D + 32 * s + 8 * grp);
      else
        kf[m][s].zero();
    }
  }
}

// Per-column LSE over leaf 2p (lse0) and leaf 2p+1 (lse1) of scale * q_col . k_t for t <= icol.
template <typename T, int D, int C>
__device__ __forceinline__ void leaf_pair_lse(const Frag<T> (&kf)[C / 8][D / 32], const Frag<T> (&qf)[D / 32],
                                              long long t0, long long icol, float scale, float& lse0, float& lse1) {
  constexpr int MT = C / 8;
  constexpr int ML = C / 16;  // M-tiles per leaf
  const int grp = lane_id() >> 4;
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = zero4();
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
#pragma unroll
    for (int m = 0; m < MT; ++m) mma(acc[m], kf[m][s], qf[s]);
  }
#pragma unroll
  for (int bit = 0; bit < 2; ++bit) {
    float x[ML * 4];
#pragma unroll
    for (int mm = 0; mm < ML; ++mm) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long long t = t0 + 16 * (bit * ML + mm) + 4 * grp + j;
        x[mm * 4 + j] = t <= icol ? acc[bit * ML + mm][j] : kNegInf;
      }
    }
    const float l = column_lse<ML * 4>(x, scale);
    if (bit == 0)
      lse0 = l;
    else
      lse1 = l;
  }
}

}  // namespace pisa
