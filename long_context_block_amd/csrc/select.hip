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

namespace pisa {

template <typename T, int D>
struct NodeRows;

// bf16 path: row r at base + r*2D holds hi[D] then lo[D].
template <int D>
struct NodeRows<uint16_t, D> {
  const uint16_t* base;
  __device__ __forceinline__ void dot(f32x4& acc, long long row, bool valid, int grp,
                                      const Frag<uint16_t> (&qf)[D / 32]) const {
    const uint16_t* p = base + row * 2 * D + (D / 4) * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      Frag<uint16_t> hi, lo;
      if (valid) {
        hi.load(p + 8 * s);
        lo.load(p + D + 8 * s);
      } else {
        hi.zero();
        lo.zero();
      }
      mma(acc, hi, qf[s]);
      mma(acc, lo, qf[s]);
    }
  }
};

// fp32 path: row r at base + r*D.
template <int D>
struct NodeRows<float, D> {
  const float* base;
  __device__ __forceinline__ void dot(f32x4& acc, long long row, bool valid, int grp,
                                      const Frag<float> (&qf)[D / 32]) const {
    const float* p = base + row * D + (D / 4) * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      Frag<float> m;
      if (valid)
        m.load(p + 8 * s);
      else
        m.zero();
      mma(acc, m, qf[s]);
    }
  }
};

// Scores of the candidates in lanes [0, n_cand) (node index cn, ascending) at a level l >= 1:
// sum over heads of the LSE over the eligible children (level l-1, first token <= i) of
// scale * q . mean(child). cspan = tokens per child node. Lanes >= n_cand get -inf.
template <typename T, int D>
__device__ float score_candidates(const NodeRows<T, D>& rows, long long level_off, const Frag<T> (&qf)[D / 32], int cn,
                                  int n_cand, long long cspan, long long i, int G, float scale) {
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  const int MT = (2 * n_cand + 15) >> 4;
  float res = kNegInf;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < MT) {
      const int row = 16 * m + r16;
      const int cidx = row >> 1;
      const int cnode = __shfl(cn, cidx);
      const long long child = 2LL * cnode + (row & 1);
      const bool valid = cidx < n_cand && child * cspan <= i;
      f32x4 acc = zero4();
      rows.dot(acc, level_off + (valid ? child : 0), valid, grp, qf);
      float hs[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int c = 8 * m + 2 * grp + a;
        const int pn = __shfl(cn, c);
        const bool v1 = c < n_cand && (2LL * pn + 1) * cspan <= i;
        const float x0 = scale * acc[2 * a], x1 = scale * acc[2 * a + 1];
        float l = v1 ? lse2(x0, x1) : x0;
        l = r16 < G ? l : 0.f;
        l += __shfl_xor(l, 1);
        l += __shfl_xor(l, 2);
        l += __shfl_xor(l, 4);
        l += __shfl_xor(l, 8);
        hs[a] = l;
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float t = __shfl(hs[a], 16 * ((lane & 7) >> 1));
        if ((lane >> 3) == m && (lane & 1) == a) res = t;
      }
    }
  }
  return lane < n_cand ? res : kNegInf;
}

// Walk from the root to level 1. Levels whose eligible node count is <= K keep every node, so the
// walk starts below the highest level with more than K eligible nodes. Returns the number of kept
// level-1 nodes; lane c < n holds the c-th (ascending). A pyramid of one leaf has the virtual
// level-1 node 0.
template <typename T, int D>
__device__ int walk_to_level1(const NodeRows<T, D>& rows, const Levels& lv, const Frag<T> (&qf)[D / 32], int C, int K,
                              int G, float scale, long long i, int* kept_out) {
  const int lane = lane_id();
  const int L = lv.n_levels - 1;
  int lstar = 0;
  for (int l = L; l >= 1; --l) {
    if (i / ((long long)C << l) + 1 > K) {
      lstar = l;
      break;
    }
  }
  int nk, kept;
  if (lstar == 0) {
    nk = (int)(i / (2LL * C) + 1);
    *kept_out = lane < nk ? lane : -1;
    return nk;
  }
  nk = (int)(i / ((long long)C << (lstar + 1)) + 1);
  kept = lane < nk ? lane : -1;
  for (int l = lstar; l >= 1; --l) {
    const long long span = (long long)C << l;
    const int par = __shfl(kept, lane >> 1);
    const int cn = 2 * par + (lane & 1);
    int n_cand = 2 * nk;
    const int last = readlane(cn, n_cand - 1);
    if ((long long)last * span > i) --n_cand;
    if (n_cand <= K) {
      kept = lane < n_cand ? cn : -1;
      nk = n_cand;
      continue;
    }
    const float sc = score_candidates<T, D>(rows, lv.off[l - 1], qf, cn, n_cand, (long long)C << (l - 1), i, G, scale);
    const bool keep = topk_keep(sc, n_cand, K);
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
        kf[m][s].load(kbh + t * D + (D / 4) * grp + 8 * s);
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

template <typename T>
struct RouteParams {
  const T* q;
  const T* k;
  const void* nodes;
  int B, Hq, Hkv, G, N, K, upw;
  float scale;
  Levels lv;
  int* kept;      // [U, K] (tiled path)
  int* sel;       // [U, K] (fused path)
  float* sel_lse; // [B, Hq, N, K] or null (fused path)
};

// Top-K of the leaf candidates and the outputs. Lane c < n_cand is candidate c = 2*slot + bit
// (leaf 2*kept[slot] + bit); ell(c, h) gives its per-head LSE. The heads are summed in index order.
template <typename F>
__device__ __forceinline__ void leaf_topk_write(int n_cand, int leaf_c, int G, int K, long long u, long long qrow0,
                                                long long qstride, F ell, int* sel, float* sel_lse) {
  const int lane = lane_id();
  const bool need_rank = n_cand > K;
  bool keep = lane < n_cand;
  if (need_rank) {
    float sc = 0.f;
    if (lane < n_cand)
      for (int h = 0; h < G; ++h) sc += ell(lane, h);
    sc = lane < n_cand ? sc : kNegInf;
    keep = topk_keep(sc, n_cand, K);
  }
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

template <typename T, int D, int C, bool FUSED>
__global__ __launch_bounds__(256) void route_kernel(RouteParams<T> p) {
  __shared__ float s_ell[4][64][17];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long U = (long long)p.B * p.Hkv * p.N;
  const int lb = xcd_logical_block(gridDim.x);
  const long long first = ((long long)lb * 4 + wave) * p.upw;
  for (int it = 0; it < p.upw; ++it) {
    const long long u = first + it;
    if (u >= U) break;
    const long long bh = u / p.N;
    const long long i = u % p.N;
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    Frag<T> qf[D / 32];
    const bool hv = r16 < p.G;
    const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
    const T* qrow = p.q + (qrow0 + (long long)(hv ? r16 : 0) * p.N) * D + (D / 4) * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (hv)
        qf[s].load(qrow + 8 * s);
      else
        qf[s].zero();
    }
    NodeRows<T, D> rows;
    if constexpr (sizeof(T) == 2)
      rows.base = (const uint16_t*)p.nodes + bh * p.lv.nodes * 2 * D;
    else
      rows.base = (const float*)p.nodes + bh * p.lv.nodes * D;
    int kept;
    const int nk = walk_to_level1<T, D>(rows, p.lv, qf, C, p.K, p.G, p.scale, i, &kept);
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
            s_ell[wave][2 * slot][r16] = l0;
            s_ell[wave][2 * slot + 1][r16] = l1;
          }
        }
        __threadfence_block();
      }
      leaf_topk_write(
          n_cand, leaf_c, p.G, p.K, u, qrow0, p.N, [&](int c, int h) { return s_ell[wave][c][h]; }, p.sel, p.sel_lse);
      __threadfence_block();
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
  int B, Hq, Hkv, G, N, K, q_tile, tasks;
  float scale;
  float* leaf_lse;  // [U, K, 2, G]
};

constexpr int kLeafTask = 64;  // pairs per wave task

// The tiled leaf stage: wave task t covers pairs [64 t, 64 t + 64) of the bucket-sorted list. Within
// each run of one bucket (same KV head and level-1 node) the key tile is loaded once and tiles of
// q_tile units x G heads are scored against it.
template <typename T, int D, int C>
__global__ __launch_bounds__(256) void leaf_lse_kernel(LeafParams<T> p) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int task = xcd_logical_block(gridDim.x) * 4 + wave;
  const long long total = *p.total;
  long long pos = (long long)task * kLeafTask;
  if (task >= p.tasks || pos >= total) return;
  const long long end = pos + kLeafTask < total ? pos + kLeafTask : total;
  while (pos < end) {
    const uint32_t pr = p.pairs[pos];
    const long long u = pr >> 5;
    const long long bh = u / p.N;
    const int node = p.kept[u * p.K + (pr & 31)];
    // end of this bucket's run inside [pos, end)
    long long seg = end;
    for (long long base = pos; base < end; base += 64) {
      const long long x = base + lane;
      bool diff = false;
      if (x < end) {
        const uint32_t q2 = p.pairs[x];
        const long long u2 = q2 >> 5;
        diff = (u2 / p.N != bh) || (p.kept[u2 * p.K + (q2 & 31)] != node);
      }
      const unsigned long long m = __ballot(diff);
      if (m) {
        seg = base + __ffsll((long long)m) - 1;
        break;
      }
    }
    const T* kbh = p.k + bh * (long long)p.N * D;
    const long long t0 = 2LL * node * C;
    Frag<T> kf[C / 8][D / 32];
    load_leaf_pair<T, D, C>(kbh, t0, p.N, kf);
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    const int cols = p.q_tile * p.G;
    for (long long tp = pos; tp < seg; tp += p.q_tile) {
      const long long pi = tp + r16 / p.G;
      const int h = r16 % p.G;
      const bool cv = r16 < cols && pi < seg;
      long long uc = 0, ic = 0;
      int slot = 0;
      Frag<T> qf[D / 32];
      if (cv) {
        const uint32_t pc = p.pairs[pi];
        uc = pc >> 5;
        slot = pc & 31;
        ic = uc % p.N;
        const T* qrow = p.q + ((((long long)b * p.Hq + (long long)r * p.G + h) * p.N) + ic) * D + (D / 4) * grp;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) qf[s].load(qrow + 8 * s);
      } else {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) qf[s].zero();
      }
      float l0, l1;
      leaf_pair_lse<T, D, C>(kf, qf, t0, cv ? ic : -1, p.scale, l0, l1);
      if (grp == 0 && cv) {
        float* dst = p.leaf_lse + ((uc * p.K + slot) * 2) * p.G + h;
        dst[0] = l0;
        dst[p.G] = l1;
      }
    }
    pos = seg;
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

__global__ __launch_bounds__(256) void finalize_kernel(FinParams<float> p) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const long long U = (long long)p.B * p.Hkv * p.N;
  const long long first = ((long long)xcd_logical_block(gridDim.x) * 4 + wave) * p.upw;
  for (int it = 0; it < p.upw; ++it) {
    const long long u = first + it;
    if (u >= U) break;
    const long long bh = u / p.N, i = u % p.N;
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    const int slot = lane >> 1;
    const int kp = slot < p.K ? p.kept[u * p.K + slot] : -1;
    const int leaf_c = 2 * kp + (lane & 1);
    const bool valid = kp >= 0 && (long long)leaf_c * p.C <= i;
    const int n_cand = __popcll(__ballot(valid));
    const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
    const float* ll = p.leaf_lse + u * p.K * 2 * p.G;
    leaf_topk_write(
        n_cand, leaf_c, p.G, p.K, u, qrow0, p.N, [&](int c, int h) { return ll[c * p.G + h]; }, p.sel, p.sel_lse);
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

__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ nodes, int K, int N, int nb, int chunks,
                                                   int use_lds, int* __restrict__ counts, int* __restrict__ ranks) {
  extern __shared__ int lc[];  // nb local counts, then nb bases
  const int bh = blockIdx.x / chunks, ch = blockIdx.x % chunks;
  const long long u0 = (long long)bh * N + (long long)ch * kRegroupUnits;
  const long long u1 = (long long)bh * N + ((long long)(ch + 1) * kRegroupUnits < N ? (long long)(ch + 1) * kRegroupUnits : N);
  const long long n_pairs = (u1 - u0) * K;
  const long long p0 = u0 * K;
  if (!use_lds) {
    for (long long x = threadIdx.x; x < n_pairs; x += blockDim.x) {
      const int nd = nodes[p0 + x];
      if (nd >= 0 && nd < nb) ranks[p0 + x] = atomicAdd(&counts[(long long)bh * nb + nd], 1);
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
    lc[nb + j] = c ? atomicAdd(&counts[(long long)bh * nb + j], c) : 0;
  }
  __syncthreads();
  for (long long x = threadIdx.x; x < n_pairs; x += blockDim.x) {
    const int nd = nodes[p0 + x];
    if (nd >= 0 && nd < nb) ranks[p0 + x] += lc[nb + nd];
  }
}

// Exclusive scan of n counts into offsets[0..n] (one work-group of 1024 threads).
__global__ __launch_bounds__(1024) void scan_kernel(const int* __restrict__ counts, long long n, int* __restrict__ offsets) {
  __shared__ long long s_part[1024];
  const long long per = (n + 1023) / 1024;
  const long long a = threadIdx.x * per, e = a + per < n ? a + per : n;
  long long s = 0;
  for (long long j = a; j < e; ++j) s += counts[j];
  s_part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const long long v = threadIdx.x >= off ? s_part[threadIdx.x - off] : 0;
    __syncthreads();
    s_part[threadIdx.x] += v;
    __syncthreads();
  }
  long long run = threadIdx.x ? s_part[threadIdx.x - 1] : 0;
  for (long long j = a; j < e; ++j) {
    offsets[j] = (int)run;
    run += counts[j];
  }
  if (threadIdx.x == 1023) offsets[n] = (int)s_part[1023];
}

__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ nodes, long long n_pairs, int K, int N,
                                                      int nb, const int* __restrict__ offsets,
                                                      const int* __restrict__ ranks, uint32_t* __restrict__ pairs) {
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < n_pairs; x += (long long)gridDim.x * blockDim.x) {
    const int nd = nodes[x];
    if (nd < 0 || nd >= nb) continue;  // out-of-range entries are not attended
    const long long u = x / K;
    const int slot = (int)(x % K);
    const long long bh = u / N;
    pairs[offsets[bh * nb + nd] + ranks[x]] = (uint32_t)((u << 5) | slot);
  }
}

hipError_t launch_regroup(const int* nodes, long long U, int K, int N, int nb, int n_heads, int* counts, int* offsets,
                          int* ranks, uint32_t* pairs, hipStream_t st) {
  const long long NB = (long long)nb * n_heads;
  long long zb = (NB + 255) / 256;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)(zb < 4096 ? zb : 4096)), dim3(256), 0, st, counts, NB);
  const int chunks = (N + kRegroupUnits - 1) / kRegroupUnits;
  const int use_lds = nb <= 8192;  // 2*nb ints of LDS, at most 64 KiB
  const size_t lds = use_lds ? (size_t)nb * 2 * sizeof(int) : 0;
  hipLaunchKernelGGL(hist_kernel, dim3(n_heads * chunks), dim3(256), lds, st, nodes, K, N, nb, chunks, use_lds, counts,
                     ranks);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, NB, offsets);
  const long long n_pairs = U * K;
  long long sb = (n_pairs + 255) / 256;
  hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)(sb < 65536 ? sb : 65536)), dim3(256), 0, st, nodes, n_pairs, K, N,
                     nb, offsets, ranks, pairs);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------ launchers
template <typename T, int D, int C, bool FUSED>
static hipError_t route_t(const SelDims& sd, const void* q, const void* k, const void* nodes, int* kept, int* sel,
                          float* sel_lse, hipStream_t st) {
  RouteParams<T> p;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.nodes = nodes;
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
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  p.upw = 4;
  const long long waves = (U + p.upw - 1) / p.upw;
  const long long blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((route_kernel<T, D, C, FUSED>), dim3((unsigned)blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename T, bool FUSED>
static hipError_t route_dc(const SelDims& sd, const void* q, const void* k, const void* nodes, int* kept, int* sel,
                           float* sel_lse, hipStream_t st) {
  if (sd.D == 128) {
    if (sd.C == 64) return route_t<T, 128, 64, FUSED>(sd, q, k, nodes, kept, sel, sel_lse, st);
    return route_t<T, 128, 32, FUSED>(sd, q, k, nodes, kept, sel, sel_lse, st);
  }
  if (sd.C == 64) return route_t<T, 64, 64, FUSED>(sd, q, k, nodes, kept, sel, sel_lse, st);
  return route_t<T, 64, 32, FUSED>(sd, q, k, nodes, kept, sel, sel_lse, st);
}

hipError_t launch_route(const SelDims& sd, const void* q, const void* k, const void* nodes, bool fused, int* kept,
                        int* sel, float* sel_lse, hipStream_t st) {
  if (sd.bf16)
    return fused ? route_dc<uint16_t, true>(sd, q, k, nodes, kept, sel, sel_lse, st)
                 : route_dc<uint16_t, false>(sd, q, k, nodes, kept, sel, sel_lse, st);
  return fused ? route_dc<float, true>(sd, q, k, nodes, kept, sel, sel_lse, st)
               : route_dc<float, false>(sd, q, k, nodes, kept, sel, sel_lse, st);
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
  p.scale = sd.scale;
  p.leaf_lse = leaf_lse;
  const long long max_pairs = (long long)sd.B * sd.Hkv * sd.N * sd.K;
  const long long tasks = (max_pairs + kLeafTask - 1) / kLeafTask;
  p.tasks = (int)tasks;
  const long long blocks = (tasks + 3) / 4;
  hipLaunchKernelGGL((leaf_lse_kernel<T, D, C>), dim3((unsigned)blocks), dim3(256), 0, st, p);
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
  p.upw = 4;
  p.sel = sel;
  p.sel_lse = sel_lse;
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  const long long waves = (U + p.upw - 1) / p.upw;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace pisa
