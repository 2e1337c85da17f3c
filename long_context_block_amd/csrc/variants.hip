// Selection variants: the ablations and options the pages name beside the method.
//
// "Block Sparse Attention with Log-Linear Complexity" digest, 方法关键点, scoring bullet: the ablations
// score blocks by the mean (PISA-1) and by the mean plus the variance (PISA-2) instead of the LSE.
// "PISA：log-linear 复杂度的金字塔稀疏注意力" explainer: pooling may be mean, sum or max (核心方法 §1); the
// per-level budget may halve from level to level (核心方法 §7, 工程落地: start near 0.2 x blocks); the
// pool chain may be truncated at long N (工程落地 ⑥).
//
// pool_leaf_kernel / pool_level_kernel build a pyramid of pooled summaries (mean, sum or element-wise
// max of the raw keys in each node's span) and, optionally, the per-dimension variance of those keys:
// leaves straight from the keys (two passes: mean, then squared deviations), upper levels from their
// children (sum of sums, max of maxes, count-weighted means; variances combined by Chan's formula).
//
// variant_walk_kernel: one wave per unit. Level by level from the starting level L' (the root, or a
// cap): the candidates are every eligible node of L', then the eligible children of the kept nodes;
// a level with more than K_l candidates scores them and keeps its K_l best (score descending, index
// ascending; an exact search for the K_l-th largest 64-bit key). Scores: LSE over the eligible
// children's summaries (levels >= 1) or the exact LSE over the leaf's raw keys (leaves), on the leaf
// tiles of the main selection; or s q . summary (PISA-1); or that plus (s^2 / 2) sum_d q_d^2 var_d
// (PISA-2). Node dot products are fp32 on the VALU: this path measures the options, the main selection
// stays the fast one.
#include "common.hpp"
#include "internal.hpp"
#include "walk_tiles.hpp"

namespace pisa {

// ------------------------------------------------------------------------------------------ pooling
template <typename T>
struct PoolParams {
  const T* k;
  int BH, N, C, D, pool;
  Levels lv;
  float* summary;   // pyramid layout
  float* variance;  // nullable
};

// One work-group (D threads) per (KV head, leaf): thread d pools dimension d over the leaf's tokens.
template <typename T>
__global__ void pool_leaf_kernel(PoolParams<T> p) {
  const int d = threadIdx.x;
  const long long bh = blockIdx.x / p.lv.n[0], j = blockIdx.x % p.lv.n[0];
  const long long t0 = j * p.C, t1 = min((long long)p.N, t0 + p.C);
  const T* kk = p.k + (bh * p.N) * p.D + d;
  float s = 0.f, m = kNegInf;
  for (long long t = t0; t < t1; ++t) {
    const float x = to_f32<T>(kk[t * p.D]);
    s += x;
    m = fmaxf(m, x);
  }
  const float cnt = (float)(t1 - t0);
  const float mean = cnt > 0.f ? s / cnt : 0.f;
  const long long row = (bh * p.lv.nodes + j) * p.D + d;
  p.summary[row] = p.pool == 0 ? mean : p.pool == 1 ? s : (cnt > 0.f ? m : 0.f);
  if (p.variance) {
    float m2 = 0.f;
    for (long long t = t0; t < t1; ++t) {
      const float e = to_f32<T>(kk[t * p.D]) - mean;
      m2 = fmaf(e, e, m2);
    }
    p.variance[row] = cnt > 0.f ? m2 / cnt : 0.f;
  }
}

// Level l from level l - 1 (one work-group of D threads per node).
__global__ void pool_level_kernel(PoolParams<uint16_t> p, int l) {
  const int d = threadIdx.x;
  const long long bh = blockIdx.x / p.lv.n[l], j = blockIdx.x % p.lv.n[l];
  const long long w = (long long)p.C << (l - 1);  // tokens per child span
  const long long c0 = 2 * j, c1 = 2 * j + 1;
  const bool has1 = c1 < p.lv.n[l - 1];
  auto count = [&](long long c) {
    const long long a = c * w, b = min((long long)p.N, a + w);
    return (float)(b > a ? b - a : 0);
  };
  const float n0 = count(c0), n1 = has1 ? count(c1) : 0.f, n = n0 + n1;
  const long long r0 = (bh * p.lv.nodes + p.lv.off[l - 1] + c0) * p.D + d;
  const long long r1 = r0 + p.D;
  const long long row = (bh * p.lv.nodes + p.lv.off[l] + j) * p.D + d;
  const float a = p.summary[r0], b = has1 ? p.summary[r1] : 0.f;
  float out;
  if (p.pool == 0)
    out = n > 0.f ? (n0 * a + n1 * b) / n : 0.f;
  else if (p.pool == 1)
    out = a + b;
  else
    out = (has1 && n1 > 0.f) ? fmaxf(a, b) : a;
  p.summary[row] = out;
  if (p.variance) {
    // Chan's combination of (count, mean, M2): M2 = M2a + M2b + delta^2 na nb / n
    const float ma = p.pool == 0 ? a : (n0 > 0.f ? a / n0 : 0.f);
    const float mb = p.pool == 0 ? b : (n1 > 0.f ? b / n1 : 0.f);
    const float va = p.variance[r0], vb = has1 ? p.variance[r1] : 0.f;
    const float delta = mb - ma;
    const float m2 = va * n0 + vb * n1 + (n > 0.f ? delta * delta * n0 * n1 / n : 0.f);
    p.variance[row] = n > 0.f ? m2 / n : 0.f;
  }
}

hipError_t launch_pool_pooled(const void* k, bool bf16, const PyrDims& pd, int pool, float* summary, float* variance,
                              hipStream_t st) {
  PoolParams<uint16_t> pb{(const uint16_t*)k, pd.BH, pd.N, pd.C, pd.D, pool, pd.lv, summary, variance};
  const long long leaves = (long long)pd.BH * pd.lv.n[0];
  if (bf16) {
    hipLaunchKernelGGL(pool_leaf_kernel<uint16_t>, dim3((unsigned)leaves), dim3(pd.D), 0, st, pb);
  } else {
    PoolParams<float> pf{(const float*)k, pd.BH, pd.N, pd.C, pd.D, pool, pd.lv, summary, variance};
    hipLaunchKernelGGL(pool_leaf_kernel<float>, dim3((unsigned)leaves), dim3(pd.D), 0, st, pf);
  }
  hipError_t e = hipGetLastError();
  for (int l = 1; l < pd.lv.n_levels && e == hipSuccess; ++l) {
    hipLaunchKernelGGL(pool_level_kernel, dim3((unsigned)((long long)pd.BH * pd.lv.n[l])), dim3(pd.D), 0, st, pb, l);
    e = hipGetLastError();
  }
  return e;
}

// ------------------------------------------------------------------------------------------ the walk
constexpr int kVariantMaxCand = kVariantLdsCand;

template <typename T>
struct VariantParams {
  const T* q;
  const T* k;
  const float* summary;
  const float* variance;
  int B, Hq, Hkv, G, N, K, score, budget, start;
  float scale;
  Levels lv;
  int* sel;
};

// Order-preserving 64-bit key: larger = higher score; equal scores order by the lower node index.
__device__ __forceinline__ unsigned long long variant_key(float v, int j) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (0xffffffffu - (uint32_t)j);
}

template <typename T, int D, int C>
__global__ __launch_bounds__(64) void variant_walk_kernel(VariantParams<T> p) {
  constexpr int LOG2C = C == 64 ? 6 : 5;
  __shared__ float s_q[16][D];                 // the group's queries (fp32)
  __shared__ int s_cand[kVariantMaxCand];      // this level's candidates (ascending)
  __shared__ float s_sc[kVariantMaxCand];      // their scores
  __shared__ int s_kept[kVariantMaxCand];      // the kept nodes of the level above (ascending)
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  const long long u = blockIdx.x;
  const long long bh = u / p.N;
  const int i = (int)(u % p.N);
  const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
  const long long qrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.N + i;
  for (int x = lane; x < p.G * D; x += 64)
    s_q[x / D][x % D] = to_f32<T>(p.q[(qrow0 + (long long)(x / D) * p.N) * D + x % D]);
  Frag<T> qf[D / 32];  // MFMA columns = heads, for the exact leaf LSE
  const bool hv = r16 < p.G;
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    if (hv)
      qf[s].load(p.q + (qrow0 + (long long)r16 * p.N) * D + 32 * s + 8 * grp);
    else
      qf[s].zero();
  }
  __syncthreads();
  const float* srow = p.summary + bh * p.lv.nodes * D;
  const float* vrow = p.variance ? p.variance + bh * p.lv.nodes * D : nullptr;
  const T* kbh = p.k + bh * (long long)p.N * D;
  int n_kept = 0;
  for (int l = p.start; l >= 0; --l) {
    const int e_l = min(p.lv.n[l], (i >> (LOG2C + l)) + 1);  // eligible nodes of level l
    // candidates, ascending
    int n_cand = 0;
    if (l == p.start) {
      for (int x = lane; x < e_l; x += 64) s_cand[x] = x;
      n_cand = e_l;
    } else {
      for (int x0 = 0; x0 < n_kept; x0 += 32) {
        // lane pair (2 t, 2 t + 1) = the two children of kept entry x0 + t
        const int x = x0 + (lane >> 1);
        const int c = x < n_kept ? 2 * s_kept[x] + (lane & 1) : 0;
        const bool ok = x < n_kept && c < e_l;
        const unsigned long long m = __ballot(ok);
        if (ok) s_cand[n_cand + __popcll(m & ((1ull << lane) - 1ull))] = c;
        n_cand += __popcll(m);
      }
    }
    __syncthreads();
    const int Kl = p.budget == 0 ? p.K : (int)min((long long)p.lv.n[l], (long long)p.K << l);
    if (n_cand <= Kl) {
      for (int x = lane; x < n_cand; x += 64) s_kept[x] = s_cand[x];
      n_kept = n_cand;
      __syncthreads();
      continue;
    }
    // scores
    if (p.score == 0 && l == 0) {
      // exact leaf LSE: one leaf-pair tile per distinct parent of the (ascending) candidates
      for (int x = 0; x < n_cand;) {
        const int par = s_cand[x] >> 1;
        Frag<T> kf[C / 8][D / 32];
        load_leaf_pair<T, D, C>(kbh, 2LL * par * C, p.N, kf);
        float l0, l1;
        leaf_pair_lse<T, D, C>(kf, qf, 2LL * par * C, i, p.scale, l0, l1);
        float sum0 = 0.f, sum1 = 0.f;  // heads in index order
        for (int h = 0; h < p.G; ++h) {
          sum0 += readlane(l0, h);
          sum1 += readlane(l1, h);
        }
        for (; x < n_cand && (s_cand[x] >> 1) == par; ++x)
          if (lane == 0) s_sc[x] = (s_cand[x] & 1) ? sum1 : sum0;
        __syncthreads();
      }
    } else {
      for (int x = lane; x < n_cand; x += 64) {
        const int c = s_cand[x];
        float sc = 0.f;
        if (p.score == 0) {
          // LSE over the eligible children (level l - 1) of scale * q . summary(child)
          const int e_child = min(p.lv.n[l - 1], (i >> (LOG2C + l - 1)) + 1);
          const int ch0 = 2 * c, ch1 = 2 * c + 1;
          const bool two = ch1 < e_child;
          const float* a = srow + (p.lv.off[l - 1] + ch0) * D;
          const float* bb = srow + (p.lv.off[l - 1] + (two ? ch1 : ch0)) * D;
          for (int h = 0; h < p.G; ++h) {
            float d0 = 0.f, d1 = 0.f;
            for (int e = 0; e < D; ++e) {
              d0 = fmaf(s_q[h][e], a[e], d0);
              d1 = fmaf(s_q[h][e], bb[e], d1);
            }
            const float x0 = p.scale * d0, x1 = p.scale * d1;
            sc += two ? lse2(x0, x1) : x0;
          }
        } else {
          const float* a = srow + (p.lv.off[l] + c) * D;
          const float* v = vrow ? vrow + (p.lv.off[l] + c) * D : nullptr;
          for (int h = 0; h < p.G; ++h) {
            float d0 = 0.f, d2 = 0.f;
            for (int e = 0; e < D; ++e) {
              d0 = fmaf(s_q[h][e], a[e], d0);
              if (p.score == 2) d2 = fmaf(s_q[h][e] * s_q[h][e], v[e], d2);
            }
            sc += p.scale * d0 + (p.score == 2 ? 0.5f * p.scale * p.scale * d2 : 0.f);
          }
        }
        s_sc[x] = sc;
      }
      __syncthreads();
    }
    // the Kl-th largest key, bit by bit from the top
    unsigned long long t = 0ull;
    for (int bit = 63; bit >= 0; --bit) {
      const unsigned long long c = t | (1ull << bit);
      int cnt = 0;
      for (int x = lane; x < n_cand; x += 64) cnt += variant_key(s_sc[x], s_cand[x]) >= c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o);
      if (cnt >= Kl) t = c;
    }
    // kept = the candidates at or above it, in ascending order
    n_kept = 0;
    for (int x0 = 0; x0 < n_cand; x0 += 64) {
      const int x = x0 + lane;
      const bool keep = x < n_cand && variant_key(s_sc[x], s_cand[x]) >= t;
      const unsigned long long m = __ballot(keep);
      if (keep) s_kept[n_kept + __popcll(m & ((1ull << lane) - 1ull))] = s_cand[x];
      n_kept += __popcll(m);
    }
    __syncthreads();
  }
  if (lane < p.K) p.sel[u * p.K + lane] = lane < n_kept ? s_kept[lane] : -1;
}

template <typename T, int D, int C>
static hipError_t variant_t(const SelDims& sd, int score, int budget, int start, const void* q, const void* k,
                            const float* summary, const float* variance, int* sel, hipStream_t st) {
  VariantParams<T> p;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.summary = summary;
  p.variance = variance;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.score = score;
  p.budget = budget;
  p.start = start;
  p.scale = sd.scale;
  p.lv = sd.lv;
  p.sel = sel;
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  hipLaunchKernelGGL((variant_walk_kernel<T, D, C>), dim3((unsigned)U), dim3(64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_variant(const SelDims& sd, int score, int budget, int start, const void* q, const void* k,
                          const float* summary, const float* variance, int* sel, hipStream_t st) {
#define PISA_VAR(T, D, C) return variant_t<T, D, C>(sd, score, budget, start, q, k, summary, variance, sel, st)
  if (sd.bf16) {
    if (sd.D == 128) {
      if (sd.C == 64) PISA_VAR(uint16_t, 128, 64);
      PISA_VAR(uint16_t, 128, 32);
    }
    if (sd.C == 64) PISA_VAR(uint16_t, 64, 64);
    PISA_VAR(uint16_t, 64, 32);
  }
  if (sd.D == 128) {
    if (sd.C == 64) PISA_VAR(float, 128, 64);
    PISA_VAR(float, 128, 32);
  }
  if (sd.C == 64) PISA_VAR(float, 64, 64);
  PISA_VAR(float, 64, 32);
#undef PISA_VAR
}

}  // namespace pisa
