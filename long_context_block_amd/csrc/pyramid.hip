// Mean-pooled key pyramid ("Block Sparse Attention with Log-Linear Complexity" digest, 方法关键点,
// pyramid bullet: leaf blocks of C tokens, mean pooling upward with merge factor 2, O(log N) levels).
//
// Stage 1 (pool_subtree): one work-group per (KV head, run of LB = 2048/d leaves). Thread (leaf,
// 8-column chunk) sums its leaf's C keys in fp32 (four interleaved partial sums), then the work-group builds levels
// 1..log2(LB) of its subtree in LDS. Stage 2 (pool_upper): one work-group per KV head builds the
// remaining levels from the stage-1 roots. A parent's mean is the token-weighted mean of its
// children's means, (c1 m1 + c2 m2) / (c1 + c2), which is the mean of the raw keys in its span; with
// full children it is (m1 + m2) / 2 rounded once. Node token counts are computed from the span.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

__device__ __forceinline__ int node_count(long long len, int span_log2_tokens_unused, long long j, long long span) {
  long long lo = j * span;
  long long c = len - lo;
  return c <= 0 ? 0 : (c >= span ? (int)span : (int)c);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_subtree_kernel(const T* __restrict__ k, int N, int nsub, Levels lv, int C,
                                                           LensArg lens, int top_level, float* __restrict__ mean,
                                                           float* __restrict__ sum) {
  constexpr int CH = D / 8;       // 8-column chunks per row
  constexpr int LB = 256 / CH;    // leaves per work-group
  __shared__ float s_mean[LB][D];
  __shared__ float s_sum[LB][D];
  const int bh = blockIdx.x / nsub;
  const int sub = blockIdx.x % nsub;
  const int b = bh / lens.hkv;
  const long long len = lens.has ? lens.len[b] : N;
  const int lam = threadIdx.x / CH;
  const int ch = threadIdx.x % CH;
  const long long head_row = (long long)bh * lv.nodes;
  // ---- leaves
  {
    const long long j = (long long)sub * LB + lam;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    int cnt = 0;
    if (j < lv.n[0]) {
      cnt = node_count(len, 0, j, C);
      const T* src = k + ((long long)bh * N + j * C) * D + ch * 8;
      auto add = [&](float (&a)[8], const Frag<T>& f) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] += f.get(e);
        } else {
          a[0] += f.a.x; a[1] += f.a.y; a[2] += f.a.z; a[3] += f.a.w;
          a[4] += f.b.x; a[5] += f.b.y; a[6] += f.b.z; a[7] += f.b.w;
        }
      };
      // four partial sums over tokens t = 4 u + w (w = 0..3), so four loads are in flight per thread;
      // combined as (p0 + p1) + (p2 + p3)
      float part[3][8];
#pragma unroll
      for (int w = 0; w < 3; ++w)
#pragma unroll
        for (int e = 0; e < 8; ++e) part[w][e] = 0.f;
      // sixteen tokens per step while they last (sixteen loads in flight), added to the same four
      // partial sums in the same order as the steps of four below
      const int c16 = cnt & ~15;
      for (int t = 0; t < c16; t += 16) {
        Frag<T> f[16];
#pragma unroll
        for (int x = 0; x < 16; ++x) f[x].load(src + (long long)(t + x) * D);
#pragma unroll
        for (int x = 0; x < 16; x += 4) {
          add(acc, f[x]);
          add(part[0], f[x + 1]);
          add(part[1], f[x + 2]);
          add(part[2], f[x + 3]);
        }
      }
      const int c4 = cnt & ~3;
      for (int t = c16; t < c4; t += 4) {
        Frag<T> f0, f1, f2, f3;
        f0.load(src + (long long)t * D);
        f1.load(src + (long long)(t + 1) * D);
        f2.load(src + (long long)(t + 2) * D);
        f3.load(src + (long long)(t + 3) * D);
        add(acc, f0);
        add(part[0], f1);
        add(part[1], f2);
        add(part[2], f3);
      }
      for (int t = c4; t < cnt; ++t) {
        Frag<T> f;
        f.load(src + (long long)t * D);
        add(acc, f);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = (acc[e] + part[0][e]) + (part[1][e] + part[2][e]);
      const float inv = cnt > 0 ? 1.f / (float)cnt : 0.f;
      float* mrow = mean + (head_row + lv.off[0] + j) * D + ch * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) mrow[e] = cnt > 0 ? acc[e] / (float)cnt : 0.f;
      (void)inv;
      if (sum) {
        float* srow = sum + (head_row + lv.off[0] + j) * D + ch * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) srow[e] = acc[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      s_mean[lam][ch * 8 + e] = cnt > 0 ? acc[e] / (float)cnt : 0.f;
      s_sum[lam][ch * 8 + e] = acc[e];
    }
  }
  __syncthreads();
  // ---- levels inside the subtree
  int nloc = LB;
  for (int l = 1; l <= top_level; ++l) {
    nloc >>= 1;
    const long long span = (long long)C << l;
    const long long cspan = (long long)C << (l - 1);
    float pm[8], ps[8];
    long long j = -1;
    if (lam < nloc) {
      j = (long long)sub * nloc + lam;
      const long long c0 = 2 * j, c1 = 2 * j + 1;
      const float w0 = (float)node_count(len, 0, c0, cspan);
      const float w1 = (float)node_count(len, 0, c1, cspan);
      const float wt = w0 + w1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float m0 = s_mean[2 * lam][ch * 8 + e], m1 = s_mean[2 * lam + 1][ch * 8 + e];
        pm[e] = wt > 0.f ? (w0 * m0 + w1 * m1) / wt : 0.f;
        ps[e] = s_sum[2 * lam][ch * 8 + e] + s_sum[2 * lam + 1][ch * 8 + e];
      }
      (void)span;
    }
    __syncthreads();
    if (lam < nloc) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_mean[lam][ch * 8 + e] = pm[e];
        s_sum[lam][ch * 8 + e] = ps[e];
      }
      if (j < lv.n[l]) {
        float* mrow = mean + (head_row + lv.off[l] + j) * D + ch * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) mrow[e] = pm[e];
        if (sum) {
          float* srow = sum + (head_row + lv.off[l] + j) * D + ch * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) srow[e] = ps[e];
        }
      }
    }
    __syncthreads();
  }
}

// Levels first_level .. n_levels-1 of each KV head, from the level below (written earlier).
template <int D>
__global__ __launch_bounds__(256) void pool_upper_kernel(int first_level, Levels lv, int C, LensArg lens, int N,
                                                         float* __restrict__ mean, float* __restrict__ sum) {
  constexpr int CH = D / 8;
  const int bh = blockIdx.x;
  const int b = bh / lens.hkv;
  const long long len = lens.has ? lens.len[b] : N;
  const long long head_row = (long long)bh * lv.nodes;
  for (int l = first_level; l < lv.n_levels; ++l) {
    const long long cspan = (long long)C << (l - 1);
    const int items = lv.n[l] * CH;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
      const int j = it / CH, ch = it % CH;
      const long long c0 = 2LL * j, c1 = 2LL * j + 1;
      const bool has1 = c1 < lv.n[l - 1];
      const float w0 = (float)node_count(len, 0, c0, cspan);
      const float w1 = has1 ? (float)node_count(len, 0, c1, cspan) : 0.f;
      const float wt = w0 + w1;
      const float* m0 = mean + (head_row + lv.off[l - 1] + c0) * D + ch * 8;
      const float* m1 = mean + (head_row + lv.off[l - 1] + (has1 ? c1 : c0)) * D + ch * 8;
      float* mo = mean + (head_row + lv.off[l] + j) * D + ch * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float a = m0[e], bb = has1 ? m1[e] : 0.f;
        mo[e] = wt > 0.f ? (w0 * a + w1 * bb) / wt : 0.f;
      }
      if (sum) {
        const float* s0 = sum + (head_row + lv.off[l - 1] + c0) * D + ch * 8;
        const float* s1 = sum + (head_row + lv.off[l - 1] + (has1 ? c1 : c0)) * D + ch * 8;
        float* so = sum + (head_row + lv.off[l] + j) * D + ch * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) so[e] = s0[e] + (has1 ? s1[e] : 0.f);
      }
    }
    __syncthreads();
  }
}

// The same levels when no sums are kept and the first input level has at most kUpperLdsRows nodes:
// that level's means are read into LDS once and every level above is built there (two barriers per
// level instead of a global round trip), each level's means also written out. Same arithmetic per
// node as pool_upper_kernel.
constexpr int kUpperLdsRows = 256;
template <int D>
__global__ __launch_bounds__(256) void pool_upper_lds_kernel(int first_level, Levels lv, int C, LensArg lens, int N,
                                                             float* __restrict__ mean) {
  constexpr int CH = D / 8;
  __shared__ __align__(16) float s_m[kUpperLdsRows][D];
  const int bh = blockIdx.x;
  const int b = bh / lens.hkv;
  const long long len = lens.has ? lens.len[b] : N;
  const long long head_row = (long long)bh * lv.nodes;
  {
    const int n_in = lv.n[first_level - 1];
    const float* src = mean + (head_row + lv.off[first_level - 1]) * D;
    for (int x = threadIdx.x; x < n_in * (D / 4); x += blockDim.x)
      *reinterpret_cast<float4*>(&s_m[x / (D / 4)][4 * (x % (D / 4))]) = *reinterpret_cast<const float4*>(src + 4 * x);
  }
  __syncthreads();
  for (int l = first_level; l < lv.n_levels; ++l) {
    const long long cspan = (long long)C << (l - 1);
    const int items = lv.n[l] * CH;
    constexpr int IPT = (kUpperLdsRows / 2) * CH / 256;  // items per thread, at most
    float res[IPT > 0 ? IPT : 1][8];
#pragma unroll
    for (int q = 0; q < (IPT > 0 ? IPT : 1); ++q) {
      const int it = threadIdx.x + 256 * q;
      if (it < items) {
        const int j = it / CH, ch = it % CH;
        const long long c0 = 2LL * j, c1 = 2LL * j + 1;
        const bool has1 = c1 < lv.n[l - 1];
        const float w0 = (float)node_count(len, 0, c0, cspan);
        const float w1 = has1 ? (float)node_count(len, 0, c1, cspan) : 0.f;
        const float wt = w0 + w1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float a = s_m[c0][ch * 8 + e], bb = has1 ? s_m[has1 ? c1 : c0][ch * 8 + e] : 0.f;
          res[q][e] = wt > 0.f ? (w0 * a + w1 * bb) / wt : 0.f;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < (IPT > 0 ? IPT : 1); ++q) {
      const int it = threadIdx.x + 256 * q;
      if (it < items) {
        const int j = it / CH, ch = it % CH;
        float* mo = mean + (head_row + lv.off[l] + j) * D + ch * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s_m[j][ch * 8 + e] = res[q][e];
          mo[e] = res[q][e];
        }
      }
    }
    __syncthreads();
  }
}

// fp32 means -> bf16 hi and lo planes: row (head_row + node) holds hi[d] then lo[d], with
// hi = rne(m) and lo = rne(m - hi), so hi + lo carries about 16 significant bits of m.
__global__ __launch_bounds__(256) void split_hilo_kernel(const float* __restrict__ mean, long long rows, int D,
                                                        uint16_t* __restrict__ hilo) {
  const long long total = rows * D;
  for (long long x = (long long)blockIdx.x * blockDim.x + threadIdx.x; x < total; x += (long long)gridDim.x * blockDim.x) {
    const long long row = x / D;
    const int c = (int)(x % D);
    const float m = mean[x];
    const uint16_t hi = f32_to_bf16(m);
    const uint16_t lo = f32_to_bf16(m - bf16_to_f32(hi));
    hilo[row * 2 * D + c] = hi;
    hilo[row * 2 * D + D + c] = lo;
  }
}

// Routing planes. Per KV head an exponent e (max |mean| 2^e in [2^14, 2^15), from 64 partial maxima);
// per routing row the fp16 planes hi = rne(2^e mean), lo = rne(2^e mean - hi) and the hi-plane score
// bound b = 2^-e (1.05 |lo| + 2^-16 |2^e mean|): for any q, |q . (hi + lo) - q . hi| = |q . lo| <=
// |q| |lo| (Cauchy-Schwarz); the 2^-16 term covers the fp32 accumulation of the dot products (each
// order of summation errs by under 2^-17 |q| |2^e mean|) and the 1.05 the rounding of the norms. 2^-e
// returns b to the units of the unscaled means. Node (l, j) is routing row roff[l] + j; rows are stored
// in the quad-interleaved layout of route_plane_chunk (rows past a level's nodes are zero, bound 0).
// Partial maxima of |mean|: kMaxParts work-groups per KV head, each over a contiguous slice.
constexpr int kMaxParts = 64;
__global__ __launch_bounds__(256) void head_max_kernel(const float* __restrict__ mean, long long rows_per_head, int D,
                                                      float* __restrict__ part_max) {
  __shared__ float s_m[4];
  const int bh = blockIdx.x / kMaxParts, part = blockIdx.x % kMaxParts;
  const long long n = rows_per_head * D;
  const long long lo = n * part / kMaxParts, hi = n * (part + 1) / kMaxParts;
  const float* m = mean + (long long)bh * n;
  float mx = 0.f;
  for (long long x = lo + threadIdx.x; x < hi; x += 256) mx = fmaxf(mx, fabsf(m[x]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) part_max[blockIdx.x] = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
}

// One wave per routing row.
__global__ __launch_bounds__(256) void split_f16_kernel(const float* __restrict__ mean, long long heads, Levels lv,
                                                       int D, const float* __restrict__ part_max,
                                                       int* __restrict__ hexp, uint16_t* __restrict__ hilo,
                                                       float* __restrict__ bound) {
  const long long rrow = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rrow >= heads * lv.rnodes) return;
  const int lane = threadIdx.x & 63;
  const long long bh = rrow / lv.rnodes;
  const int R = (int)(rrow - bh * lv.rnodes);
  // the level holding routing row R, and the node's index in it (past the level's nodes: padding)
  int l = 0;
  while (l + 1 < lv.n_levels && R >= lv.roff[l + 1]) ++l;
  const int j = R - (int)lv.roff[l];
  const bool node = j < lv.n[l];
  static_assert(kMaxParts == 64, "one partial per lane");
  float mx = part_max[bh * kMaxParts + lane];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const int e = f16_range_exp(mx);
  if (lane == 0 && R == 0) hexp[bh] = e;
  uint16_t* head = hilo + bh * lv.rnodes * 2 * D;
  const float* mrow = mean + (bh * lv.nodes + lv.off[l] + (node ? j : 0)) * D;
  float sv = 0.f, sl = 0.f;
  for (int c = lane; c < D; c += 64) {
    const float v = node ? ldexpf(mrow[c], e) : 0.f;
    const uint16_t hb = f32_to_f16_bits(v);
    const uint16_t lb = f32_to_f16_bits(v - f16_bits_to_f32(hb));
    route_plane_chunk<uint16_t>(head, R, 0, c >> 3, D)[c & 7] = hb;
    route_plane_chunk<uint16_t>(head, R, 1, c >> 3, D)[c & 7] = lb;
    const float lf = f16_bits_to_f32(lb);
    sv += v * v;
    sl += lf * lf;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    sv += __shfl_xor(sv, o);
    sl += __shfl_xor(sl, o);
  }
  if (lane == 0) bound[rrow] = node ? ldexpf(1.05f * sqrtf(sl) + 1.52587890625e-05f * sqrtf(sv), -e) : 0.f;
}

// ------------------------------------------------------------------------------------------ host
template <typename T, int D>
static hipError_t launch_pool_t(const T* k, const PyrDims& pd, LensArg lens, int max_level, float* mean, float* sum,
                                hipStream_t st) {
  constexpr int LB = 256 / (D / 8);
  int sub_top = 0;
  while ((1 << (sub_top + 1)) <= LB && sub_top + 1 <= max_level) ++sub_top;
  const int nsub = (pd.lv.n[0] + LB - 1) / LB;
  const int grid = pd.BH * nsub;
  hipLaunchKernelGGL((pool_subtree_kernel<T, D>), dim3(grid), dim3(256), 0, st, k, pd.N, nsub, pd.lv, pd.C, lens,
                     sub_top, mean, sum);
  if (max_level > sub_top) {
    if (!sum && pd.lv.n[sub_top] <= kUpperLdsRows)
      hipLaunchKernelGGL((pool_upper_lds_kernel<D>), dim3(pd.BH), dim3(256), 0, st, sub_top + 1, pd.lv, pd.C, lens,
                         pd.N, mean);
    else
      hipLaunchKernelGGL((pool_upper_kernel<D>), dim3(pd.BH), dim3(256), 0, st, sub_top + 1, pd.lv, pd.C, lens,
                         pd.N, mean, sum);
  }
  return hipGetLastError();
}

hipError_t launch_pool(const void* k, bool bf16, const PyrDims& pd, LensArg lens, int max_level, float* mean, float* sum,
                       hipStream_t st) {
  if (bf16) {
    if (pd.D == 128) return launch_pool_t<uint16_t, 128>((const uint16_t*)k, pd, lens, max_level, mean, sum, st);
    return launch_pool_t<uint16_t, 64>((const uint16_t*)k, pd, lens, max_level, mean, sum, st);
  }
  if (pd.D == 128) return launch_pool_t<float, 128>((const float*)k, pd, lens, max_level, mean, sum, st);
  return launch_pool_t<float, 64>((const float*)k, pd, lens, max_level, mean, sum, st);
}

hipError_t launch_route_planes(const float* mean, long long heads, const Levels& lv, int D, float* part_max,
                               int* hexp, uint16_t* hilo, float* bound, hipStream_t st) {
  hipLaunchKernelGGL(head_max_kernel, dim3((unsigned)(heads * kMaxParts)), dim3(256), 0, st, mean, lv.nodes, D,
                     part_max);
  const long long rows = heads * lv.rnodes;
  hipLaunchKernelGGL(split_f16_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, mean, heads, lv, D,
                     part_max, hexp, hilo, bound);
  return hipGetLastError();
}

hipError_t launch_split_hilo(const float* mean, long long rows, int D, uint16_t* hilo, hipStream_t st) {
  const long long total = rows * D;
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(split_hilo_kernel, dim3((unsigned)blocks), dim3(256), 0, st, mean, rows, D, hilo);
  return hipGetLastError();
}

}  // namespace pisa
