// Selection quality ("Block Sparse Attention with Log-Linear Complexity" digest, 关键实验: the block
// selection is judged by its Recall@K and by the attention mass ratio, the share of full attention's
// softmax mass that falls inside the selected blocks).
//
// flat_leaf_lse_kernel: the dense causal pass. For chosen query positions it scores EVERY leaf, not a
// bounded candidate set: per (query head, position, leaf j) the exact LSE over the leaf's tokens
// t <= i of s * q . k_t (-inf for leaves after i), and per (query head, position) the LSE of the whole
// causal row. One wave per 16 matrix columns (16 / G positions x G heads of one KV head) walks the
// leaf pairs from the start of the sequence; the per-leaf arithmetic is the selection's leaf stage
// (same tiles, same LSE code), so a leaf's value here equals the one the selection computes for it.
//
// quality_kernel: per unit, the flat exact Top-K over the head-summed leaf LSEs (score descending,
// index ascending), the recall of a given selection against it, and the selection's per-head share of
// the row's softmax mass, sum over its leaves of exp(leaf LSE - row LSE).
#include "common.hpp"
#include "internal.hpp"
#include "walk_tiles.hpp"

namespace pisa {

template <typename T>
struct FlatParams {
  const T* q;
  const T* k;
  const int* pos;  // [n_pos] query positions
  int n_pos, B, Hq, Hkv, G, N, n0, tiles;
  float scale;
  float* leaf_lse;  // [B, Hq, n_pos, n0]
  float* row_lse;   // [B, Hq, n_pos]
};

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void flat_leaf_lse_kernel(FlatParams<T> p) {
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long task = (long long)blockIdx.x * 4 + wave;  // (bh, tile of 16 / G positions)
  if (task >= (long long)p.B * p.Hkv * p.tiles) return;
  const int bh = (int)(task / p.tiles), tile = (int)(task % p.tiles);
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const int upc = 16 / p.G;
  const int pidx = tile * upc + r16 / p.G, h = r16 % p.G;
  // a column is live if its position index exists and its position lies in [0, N)
  const int ip = pidx < p.n_pos ? p.pos[pidx] : -1;
  const bool live = pidx < p.n_pos && ip >= 0 && ip < p.N;
  const int i = live ? ip : -1;
  Frag<T> qf[D / 32];
  const long long qrow = ((long long)b * p.Hq + (long long)r * p.G + h) * p.N + (live ? i : 0);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    if (live)
      qf[s].load(p.q + qrow * D + 32 * s + 8 * grp);
    else
      qf[s].zero();
  }
  // leaf pairs up to the last one any live column of the wave can see
  int imax = i;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) imax = max(imax, __shfl_xor(imax, o));
  const int npair = imax < 0 ? 0 : (imax / (2 * C)) + 1;
  const T* kbh = p.k + (long long)bh * p.N * D;
  float* out = p.leaf_lse + (((long long)b * p.Hq + (long long)r * p.G + h) * p.n_pos + (pidx < p.n_pos ? pidx : 0)) * p.n0;
  float row = kNegInf;
  for (int pr = 0; pr < npair; ++pr) {
    Frag<T> kf[C / 8][D / 32];
    load_leaf_pair<T, D, C>(kbh, 2LL * pr * C, p.N, kf);
    float l0, l1;
    leaf_pair_lse<T, D, C>(kf, qf, 2LL * pr * C, i, p.scale, l0, l1);
    row = lse2_inf(lse2_inf(row, l0), l1);
    if (grp == 0 && pidx < p.n_pos) {
      out[2 * pr] = live ? l0 : __builtin_nanf("");
      if (2 * pr + 1 < p.n0) out[2 * pr + 1] = live ? l1 : __builtin_nanf("");
    }
  }
  // leaves past the wave's last pair: after every live column's position
  if (pidx < p.n_pos)
    for (int j = 2 * npair + grp; j < p.n0; j += 4) out[j] = live ? kNegInf : __builtin_nanf("");
  if (grp == 0 && pidx < p.n_pos)
    p.row_lse[((long long)b * p.Hq + (long long)r * p.G + h) * p.n_pos + pidx] = live ? row : __builtin_nanf("");
}

struct QualityParams {
  const float* leaf_lse;
  const float* row_lse;
  const int* pos;
  const int* sel;  // [B, Hkv, N, K]
  int n_pos, B, Hq, Hkv, G, N, n0, K, C;
  int* flat_sel;   // [B, Hkv, n_pos, K]
  float* recall;   // [B, Hkv, n_pos]
  float* mass;     // [B, Hq, n_pos]
};

// Order-preserving 64-bit key of (score, leaf j): larger key = higher score, equal scores by the lower
// index. Distinct for distinct j.
__device__ __forceinline__ unsigned long long flat_key(float v, int j) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)o << 32) | (0xffffffffu - (uint32_t)j);
}

// One wave (a work-group of 64 threads) per unit (b, r, position index). The head-summed leaf LSEs of
// the eligible leaves go to LDS; the K-th largest key is found bit by bit from the top (64 passes,
// each counting the keys at or above a candidate); the flat selection is every key at or above it.
__global__ __launch_bounds__(64) void quality_kernel(QualityParams p) {
  extern __shared__ float s_f[];  // n0 head-summed leaf LSEs
  const int lane = lane_id();
  const long long u = blockIdx.x;  // (bh, pidx)
  const int bh = (int)(u / p.n_pos), pidx = (int)(u % p.n_pos);
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const int ip = p.pos[pidx];
  const bool live = ip >= 0 && ip < p.N;
  int* fsel = p.flat_sel + u * p.K;
  if (!live) {
    if (lane < p.K) fsel[lane] = -1;
    if (lane == 0) p.recall[u] = __builtin_nanf("");
    if (lane < p.G) p.mass[((long long)b * p.Hq + (long long)r * p.G + lane) * p.n_pos + pidx] = __builtin_nanf("");
    return;
  }
  const int i = ip;
  const int ne = min(p.n0, i / p.C + 1);  // eligible leaves
  const long long hrow0 = ((long long)b * p.Hq + (long long)r * p.G) * p.n_pos + pidx;  // head 0's row
  for (int j = lane; j < ne; j += 64) {
    float x = 0.f;  // heads in index order
    for (int h = 0; h < p.G; ++h) x += p.leaf_lse[(hrow0 + (long long)h * p.n_pos) * p.n0 + j];
    s_f[j] = x;
  }
  __syncthreads();
  const int kk = min(p.K, ne);
  unsigned long long t = 0ull;  // the kk-th largest key
  if (ne > p.K) {
    for (int bit = 63; bit >= 0; --bit) {
      const unsigned long long c = t | (1ull << bit);
      int cnt = 0;
      for (int j = lane; j < ne; j += 64) cnt += flat_key(s_f[j], j) >= c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o);
      if (cnt >= kk) t = c;
    }
  }
  // flat selection in ascending leaf order (every key >= t; all eligible leaves when ne <= K)
  int nout = 0;
  for (int j0 = 0; j0 < ne; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j < ne && flat_key(s_f[j], j) >= t;
    const unsigned long long m = __ballot(keep);
    const int at = nout + __popcll(m & ((1ull << lane) - 1ull));
    if (keep && at < p.K) fsel[at] = j;
    nout += __popcll(m);
  }
  if (lane >= nout && lane < p.K) fsel[lane] = -1;
  // the evaluated selection of this unit
  const int sj = lane < p.K ? p.sel[(((long long)bh * p.N) + i) * p.K + lane] : -1;
  const bool sv = sj >= 0 && sj < ne;
  const int js = sv ? sj : 0;  // an index that exists, for lanes without a selected leaf
  const bool hit = sv && flat_key(s_f[js], js) >= t;
  const int nhit = __popcll(__ballot(hit));
  if (lane == 0) p.recall[u] = (float)nhit / (float)kk;
  for (int h = 0; h < p.G; ++h) {
    const long long hrow = hrow0 + (long long)h * p.n_pos;
    const float L = p.row_lse[hrow];
    const float lj = p.leaf_lse[hrow * p.n0 + js];
    float w = sv ? fast_exp2((lj - L) * kLog2e) : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) w += __shfl_xor(w, o);
    if (lane == 0) p.mass[hrow] = w;
  }
}

// ------------------------------------------------------------------------------------------ launchers
template <typename T, int D, int C>
static hipError_t flat_t(const SelDims& sd, const void* q, const void* k, const int* pos, int n_pos, float* leaf_lse,
                         float* row_lse, hipStream_t st) {
  FlatParams<T> p;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.pos = pos;
  p.n_pos = n_pos;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.n0 = sd.lv.n[0];
  p.scale = sd.scale;
  p.leaf_lse = leaf_lse;
  p.row_lse = row_lse;
  const int upc = 16 / sd.G;
  p.tiles = (n_pos + upc - 1) / upc;
  const long long waves = (long long)sd.B * sd.Hkv * p.tiles;
  hipLaunchKernelGGL((flat_leaf_lse_kernel<T, D, C>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_flat_leaf_lse(const SelDims& sd, const void* q, const void* k, const int* pos, int n_pos,
                                float* leaf_lse, float* row_lse, hipStream_t st) {
#define PISA_FLAT(T, D, C) return flat_t<T, D, C>(sd, q, k, pos, n_pos, leaf_lse, row_lse, st)
  if (sd.bf16) {
    if (sd.D == 128) {
      if (sd.C == 64) PISA_FLAT(uint16_t, 128, 64);
      PISA_FLAT(uint16_t, 128, 32);
    }
    if (sd.C == 64) PISA_FLAT(uint16_t, 64, 64);
    PISA_FLAT(uint16_t, 64, 32);
  }
  if (sd.D == 128) {
    if (sd.C == 64) PISA_FLAT(float, 128, 64);
    PISA_FLAT(float, 128, 32);
  }
  if (sd.C == 64) PISA_FLAT(float, 64, 64);
  PISA_FLAT(float, 64, 32);
#undef PISA_FLAT
}

hipError_t launch_quality(const SelDims& sd, const float* leaf_lse, const float* row_lse, const int* pos, int n_pos,
                          const int* sel, int* flat_sel, float* recall, float* mass, hipStream_t st) {
  QualityParams p;
  p.leaf_lse = leaf_lse;
  p.row_lse = row_lse;
  p.pos = pos;
  p.sel = sel;
  p.n_pos = n_pos;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.n0 = sd.lv.n[0];
  p.K = sd.K;
  p.C = sd.C;
  p.flat_sel = flat_sel;
  p.recall = recall;
  p.mass = mass;
  const long long units = (long long)sd.B * sd.Hkv * n_pos;
  hipLaunchKernelGGL(quality_kernel, dim3((unsigned)units), dim3(64), (size_t)p.n0 * sizeof(float), st, p);
  return hipGetLastError();
}

}  // namespace pisa
