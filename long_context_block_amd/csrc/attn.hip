// Block-sparse attention over the selected leaf blocks ("PISA：log-linear 复杂度的金字塔稀疏注意力"
// explainer, 核心方法 §7: attention runs on the selected finest blocks only; the softmax normalises
// over the selected tokens).
//
// Leaf-major schedule. The (unit, slot) pairs are bucketed by selected leaf (regroup). A wave task is
// a run of 64 sorted pairs; for each bucket in it the wave loads the leaf's K tile into registers and
// its V tile transposed through LDS once, then runs tiles of 16/G units x G heads:
//   S = K q^T (MFMA), masked to t <= i; per column m = max, p = exp(s (x - m)), l = sum p;
//   O^T = V^T P (MFMA, P in the input type) ; partial = O / l, lse = s m + ln l.
// The K tile rows are permuted so that after the first MFMA each lane group holds 8 consecutive
// tokens per 32-token step, which is exactly the B operand the second MFMA needs (no shuffle).
// attn_merge combines a unit's K partials with weights exp(lse_k - LSE), LSE = LSE_k lse_k.
#include "attn_tiles.hpp"
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

template <typename T>
struct AttnParams {
  const T* q;
  const T* k;
  const T* v;
  const int* sel;
  const uint32_t* pairs;
  const int* total;
  int B, Hq, Hkv, G, N, K, tasks, chunk_log2;
  float scale;
  T* part;         // [U, K, G, D]
  float* part_lse; // [U, K, G]
};

constexpr int kAttnTask = 256;

template <typename T, int D, int C>
__global__ __launch_bounds__(256) void attn_leaf_kernel(AttnParams<T> p) {
  constexpr int MS = C / 16;  // M-tiles of S
  constexpr int KS = C / 32;  // k steps of the PV product
  constexpr int MO = D / 16;  // M-tiles of O^T
  constexpr int VT_LD = C + 8;
  __shared__ __align__(16) uint16_t s_vt[(sizeof(T) == 2) ? 4 : 1][D][VT_LD];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int task = xcd_logical_block(gridDim.x) * 4 + wave;
  const long long total = *p.total;
  const long long pos0 = (long long)task * kAttnTask;
  if (task >= p.tasks || pos0 >= total) return;
  const int tile_units = 16 / p.G;
  PairRun run;
  run.base = pos0;
  run.end = pos0 + kAttnTask < total ? pos0 + kAttnTask : total;
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
                                   p.sel[u * p.K + (run.pr[w] & 31)]
                             : -1;
  }
  long long pos = pos0;
  while (pos < run.end) {
    const uint32_t pr0 = run.pair(pos);
    const long long u0 = readlane((int)(pr0 >> 5), 0);
    const long long bh = u0 / p.N;
    const int leaf = p.sel[u0 * p.K + (readlane((int)pr0, 0) & 31)];
    const long long seg = run.run_end(pos, (bh * nch + ((u0 % p.N) >> p.chunk_log2)) * (1LL << 32) + leaf);
    const long long t0 = (long long)leaf * C;
    const T* kbh = p.k + bh * (long long)p.N * D;
    const T* vbh = p.v + bh * (long long)p.N * D;
    Frag<T> kf[MS][D / 32];
    load_attn_k<T, D, C>(kbh, t0, p.N, kf);
    Frag<T> vf[MO][KS];
    load_attn_vt<T, D, C>(vbh, t0, p.N, s_vt[(sizeof(T) == 2) ? wave : 0], vf);
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    const int h = r16 % p.G;
    const T* qhead = p.q + (((long long)b * p.Hq + (long long)r * p.G + h) * p.N) * D + 8 * grp;
    const long long ubase = bh * p.N;
    struct Tile {
      Frag<T> qf[D / 32];
      long long u;
      int slot;
      bool valid;
    };
    auto fetch = [&](Tile& t, long long tp) {
      const long long pi = tp + r16 / p.G;
      t.valid = pi < seg;
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
    auto attend = [&](const Tile& cur) {
      Frag<T> qf[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) qf[s] = cur.qf[s];
      const long long uc = cur.u;
      const int slot = cur.slot;
      const bool cv = cur.valid;
      const long long ic = cv ? uc - ubase : -1;
      f32x4 oacc[MO];
      float lse, inv;
      attend_tile<T, D, C>(kf, vf, qf, t0, ic, p.scale, oacc, lse, inv);
      if (cv) {
        const long long prow = (uc * p.K + slot) * p.G + h;
        T* dst = p.part + prow * D;
#pragma unroll
        for (int mt = 0; mt < MO; ++mt) {
          const int n0 = 16 * mt + 4 * grp;
          if constexpr (sizeof(T) == 2) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16(oacc[mt][0] * inv) | ((uint32_t)f32_to_bf16(oacc[mt][1] * inv) << 16);
            w.y = (uint32_t)f32_to_bf16(oacc[mt][2] * inv) | ((uint32_t)f32_to_bf16(oacc[mt][3] * inv) << 16);
            *reinterpret_cast<uint2*>((uint16_t*)dst + n0) = w;
          } else {
            *reinterpret_cast<float4*>((float*)dst + n0) =
                make_float4(oacc[mt][0] * inv, oacc[mt][1] * inv, oacc[mt][2] * inv, oacc[mt][3] * inv);
          }
        }
        if (grp == 0) p.part_lse[prow] = lse;
      }
    };
    const long long step = tile_units;
    const long long ntiles = (seg - pos + step - 1) / step;
    // ring of R tiles: the query fragments of tile t+R are requested as tile t finishes
    // (bf16 tiles are small enough for R = 4 without spilling; fp32 keeps R = 2)
    constexpr int R = sizeof(T) == 2 ? 4 : 2;
    Tile X[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < ntiles) fetch(X[r], pos + r * step);
    for (long long t = 0; t < ntiles; t += R) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (t + r < ntiles) {
          attend(X[r]);
          if (t + r + R < ntiles) fetch(X[r], pos + (t + r + R) * step);
        }
      }
    }
    pos = seg;
  }
}

template <typename T>
struct MergeParams {
  const int* sel;
  const T* part;
  const float* part_lse;
  int B, Hq, Hkv, G, N, K;
  T* o;
  float* o_lse;
};

// One wave per unit; lane e covers output columns e and e + 64 (D = 128) or e (D = 64).
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams<T> p) {
  constexpr int PER = D / 64;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const long long U = (long long)p.B * p.Hkv * p.N;
  const long long u = (long long)xcd_logical_block(gridDim.x) * 4 + wave;
  if (u >= U) return;
  const long long bh = u / p.N, i = u % p.N;
  const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
  const bool has = lane < p.K && p.sel[u * p.K + lane] >= 0;
  const int nsel = __popcll(__ballot(has));
  for (int h = 0; h < p.G; ++h) {
    const float pl = has ? p.part_lse[(u * p.K + lane) * p.G + h] : kNegInf;
    float m = pl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float w = has ? fast_exp2((pl - m) * kLog2e) : 0.f;
    float ws = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) ws += __shfl_xor(ws, o);
    const float lse = m + kLn2 * fast_log2(ws);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    for (int kk = 0; kk < nsel; ++kk) {
      const float wk = readlane(w, kk) / ws;
      const T* src = p.part + ((u * p.K + kk) * p.G + h) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += wk * to_f32<T>(src[lane + 64 * e]);
    }
    const long long orow = ((long long)b * p.Hq + (long long)r * p.G + h) * p.N + i;
#pragma unroll
    for (int e = 0; e < PER; ++e) p.o[orow * D + lane + 64 * e] = from_f32<T>(acc[e]);
    if (p.o_lse && lane == 0) p.o_lse[orow] = lse;
  }
}

// ------------------------------------------------------------------------------------------ launchers
template <typename T, int D, int C>
static hipError_t attn_leaf_t(const SelDims& sd, const void* q, const void* k, const void* v, const int* sel,
                              const uint32_t* pairs, const int* total, void* part, float* part_lse, hipStream_t st) {
  AttnParams<T> p;
  p.q = (const T*)q;
  p.k = (const T*)k;
  p.v = (const T*)v;
  p.sel = sel;
  p.pairs = pairs;
  p.total = total;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.chunk_log2 = sd.chunk_log2;
  p.scale = sd.scale;
  p.part = (T*)part;
  p.part_lse = part_lse;
  const long long max_pairs = (long long)sd.B * sd.Hkv * sd.N * sd.K;
  const long long tasks = (max_pairs + kAttnTask - 1) / kAttnTask;
  p.tasks = (int)tasks;
  hipLaunchKernelGGL((attn_leaf_kernel<T, D, C>), dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_leaf(const SelDims& sd, const void* q, const void* k, const void* v, const int* sel,
                            const uint32_t* pairs, const int* total, void* part, float* part_lse, hipStream_t st) {
#define PISA_ATTN(T, D, C) return attn_leaf_t<T, D, C>(sd, q, k, v, sel, pairs, total, part, part_lse, st)
  if (sd.bf16) {
    if (sd.D == 128) {
      if (sd.C == 64) PISA_ATTN(uint16_t, 128, 64);
      PISA_ATTN(uint16_t, 128, 32);
    }
    if (sd.C == 64) PISA_ATTN(uint16_t, 64, 64);
    PISA_ATTN(uint16_t, 64, 32);
  }
  if (sd.D == 128) {
    if (sd.C == 64) PISA_ATTN(float, 128, 64);
    PISA_ATTN(float, 128, 32);
  }
  if (sd.C == 64) PISA_ATTN(float, 64, 64);
  PISA_ATTN(float, 64, 32);
#undef PISA_ATTN
}

template <typename T, int D>
static hipError_t merge_t(const SelDims& sd, const int* sel, const void* part, const float* part_lse, void* o,
                          float* o_lse, hipStream_t st) {
  MergeParams<T> p;
  p.sel = sel;
  p.part = (const T*)part;
  p.part_lse = part_lse;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.o = (T*)o;
  p.o_lse = o_lse;
  const long long U = (long long)sd.B * sd.Hkv * sd.N;
  hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3((unsigned)((U + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const SelDims& sd, const int* sel, const void* part, const float* part_lse, void* o,
                             float* o_lse, hipStream_t st) {
  if (sd.bf16) return sd.D == 128 ? merge_t<uint16_t, 128>(sd, sel, part, part_lse, o, o_lse, st)
                                  : merge_t<uint16_t, 64>(sd, sel, part, part_lse, o, o_lse, st);
  return sd.D == 128 ? merge_t<float, 128>(sd, sel, part, part_lse, o, o_lse, st)
                     : merge_t<float, 64>(sd, sel, part, part_lse, o, o_lse, st);
}

}  // namespace pisa
