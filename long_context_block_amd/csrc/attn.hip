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
  int B, Hq, Hkv, G, N, K, tasks;
  float scale;
  T* part;         // [U, K, G, D]
  float* part_lse; // [U, K, G]
};

constexpr int kAttnTask = 64;

// Token offset (within the leaf) of D-row 4*grp + j of M-tile m after the first MFMA.
__device__ __forceinline__ int attn_token(int m, int grp, int j) { return 32 * (m >> 1) + 8 * grp + 4 * (m & 1) + j; }

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
  long long pos = (long long)task * kAttnTask;
  if (task >= p.tasks || pos >= total) return;
  const long long end = pos + kAttnTask < total ? pos + kAttnTask : total;
  const int tile_units = 16 / p.G;
  while (pos < end) {
    const uint32_t pr = p.pairs[pos];
    const long long u = pr >> 5;
    const long long bh = u / p.N;
    const int leaf = p.sel[u * p.K + (pr & 31)];
    long long seg = end;
    for (long long base = pos; base < end; base += 64) {
      const long long x = base + lane;
      bool diff = false;
      if (x < end) {
        const uint32_t q2 = p.pairs[x];
        const long long u2 = q2 >> 5;
        diff = (u2 / p.N != bh) || (p.sel[u2 * p.K + (q2 & 31)] != leaf);
      }
      const unsigned long long m = __ballot(diff);
      if (m) {
        seg = base + __ffsll((long long)m) - 1;
        break;
      }
    }
    const long long t0 = (long long)leaf * C;
    const T* kbh = p.k + bh * (long long)p.N * D;
    const T* vbh = p.v + bh * (long long)p.N * D;
    // K tile, rows permuted (see attn_token).
    Frag<T> kf[MS][D / 32];
#pragma unroll
    for (int m = 0; m < MS; ++m) {
      const long long t = t0 + attn_token(m, r16 >> 2, r16 & 3);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        if (t < p.N)
          kf[m][s].load(kbh + t * D + (D / 4) * grp + 8 * s);
        else
          kf[m][s].zero();
      }
    }
    // V^T tile: lane (row n = 16 mt + r16, grp) needs V[32 ks + 8 grp + e][n], e = 0..7.
    Frag<T> vf[MO][KS];
    if constexpr (sizeof(T) == 2) {
      constexpr int CHR = D / 8;  // 8-element chunks per V row
#pragma unroll
      for (int it = 0; it < (C * CHR) / 64; ++it) {
        const int qd = it * 64 + lane;
        const int t = qd / CHR, c0 = (qd % CHR) * 8;
        Frag<uint16_t> f;
        if (t0 + t < p.N)
          f.load((const uint16_t*)vbh + (t0 + t) * D + c0);
        else
          f.zero();
        const uint32_t w[4] = {f.u.x, f.u.y, f.u.z, f.u.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) s_vt[wave][c0 + e][t] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
      }
      __threadfence_block();
#pragma unroll
      for (int mt = 0; mt < MO; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          vf[mt][ks].u = *reinterpret_cast<const uint4*>(&s_vt[wave][16 * mt + r16][32 * ks + 8 * grp]);
      __threadfence_block();
    } else {
#pragma unroll
      for (int mt = 0; mt < MO; ++mt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float e8[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const long long t = t0 + 32 * ks + 8 * grp + e;
            e8[e] = t < p.N ? (float)vbh[t * D + 16 * mt + r16] : 0.f;
          }
          Frag<float>& f = reinterpret_cast<Frag<float>&>(vf[mt][ks]);
          f.a = make_float4(e8[0], e8[1], e8[2], e8[3]);
          f.b = make_float4(e8[4], e8[5], e8[6], e8[7]);
        }
    }
    const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
    for (long long tp = pos; tp < seg; tp += tile_units) {
      const long long pi = tp + r16 / p.G;
      const int h = r16 % p.G;
      const bool cv = pi < seg;
      long long uc = 0, ic = -1;
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
      f32x4 sacc[MS];
#pragma unroll
      for (int m = 0; m < MS; ++m) sacc[m] = zero4();
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
#pragma unroll
        for (int m = 0; m < MS; ++m) mma(sacc[m], kf[m][s], qf[s]);
      // masked softmax statistics per column
      float mx = kNegInf;
#pragma unroll
      for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const long long t = t0 + attn_token(m, grp, j);
          const float x = t <= ic ? sacc[m][j] : kNegInf;
          sacc[m][j] = x;
          mx = fmaxf(mx, x);
        }
      mx = colgroup_max(mx);
      const bool any = mx != kNegInf;
      const float ms = any ? mx : 0.f;
      const float c2 = p.scale * kLog2e;
      float lsum = 0.f;
#pragma unroll
      for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = fast_exp2((sacc[m][j] - ms) * c2);
          sacc[m][j] = e;
          lsum += e;
        }
      lsum = colgroup_sum(lsum);
      // P as the B operand of O^T = V^T P
      Frag<T> pf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (sizeof(T) == 2) {
          const f32x4 a = sacc[2 * ks], bb = sacc[2 * ks + 1];
          Frag<uint16_t>& f = reinterpret_cast<Frag<uint16_t>&>(pf[ks]);
          f.u.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
          f.u.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
          f.u.z = (uint32_t)f32_to_bf16(bb[0]) | ((uint32_t)f32_to_bf16(bb[1]) << 16);
          f.u.w = (uint32_t)f32_to_bf16(bb[2]) | ((uint32_t)f32_to_bf16(bb[3]) << 16);
        } else {
          Frag<float>& f = reinterpret_cast<Frag<float>&>(pf[ks]);
          f.a = make_float4(sacc[2 * ks][0], sacc[2 * ks][1], sacc[2 * ks][2], sacc[2 * ks][3]);
          f.b = make_float4(sacc[2 * ks + 1][0], sacc[2 * ks + 1][1], sacc[2 * ks + 1][2], sacc[2 * ks + 1][3]);
        }
      }
      f32x4 oacc[MO];
#pragma unroll
      for (int mt = 0; mt < MO; ++mt) {
        oacc[mt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(oacc[mt], vf[mt][ks], pf[ks]);
      }
      if (cv) {
        const float inv = any ? 1.f / lsum : 0.f;
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
        if (grp == 0) p.part_lse[prow] = any ? p.scale * ms + kLn2 * fast_log2(lsum) : kNegInf;
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
