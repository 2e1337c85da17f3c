// Flat block selection of ordinary block-sparse attention, for comparison ("Block Sparse Attention
// with Log-Linear Complexity" digest, 动机: each query scores every key block, O(N^2/C)).
//
// Score of leaf j for unit (b, r, i): sum over the group's heads of s * q_h . mean_j, which equals
// s * (sum_h q_h) . mean_j, so the heads are summed first (fp32) and one dot product per (unit, leaf)
// remains. A wave owns 16 consecutive positions of one KV head (the 16 matrix columns) and streams
// the eligible leaves in 16-row M-tiles: bf16 inputs use hi/lo splits of both operands
// (hi.hi + hi.lo + lo.hi, about 16 significant bits), fp32 inputs the fp32 MFMA. Each lane keeps the
// best K of the leaves it sees (a quarter of them) by replace-the-worst; the four lists of a column
// are merged at the end by a rank count. Order: score descending, then leaf index ascending.
#include "common.hpp"
#include "internal.hpp"

namespace pisa {

template <typename T>
struct BsaParams {
  const T* q;
  const float* mean;       // [BH, n0, D] leaf means (fp32 inputs)
  const uint16_t* hilo;    // [BH, n0, 2, D] bf16 hi/lo leaf means (bf16 inputs)
  int B, Hq, Hkv, G, N, C, K, n0;
  float scale;
  int* sel;
};

__device__ __forceinline__ bool bsa_better(float s, int j, float s2, int j2) { return s > s2 || (s == s2 && j < j2); }

template <typename T, int D, int KMAX>
__global__ __launch_bounds__(256) void bsa_kernel(BsaParams<T> p) {
  __shared__ float s_sc[4][16][4 * KMAX];
  __shared__ int s_ix[4][16][4 * KMAX];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const int tiles_per_head = (p.N + 15) / 16;
  const long long task = (long long)xcd_logical_block(gridDim.x) * 4 + wave;
  if (task >= (long long)p.B * p.Hkv * tiles_per_head) return;
  const long long bh = task / tiles_per_head;
  const int i0 = (int)(task % tiles_per_head) * 16;
  const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
  const int ic = i0 + r16;  // this lane's column position
  const bool col_ok = ic < p.N;
  // summed query of the column, as B fragments
  Frag<T> qhi[D / 32], qlo[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (col_ok) {
      for (int h = 0; h < p.G; ++h) {
        const T* qrow = p.q + ((((long long)b * p.Hq + (long long)r * p.G + h) * p.N) + ic) * D + 32 * s + 8 * grp;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += to_f32<T>(qrow[e]);
      }
    }
    if constexpr (sizeof(T) == 2) {
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16(acc[e]);
        lo[e] = f32_to_bf16(acc[e] - bf16_to_f32(hi[e]));
      }
      Frag<uint16_t>& fh = reinterpret_cast<Frag<uint16_t>&>(qhi[s]);
      Frag<uint16_t>& fl = reinterpret_cast<Frag<uint16_t>&>(qlo[s]);
      fh.u = make_uint4(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16), hi[4] | (hi[5] << 16), hi[6] | (hi[7] << 16));
      fl.u = make_uint4(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16), lo[4] | (lo[5] << 16), lo[6] | (lo[7] << 16));
    } else {
      Frag<float>& f = reinterpret_cast<Frag<float>&>(qhi[s]);
      f.a = make_float4(acc[0], acc[1], acc[2], acc[3]);
      f.b = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
  }
  float bs[KMAX];
  int bj[KMAX];
#pragma unroll
  for (int e = 0; e < KMAX; ++e) {
    bs[e] = kNegInf;
    bj[e] = 0x7fffffff;
  }
  float ws = kNegInf;  // worst kept (score, index)
  int wj = 0x7fffffff;
  int wpos = 0;
  const int last_pos = (i0 + 15 < p.N ? i0 + 15 : p.N - 1);
  const int n_elig = last_pos / p.C + 1;
  const int MT = (n_elig + 15) / 16;
  for (int mt = 0; mt < MT; ++mt) {
    const int jr = 16 * mt + r16;  // A row (leaf) this lane loads
    const bool rv = jr < p.n0;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if constexpr (sizeof(T) == 2) {
        Frag<uint16_t> ahi, alo;
        if (rv) {
          const uint16_t* row = p.hilo + ((bh * p.n0) + jr) * 2 * D + 32 * s + 8 * grp;
          ahi.load(row);
          alo.load(row + D);
        } else {
          ahi.zero();
          alo.zero();
        }
        mma(acc, ahi, reinterpret_cast<Frag<uint16_t>&>(qhi[s]));
        mma(acc, ahi, reinterpret_cast<Frag<uint16_t>&>(qlo[s]));
        mma(acc, alo, reinterpret_cast<Frag<uint16_t>&>(qhi[s]));
      } else {
        Frag<float> a;
        if (rv)
          a.load(p.mean + ((bh * p.n0) + jr) * D + 32 * s + 8 * grp);
        else
          a.zero();
        mma(acc, a, reinterpret_cast<Frag<float>&>(qhi[s]));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int leaf = 16 * mt + 4 * grp + j;
      const bool ok = col_ok && leaf < p.n0 && (long long)leaf * p.C <= ic;
      const float sc = p.scale * acc[j];
      if (ok && bsa_better(sc, leaf, ws, wj)) {
#pragma unroll
        for (int e = 0; e < KMAX; ++e)
          if (e == wpos) {
            bs[e] = sc;
            bj[e] = leaf;
          }
        ws = kNegInf;
        wj = -1;
        wpos = 0;
        bool first = true;
#pragma unroll
        for (int e = 0; e < KMAX; ++e) {
          if (e < p.K) {
            if (first || bsa_better(ws, wj, bs[e], bj[e])) {
              ws = bs[e];
              wj = bj[e];
              wpos = e;
              first = false;
            }
          }
        }
      }
    }
  }
  // merge the 4 lane lists of each column
#pragma unroll
  for (int e = 0; e < KMAX; ++e) {
    s_sc[wave][r16][grp * KMAX + e] = e < p.K ? bs[e] : kNegInf;
    s_ix[wave][r16][grp * KMAX + e] = e < p.K ? bj[e] : 0x7fffffff;
  }
  __threadfence_block();
  constexpr int NH = (4 * KMAX + 63) / 64;  // candidates per lane
  for (int c = 0; c < 16; ++c) {
    const int pos = i0 + c;
    if (pos >= p.N) break;
    const long long u = bh * p.N + pos;
    float cs[NH];
    int cj[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int x = lane + 64 * h;
      const bool in = x < 4 * KMAX;
      cs[h] = in ? s_sc[wave][c][x] : kNegInf;
      cj[h] = in ? s_ix[wave][c][x] : 0x7fffffff;
    }
    int rank[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) rank[h] = 0;
    for (int y = 0; y < 4 * KMAX; ++y) {
      const float ys = s_sc[wave][c][y];
      const int yj = s_ix[wave][c][y];
#pragma unroll
      for (int h = 0; h < NH; ++h) rank[h] += bsa_better(ys, yj, cs[h], cj[h]);
    }
    // kept: rank < K and a real leaf. The lane lists hold disjoint leaves, so a kept leaf's output
    // position is the number of kept leaves with a smaller index: counted over the kept lanes only
    // (at most K of them, a scalar loop over the ballot bits).
    bool kp[NH];
    unsigned long long km[NH];
    int nkept = 0, opos[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      kp[h] = rank[h] < p.K && cj[h] != 0x7fffffff;
      km[h] = __ballot(kp[h]);
      nkept += __popcll(km[h]);
      opos[h] = 0;
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      unsigned long long mm = km[hh];
      while (mm) {
        const int y = __builtin_ctzll(mm);
        mm &= mm - 1ull;
        const int yj = readlane(cj[hh], y);
#pragma unroll
        for (int h = 0; h < NH; ++h) opos[h] += yj < cj[h];
      }
    }
#pragma unroll
    for (int h = 0; h < NH; ++h)
      if (kp[h]) p.sel[u * p.K + opos[h]] = cj[h];
    if (lane < p.K && lane >= nkept) p.sel[u * p.K + lane] = -1;
  }
}

template <typename T, int D, int KMAX>
static hipError_t bsa_t(const SelDims& sd, const void* q, const float* mean, const uint16_t* hilo, int* sel,
                        hipStream_t st) {
  BsaParams<T> p;
  p.q = (const T*)q;
  p.mean = mean;
  p.hilo = hilo;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.C = sd.C;
  p.K = sd.K;
  p.n0 = sd.lv.n[0];
  p.scale = sd.scale;
  p.sel = sel;
  const long long tasks = (long long)sd.B * sd.Hkv * ((sd.N + 15) / 16);
  hipLaunchKernelGGL((bsa_kernel<T, D, KMAX>), dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_bsa(const SelDims& sd, const void* q, const float* leaf_mean, const uint16_t* leaf_hilo, int* sel,
                      hipStream_t st) {
#define PISA_BSA(T, D, KM) return bsa_t<T, D, KM>(sd, q, leaf_mean, leaf_hilo, sel, st)
  if (sd.bf16) {
    if (sd.D == 128) {
      if (sd.K <= 16) PISA_BSA(uint16_t, 128, 16);
      PISA_BSA(uint16_t, 128, 32);
    }
    if (sd.K <= 16) PISA_BSA(uint16_t, 64, 16);
    PISA_BSA(uint16_t, 64, 32);
  }
  if (sd.D == 128) {
    if (sd.K <= 16) PISA_BSA(float, 128, 16);
    PISA_BSA(float, 128, 32);
  }
  if (sd.K <= 16) PISA_BSA(float, 64, 16);
  PISA_BSA(float, 64, 32);
#undef PISA_BSA
}

}  // namespace pisa
