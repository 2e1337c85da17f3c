// Device tiles of block-sparse attention over one leaf (C keys) for up to 16 (unit, head) columns,
// shared by the prefill attention kernel and the fused decode step (see attn.hip for the citation).
//
// S = K q^T on MFMA with the K tile rows permuted so that, after that MFMA, lane group g holds the 8
// consecutive tokens 32 ks + 8 g .. +8 of each 32-token step: exactly the B operand of
// O^T = V^T P, so P never moves between lanes. V^T comes from a transposed copy of the V tile in LDS
// (bf16) or from direct loads (fp32).
#pragma once
#include "common.hpp"

namespace pisa {

// Token offset (within the leaf) of D-row 4*grp + j of M-tile m after the first MFMA.
__device__ __forceinline__ int attn_token(int m, int grp, int j) { return 32 * (m >> 1) + 8 * grp + 4 * (m & 1) + j; }

// K tile of the leaf starting at token t0, rows permuted (attn_token), zero past N.
template <typename T, int D, int C>
__device__ __forceinline__ void load_attn_k(const T* kbh, long long t0, long long N, Frag<T> (&kf)[C / 16][D / 32]) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
  for (int m = 0; m < C / 16; ++m) {
    const long long t = t0 + attn_token(m, r16 >> 2, r16 & 3);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (t < N)
        kf[m][s].load(kbh + t * D + 32 * s + 8 * grp);
      else
        kf[m][s].zero();
    }
  }
}

// V^T fragments: lane (row n = 16 mt + r16, grp) gets V[32 ks + 8 grp + e][n], e = 0..7. bf16 goes
// through vt, this wave's [D][C + 8] LDS scratch.
template <typename T, int D, int C>
__device__ __forceinline__ void load_attn_vt(const T* vbh, long long t0, long long N, uint16_t (*vt)[C + 8],
                                             Frag<T> (&vf)[D / 16][C / 32]) {
  constexpr int MO = D / 16, KS = C / 32;
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  if constexpr (sizeof(T) == 2) {
    constexpr int CHR = D / 8;  // 8-element chunks per V row
#pragma unroll
    for (int it = 0; it < (C * CHR) / 64; ++it) {
      const int qd = it * 64 + lane;
      const int t = qd / CHR, c0 = (qd % CHR) * 8;
      Frag<uint16_t> f;
      if (t0 + t < N)
        f.load((const uint16_t*)vbh + (t0 + t) * D + c0);
      else
        f.zero();
      const uint32_t w[4] = {f.u.x, f.u.y, f.u.z, f.u.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[c0 + e][t] = (uint16_t)((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
    }
    __threadfence_block();
#pragma unroll
    for (int mt = 0; mt < MO; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        reinterpret_cast<Frag<uint16_t>&>(vf[mt][ks]).u =
            *reinterpret_cast<const uint4*>(&vt[16 * mt + r16][32 * ks + 8 * grp]);
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
          e8[e] = t < N ? to_f32<T>(vbh[t * D + 16 * mt + r16]) : 0.f;
        }
        Frag<float>& f = reinterpret_cast<Frag<float>&>(vf[mt][ks]);
        f.a = make_float4(e8[0], e8[1], e8[2], e8[3]);
        f.b = make_float4(e8[4], e8[5], e8[6], e8[7]);
      }
  }
}

// One leaf for the 16 columns whose query fragments are qf and whose positions are ic (-1: none):
// oacc = sum_t p_t v_t with p_t = exp(s (x_t - m)) over t <= ic; lse = s m + ln l (-inf if empty),
// inv = 1 / l. Lane (col, grp) gets O[col][16 mt + 4 grp + j] in oacc[mt][j].
template <typename T, int D, int C>
__device__ __forceinline__ void attend_tile(const Frag<T> (&kf)[C / 16][D / 32], const Frag<T> (&vf)[D / 16][C / 32],
                                            const Frag<T> (&qf)[D / 32], long long t0, long long ic, float scale,
                                            f32x4 (&oacc)[D / 16], float& lse, float& inv) {
  constexpr int MS = C / 16, KS = C / 32, MO = D / 16;
  const int grp = lane_id() >> 4;
  f32x4 sacc[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) sacc[m] = zero4();
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int m = 0; m < MS; ++m) mma(sacc[m], kf[m][s], qf[s]);
  float mx = kNegInf;
  const long long lim64 = ic - t0;
  const int lim = lim64 < 0 ? -1 : (lim64 > C ? C : (int)lim64);
#pragma unroll
  for (int m = 0; m < MS; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x = attn_token(m, grp, j) <= lim ? sacc[m][j] : kNegInf;
      sacc[m][j] = x;
      mx = fmaxf(mx, x);
    }
  mx = colgroup_max(mx);
  const bool any = mx != kNegInf;
  const float ms = any ? mx : 0.f;
  const float c2 = scale * kLog2e;
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
#pragma unroll
  for (int mt = 0; mt < MO; ++mt) {
    oacc[mt] = zero4();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) mma(oacc[mt], vf[mt][ks], pf[ks]);
  }
  inv = any ? 1.f / lsum : 0.f;
  lse = any ? scale * ms + kLn2 * fast_log2(lsum) : kNegInf;
}

}  // namespace pisa
