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

// Output dimension in D-row 4*grp + j of M-tile mt of O^T. The rows of V^T are permuted so that the
// pair of M-tiles (2c, 2c + 1) gives lane group grp the 8 consecutive dimensions 32 c + 8 grp .. +8:
// a row's 4 lanes hold 64 contiguous bytes of it per M-tile pair.
template <int D>
__device__ __forceinline__ int attn_out_dim(int mt, int grp, int j) {
  return 32 * (mt >> 1) + 8 * grp + 4 * (mt & 1) + j;
}
// Stores 16 bf16 rows of D dimensions that a wave holds in that output layout: lane (r16, grp) has chunk c
// of row r16 (dimensions 32 c + 8 grp .. +8, 16 bytes) in w[c]; own points at dimension 8 grp of row r16
// and other at dimension 8 grp of row r16 ^ 8. Rows r16 and r16 ^ 8 trade chunks by a DPP rotation by 8
// within each 16-lane row, so that every store writes whole 128-byte lines: for the chunk pair (2 L,
// 2 L + 1) the first store covers rows 0-7 (the lanes of rows 8-15 writing chunk 2 L + 1 of row r16 ^ 8)
// and the second rows 8-15, instead of four stores of 64-byte half lines. The same bytes reach the same
// places.
template <int D>
__device__ __forceinline__ void store_rows_lines(uint16_t* own, uint16_t* other, const uint4 (&w)[D / 32]) {
  static_assert(D % 64 == 0, "row of whole 128-byte lines");
  const bool lo = (lane_id() & 15) < 8;
  uint16_t* dst_a = lo ? own : other;  // rows 0-7
  uint16_t* dst_b = lo ? other : own;  // rows 8-15
  auto ror8 = [](uint32_t v) { return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false); };
#pragma unroll
  for (int L = 0; L < D / 64; ++L) {
    const uint4 a = w[2 * L], b = w[2 * L + 1];
    const uint4 xa = make_uint4(ror8(a.x), ror8(a.y), ror8(a.z), ror8(a.w));  // row r16 ^ 8's chunk 2 L
    const uint4 xb = make_uint4(ror8(b.x), ror8(b.y), ror8(b.z), ror8(b.w));  // and its chunk 2 L + 1
    const int c = lo ? 2 * L : 2 * L + 1;  // the chunk this lane writes in both stores
    // component-wise selects (a select of whole vectors would go through memory)
    *reinterpret_cast<uint4*>(dst_a + 32 * c) =
        make_uint4(lo ? a.x : xb.x, lo ? a.y : xb.y, lo ? a.z : xb.z, lo ? a.w : xb.w);
    *reinterpret_cast<uint4*>(dst_b + 32 * c) =
        make_uint4(lo ? xa.x : b.x, lo ? xa.y : b.y, lo ? xa.z : b.z, lo ? xa.w : b.w);
  }
}
// The value v of lane r16 ^ 8 (same lane group).
__device__ __forceinline__ int row_partner(int v) { return __builtin_amdgcn_update_dpp(0, v, 0x128, 0xf, 0xf, false); }

// Inverse: the V^T row (16 mt + 4 grp + j) that holds dimension d.
template <int D>
__device__ __forceinline__ int attn_vt_row(int d) {
  const int mt = 2 * (d >> 5) + ((d >> 2) & 1), grp = (d >> 3) & 3, j = d & 3;
  return 16 * mt + 4 * grp + j;
}

// 16 bytes at p; NT: a non-temporal load, for data read once per kernel (a streamed cache tile), so
// that it does not displace data that is read again.
template <bool NT>
__device__ __forceinline__ uint4 load16(const uint16_t* p) {
  if constexpr (NT) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(x.x, x.y, x.z, x.w);
  } else {
    return *reinterpret_cast<const uint4*>(p);
  }
}

// K tile of the leaf starting at token t0, rows permuted (attn_token). Rows past N repeat row N - 1:
// those tokens are later than every query, so the causal mask drops them before any use. NT (bf16):
// non-temporal loads.
template <typename T, int D, int C, bool NT = false>
__device__ __forceinline__ void load_attn_k(const T* kbh, long long t0, long long N, Frag<T> (&kf)[C / 16][D / 32]) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
#pragma unroll
  for (int m = 0; m < C / 16; ++m) {
    long long t = t0 + attn_token(m, r16 >> 2, r16 & 3);
    t = t < N ? t : N - 1;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if constexpr (sizeof(T) == 2)
        kf[m][s].u = load16<NT>(reinterpret_cast<const uint16_t*>(kbh) + t * D + 32 * s + 8 * grp);
      else
        kf[m][s].load(kbh + t * D + 32 * s + 8 * grp);
    }
  }
}

// Stage the bf16 V tile of the leaf at t0 transposed into vt, this wave's [D][C + 8] LDS scratch:
// dimension d goes to row attn_vt_row(d). Tokens past N repeat token N - 1 (their probabilities are
// exactly zero). Each lane writes (token 2tp, token 2tp + 1) pairs as 32-bit words.
template <int D, int C, bool NT = false>
__device__ __forceinline__ void stage_attn_vt(const uint16_t* vbh, long long t0, long long N, uint16_t (*vt)[C + 8]) {
  const int lane = lane_id();
  constexpr int CHR = D / 8;               // 8-element chunks per V row
  constexpr int NIT = (C / 2) * CHR / 64;  // token pairs x chunks per lane
  static_assert(((C / 2) * CHR) % 64 == 0, "tile shape");
  uint4 f0[NIT], f1[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int qd = it * 64 + lane;
    const int tp = qd / CHR, c0 = (qd % CHR) * 8;
    long long ta = t0 + 2 * tp, tb = ta + 1;
    ta = ta < N ? ta : N - 1;
    tb = tb < N ? tb : N - 1;
    f0[it] = load16<NT>(vbh + ta * D + c0);
    f1[it] = load16<NT>(vbh + tb * D + c0);
  }
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int qd = it * 64 + lane;
    const int tp = qd / CHR, c0 = (qd % CHR) * 8;
    const uint32_t a[4] = {f0[it].x, f0[it].y, f0[it].z, f0[it].w};
    const uint32_t b[4] = {f1[it].x, f1[it].y, f1[it].z, f1[it].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<uint32_t*>(&vt[attn_vt_row<D>(c0 + e)][2 * tp]) = w;
    }
  }
  __threadfence_block();
}

// V^T A-fragment (M-tile mt, k step ks) from the staged tile: lane (row 16 mt + r16, grp) gets
// V[32 ks + 8 grp + e][attn_out_dim(mt, r16 / 4, r16 % 4)], e = 0..7.
template <int C>
__device__ __forceinline__ Frag<uint16_t> vt_frag(const uint16_t (*vt)[C + 8], int mt, int ks) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
  Frag<uint16_t> f;
  f.u = *reinterpret_cast<const uint4*>(&vt[16 * mt + r16][32 * ks + 8 * grp]);
  return f;
}

// All V^T fragments in registers (bf16 staged through vt, with non-temporal loads if NT; fp32 loaded
// directly).
template <typename T, int D, int C, bool NT = false>
__device__ __forceinline__ void load_attn_vt(const T* vbh, long long t0, long long N, uint16_t (*vt)[C + 8],
                                             Frag<T> (&vf)[D / 16][C / 32]) {
  constexpr int MO = D / 16, KS = C / 32;
  const int lane = lane_id(), r16 = lane & 15, grp = lane >> 4;
  if constexpr (sizeof(T) == 2) {
    stage_attn_vt<D, C, NT>((const uint16_t*)vbh, t0, N, vt);
#pragma unroll
    for (int mt = 0; mt < MO; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) reinterpret_cast<Frag<uint16_t>&>(vf[mt][ks]) = vt_frag<C>(vt, mt, ks);
    __threadfence_block();
  } else {
#pragma unroll
    for (int mt = 0; mt < MO; ++mt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float e8[8];
        const int d = attn_out_dim<D>(mt, r16 >> 2, r16 & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          long long t = t0 + 32 * ks + 8 * grp + e;
          t = t < N ? t : N - 1;
          e8[e] = to_f32<T>(vbh[t * D + d]);
        }
        Frag<float>& f = reinterpret_cast<Frag<float>&>(vf[mt][ks]);
        f.a = make_float4(e8[0], e8[1], e8[2], e8[3]);
        f.b = make_float4(e8[4], e8[5], e8[6], e8[7]);
      }
  }
}

// One leaf for the 16 columns whose query fragments are qf and whose positions are ic (-1: none):
// oacc = sum_t p_t v_t with p_t = exp(s (x_t - m)) over t <= ic; lse = s m + ln l (-inf if empty),
// inv = 1 / l. Lane (col, grp) gets O[col][attn_out_dim(mt, grp, j)] in oacc[mt][j].
// kfrag(m, s) returns the K A-fragment of S M-tile m, k step s; vfrag(mt, ks) the V^T A-fragment of
// O^T M-tile mt, k step ks.
// kPhased: keep the scheduler from hoisting the V^T fragment reads above the softmax (LDS-sourced
// fragments would otherwise all be live at once).
template <typename T, int D, int C, bool kPhased = false, typename KFrag, typename VFrag>
__device__ __forceinline__ void attend_tile_kv(KFrag kfrag, VFrag vfrag, const Frag<T> (&qf)[D / 32], long long t0,
                                               long long ic, float scale, f32x4 (&oacc)[D / 16], float& lse,
                                               float& inv) {
  constexpr int MS = C / 16, KS = C / 32, MO = D / 16;
  const int grp = lane_id() >> 4;
  f32x4 sacc[MS];
#pragma unroll
  for (int m = 0; m < MS; ++m) sacc[m] = zero4();
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
#pragma unroll
    for (int m = 0; m < MS; ++m) mma(sacc[m], kfrag(m, s), qf[s]);
  float mx = kNegInf;
  const long long lim64 = ic - t0;
  const int lim = lim64 < 0 ? -1 : (lim64 > C ? C : (int)lim64);
  bool all_visible = false;
  if constexpr (sizeof(T) == 2) all_visible = __all(lim >= C - 1);
  if (all_visible) {
    // bf16: every column sees the whole leaf (the usual case away from the diagonal): no mask (same values)
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max_nn(mx, sacc[m][j]);
  } else {
#pragma unroll
    for (int m = 0; m < MS; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = attn_token(m, grp, j) <= lim ? sacc[m][j] : kNegInf;
        sacc[m][j] = x;
        mx = max_nn(mx, x);
      }
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
  if constexpr (kPhased) __builtin_amdgcn_sched_barrier(0);
  Frag<T> pf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (sizeof(T) == 2) {
      const f32x4 a = sacc[2 * ks], bb = sacc[2 * ks + 1];
      Frag<uint16_t>& f = reinterpret_cast<Frag<uint16_t>&>(pf[ks]);
      f.u.x = pack_bf16x2(a[0], a[1]);
      f.u.y = pack_bf16x2(a[2], a[3]);
      f.u.z = pack_bf16x2(bb[0], bb[1]);
      f.u.w = pack_bf16x2(bb[2], bb[3]);
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
    for (int ks = 0; ks < KS; ++ks) mma(oacc[mt], vfrag(mt, ks), pf[ks]);
  }
  inv = any ? 1.f / lsum : 0.f;
  lse = any ? scale * ms + kLn2 * fast_log2(lsum) : kNegInf;
}

template <typename T, int D, int C>
__device__ __forceinline__ void attend_tile(const Frag<T> (&kf)[C / 16][D / 32], const Frag<T> (&vf)[D / 16][C / 32],
                                            const Frag<T> (&qf)[D / 32], long long t0, long long ic, float scale,
                                            f32x4 (&oacc)[D / 16], float& lse, float& inv) {
  attend_tile_kv<T, D, C>([&](int m, int s) -> const Frag<T>& { return kf[m][s]; },
                          [&](int mt, int ks) -> const Frag<T>& { return vf[mt][ks]; }, qf, t0, ic, scale, oacc, lse,
                          inv);
}

// ---- work-group shared bf16 tiles (C x D keys, swizzled; D x (C + 8) transposed values)
// 16-byte chunk c of key row t is stored at chunk c ^ kswz(t): the 16 rows that one K-fragment read
// touches (attn_token of one M-tile) then fall on distinct chunk columns, so the read is free of
// bank conflicts.
template <int D>
__device__ __forceinline__ int kswz(int t) {
  return ((t & 3) | ((t >> 1) & 12)) & (D / 8 - 1);
}

// Cooperative staging by the work-group's 256 threads: K rows into sk (swizzled), V^T into svt.
// Tokens past N repeat token N - 1 (masked for every query).
template <int D, int C>
__device__ __forceinline__ void stage_kv_wg(const uint16_t* kbh, const uint16_t* vbh, long long t0, long long N,
                                            uint16_t (*sk)[D], uint16_t (*svt)[C + 8]) {
  const int tid = threadIdx.x;
  constexpr int CHR = D / 8;  // 16-byte chunks per row
  // K: C * CHR chunks; V: (C / 2) * CHR (token pair, chunk) items
  constexpr int KN = C * CHR, VN = (C / 2) * CHR;
  constexpr int KIT = (KN + 255) / 256, VIT = (VN + 255) / 256;
  uint4 kk[KIT], v0[VIT], v1[VIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    long long tt = t0 + t;
    tt = tt < N ? tt : N - 1;
    if (KN % 256 == 0 || x < KN) kk[it] = *reinterpret_cast<const uint4*>(kbh + tt * D + 8 * c);
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int x = it * 256 + tid, tp = x / CHR, c0 = (x % CHR) * 8;
    long long ta = t0 + 2 * tp, tb = ta + 1;
    ta = ta < N ? ta : N - 1;
    tb = tb < N ? tb : N - 1;
    if (VN % 256 == 0 || x < VN) {
      v0[it] = *reinterpret_cast<const uint4*>(vbh + ta * D + c0);
      v1[it] = *reinterpret_cast<const uint4*>(vbh + tb * D + c0);
    }
  }
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    if (KN % 256 == 0 || x < KN) *reinterpret_cast<uint4*>(&sk[t][8 * (c ^ kswz<D>(t))]) = kk[it];
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int x = it * 256 + tid, tp = x / CHR, c0 = (x % CHR) * 8;
    if (VN % 256 != 0 && x >= VN) continue;
    const uint32_t a[4] = {v0[it].x, v0[it].y, v0[it].z, v0[it].w};
    const uint32_t b[4] = {v1[it].x, v1[it].y, v1[it].z, v1[it].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = __builtin_amdgcn_perm(b[e >> 1], a[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<uint32_t*>(&svt[attn_vt_row<D>(c0 + e)][2 * tp]) = w;
    }
  }
}

// Cooperative staging of C rows (tokens t0 .. t0 + C - 1, past N: token N - 1) into a swizzled [C][D]
// tile, the layout stage_kv_wg gives the keys.
template <int D, int C>
__device__ __forceinline__ void stage_rows_wg(const uint16_t* src, long long t0, long long N, uint16_t (*sk)[D]) {
  const int tid = threadIdx.x;
  constexpr int CHR = D / 8;
  constexpr int KN = C * CHR;
  constexpr int KIT = (KN + 255) / 256;
  uint4 kk[KIT];
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    long long tt = t0 + t;
    tt = tt < N ? tt : N - 1;
    if (KN % 256 == 0 || x < KN) kk[it] = *reinterpret_cast<const uint4*>(src + tt * D + 8 * c);
  }
#pragma unroll
  for (int it = 0; it < KIT; ++it) {
    const int x = it * 256 + tid, t = x / CHR, c = x % CHR;
    if (KN % 256 == 0 || x < KN) *reinterpret_cast<uint4*>(&sk[t][8 * (c ^ kswz<D>(t))]) = kk[it];
  }
}

// K A-fragment (S M-tile m, k step s) from the swizzled shared tile.
template <int D>
__device__ __forceinline__ Frag<uint16_t> k_frag_wg(const uint16_t (*sk)[D], int m, int s) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
  const int t = attn_token(m, r16 >> 2, r16 & 3);
  Frag<uint16_t> f;
  f.u = *reinterpret_cast<const uint4*>(&sk[t][8 * ((4 * s + grp) ^ kswz<D>(t))]);
  return f;
}

}  // namespace pisa
