// Shared device helpers for the PISA kernels (gfx950 / CDNA4, wave64).
//
// Matrix tiles use v_mfma_f32_16x16x32_bf16 (bf16 inputs, fp32 accumulate) or, for fp32 inputs,
// eight v_mfma_f32_16x16x4_f32 per 32-wide k step. Per lane: A row = B column = lane % 16, lane group
// g = lane / 16 supplies 8 consecutive k elements of the step; the D tile gives lane (col = lane % 16,
// g) the rows 4g .. 4g+3. The k order inside a dot product is free, so k step s of lane group g covers
// d elements [32 s + 8 g, +8): the four lanes of a row read 64 (bf16) or 128 (fp32) contiguous bytes
// per load instruction.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pisa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kMaxLevels = 32;

// Pyramid layout of one KV head: level sizes and leaf-first offsets (rows of d floats).
struct Levels {
  int n_levels;  // including the root
  int n[kMaxLevels];
  long long off[kMaxLevels];
  long long nodes;  // rows per KV head
  // Rows of the fp16 routing planes: level l starts at roff[l], and a level of at least 4 nodes takes a
  // multiple of 4 rows (the tail rows are zero), so the 4 grandchildren 4j .. 4j+3 of a node always
  // form one aligned group of 4. rnodes (a multiple of 4) = routing rows per KV head.
  long long roff[kMaxLevels];
  long long rnodes;
};

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// v, opaque to the optimiser: values derived from it are computed where they are used instead of being
// hoisted out of the enclosing loops (where they would occupy registers for the whole loop)
__device__ __forceinline__ int opaque_int(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }

// fp32 -> bf16, round to nearest, ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values -> a packed bf16 pair (round to nearest even), a in the low half. gfx950 does this
// in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) { return f32_to_bf16(x); }

// 8 consecutive k elements of one lane.
template <typename T>
struct Frag;

template <>
struct Frag<uint16_t> {
  uint4 u;
  __device__ __forceinline__ void zero() { u = make_uint4(0u, 0u, 0u, 0u); }
  __device__ __forceinline__ void load(const uint16_t* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int e) const {
    uint32_t w = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
    return bf16_to_f32((uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
  }
};

template <>
struct Frag<float> {
  float4 a, b;
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u), __builtin_bit_cast(bf16x8_t, b.u),
                                                acc, 0, 0, 0);
}

// Quad-coalesced gathers of a 16-row operand tile. In the MFMA operand layout lane r + 16 g holds
// row r, so the four lanes of a quad would read four rows (four cache lines per quad). Instead lane
// 4 r + g loads row r's chunks 4 s + g (s = 0 .. NS-1; each quad reads one contiguous 64-byte piece of
// one row per load), and quad_rows_to_mfma() moves every lane's chunks to lane r + 16 g.
__device__ __forceinline__ int quad_row() { return lane_id() >> 2; }
__device__ __forceinline__ int quad_chunk() { return lane_id() & 3; }
template <int NS>
__device__ __forceinline__ void quad_rows_to_mfma(Frag<uint16_t> (&f)[NS]) {
  const int lane = lane_id();
  const int src = ((lane & 15) * 4 + (lane >> 4)) * 4;  // byte address of the source lane
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    f[s].u.x = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f[s].u.x);
    f[s].u.y = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f[s].u.y);
    f[s].u.z = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f[s].u.z);
    f[s].u.w = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)f[s].u.w);
  }
}

// fp16 operands held in Frag<uint16_t> bit patterns (routing planes and scaled queries).
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void mma_f16(f32x4& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a.u), __builtin_bit_cast(f16x8_t, b.u),
                                               acc, 0, 0, 0);
}
// fp16 routing planes, quad-interleaved: routing rows 4a .. 4a+3 form one group of 8 D values, the
// hi plane (4 D) then the lo plane (4 D); within a plane, 16-byte chunk c of the group's 4 rows is 64
// contiguous bytes (row 4a + q at element 32 c + 8 q). The four lanes of a quad that read chunk c of
// the 4 grandchildren of one node thus read one 64-byte segment. Returns the chunk's 8 elements.
template <typename T>
__device__ __forceinline__ T* route_plane_chunk(T* head, int R, int plane, int c, int D) {
  return head + ((unsigned)(R >> 2) * 2u + (unsigned)plane) * (4u * (unsigned)D) + 32 * c + 8 * (R & 3);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16_bits_to_f32(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// Exponent e with max * 2^e in [2^14, 2^15) for max > 0 (0 for max == 0): scaled values neither
// overflow fp16 nor, for the ones that matter, fall below its normal range.
__device__ __forceinline__ int f16_range_exp(float max_abs) {
  int ex;
  frexpf(max_abs, &ex);  // max_abs = f 2^ex, f in [0.5, 1)
  return max_abs > 0.f ? 15 - ex : 0;
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Max / sum over the 4 lane groups that hold one tile column (lanes c, c+16, c+32, c+48), on the
// gfx950 lane-swap instructions (VALU, no LDS round trip). v_permlane16_swap(v, v) returns, in every
// lane, the pair (value of the lower 16-lane row, value of the upper row) of its row pair, and
// v_permlane32_swap(v, v) the pair (lower half, upper half); combining the two halves of the pair in
// that order gives every lane of the column the same, order-fixed result.
__device__ __forceinline__ void swap16(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float v, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
// max(a, b) for values that are never NaN, as one instruction: fmaxf first quiets each operand that the
// compiler cannot prove is not a signalling NaN (two extra instructions after a lane swap), while the
// NaN-propagating maximum needs no quieting and agrees with fmaxf on every value that is not NaN (up to
// the sign of a zero result); chains of it become three-operand maxima
__device__ __forceinline__ float max_nn(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float min_nn(float a, float b) { return __builtin_elementwise_minimum(a, b); }
__device__ __forceinline__ float colgroup_max(float v) {
  float a, b;
  swap16(v, a, b);
  v = max_nn(a, b);
  swap32(v, a, b);
  return max_nn(a, b);
}
__device__ __forceinline__ float colgroup_sum(float v) {
  float a, b;
  swap16(v, a, b);
  v = a + b;
  swap32(v, a, b);
  return a + b;
}

// LSE of scale * x over the NV values this lane holds for a column plus those of the column's
// other 3 lane groups. Invalid entries are -inf. Returns -inf if all are invalid.
template <int NV>
__device__ __forceinline__ float column_lse(const float (&x)[NV], float scale) {
  float m = x[0];
#pragma unroll
  for (int j = 1; j < NV; ++j) m = max_nn(m, x[j]);
  m = colgroup_max(m);
  const bool any = m != kNegInf;
  const float ms = any ? m : 0.f;
  const float c = scale * kLog2e, mc = ms * c;
  float acc = fast_exp2(fmaf(x[0], c, -mc));  // (x - m) c, one rounding
#pragma unroll
  for (int j = 1; j < NV; ++j) acc += fast_exp2(fmaf(x[j], c, -mc));
  acc = colgroup_sum(acc);
  return any ? scale * ms + kLn2 * fast_log2(acc) : kNegInf;
}

// LSE of two already-scaled values.
__device__ __forceinline__ float lse2(float a, float b) {
  const float m = max_nn(a, b);
  const float d = min_nn(a, b) - m;
  return m + kLn2 * fast_log2(1.f + fast_exp2(d * kLog2e));
}

// LSE of two already-scaled values, either of which may be -inf.
__device__ __forceinline__ float lse2_inf(float a, float b) {
  if (a == kNegInf) return b;
  if (b == kNegInf) return a;
  return lse2(a, b);
}

// Sum over the 16 lanes of each row by DPP row rotations: every lane gets the row total (the order of
// the additions depends on the lane, so read one fixed lane when bit reproducibility matters).
template <int CTRL>
__device__ __forceinline__ float dpp_rot(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_rot<0x128>(v);  // row_ror:8
  v += dpp_rot<0x124>(v);  // row_ror:4
  v += dpp_rot<0x122>(v);  // row_ror:2
  return v + dpp_rot<0x121>(v);  // row_ror:1
}

// v of lane (this lane ^ O): a DPP quad permutation for O = 1, 2 (no LDS round trip), else a shuffle.
template <int O>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (O == 1)
    return dpp_rot<0xB1>(v);  // quad_perm [1, 0, 3, 2]
  else if constexpr (O == 2)
    return dpp_rot<0x4E>(v);  // quad_perm [2, 3, 0, 1]
  else
    return __shfl_xor(v, O);
}
// Butterfly sum over the G consecutive lanes of a group (strides G/2 .. 1, in that order).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 16) v += xor_lane<8>(v);
  if constexpr (G >= 8) v += xor_lane<4>(v);
  if constexpr (G >= 4) v += xor_lane<2>(v);
  if constexpr (G >= 2) v += xor_lane<1>(v);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 16) v = max_nn(v, xor_lane<8>(v));
  if constexpr (G >= 8) v = max_nn(v, xor_lane<4>(v));
  if constexpr (G >= 4) v = max_nn(v, xor_lane<2>(v));
  if constexpr (G >= 2) v = max_nn(v, xor_lane<1>(v));
  return v;
}

// Wave-uniform read of lane c.
__device__ __forceinline__ int readlane(int v, int c) { return __builtin_amdgcn_readlane(v, c); }
__device__ __forceinline__ float readlane(float v, int c) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), c));
}

// Max / min over all 64 lanes of the wave (every lane gets the result): DPP row reductions, then the
// four row results read back with readlane.
__device__ __forceinline__ float wave_max(float v) {
  v = max_nn(v, dpp_rot<0x128>(v));
  v = max_nn(v, dpp_rot<0x124>(v));
  v = max_nn(v, dpp_rot<0x122>(v));
  v = max_nn(v, dpp_rot<0x121>(v));
  return max_nn(max_nn(readlane(v, 0), readlane(v, 16)), max_nn(readlane(v, 32), readlane(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = min_nn(v, dpp_rot<0x128>(v));
  v = min_nn(v, dpp_rot<0x124>(v));
  v = min_nn(v, dpp_rot<0x122>(v));
  v = min_nn(v, dpp_rot<0x121>(v));
  return min_nn(min_nn(readlane(v, 0), readlane(v, 16)), min_nn(readlane(v, 32), readlane(v, 48)));
}


// Top-K ranking key of candidate c with score v: the order-preserving unsigned image of the float with
// its 6 low bits replaced by 63 - c, so that a larger key means a higher score, and exactly equal
// scores order by the lower index. Scores closer than 2^-17 relative also order by index. Callers key
// v = score - ref, with ref the score of the ranking's first candidate (topk_ref): the quantum is then
// relative to a candidate's distance from that one, 64 ulp < 1e-3 whenever the distance is below 256,
// whatever the size of the scores themselves (a unit's candidates differ by far less).
__device__ __forceinline__ uint32_t topk_key(float v, int c) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (o & ~63u) | (uint32_t)(63 - c);
}

// The reference of a ranking whose candidate c sits in lane c: lane 0's value if finite, else 0.
__device__ __forceinline__ float topk_ref(float v) {
  const float r = readlane(v, 0);
  return __builtin_isfinite(r) ? r : 0.f;
}

// Candidates c in [0, n) (ascending node order, one per lane) with scores `score`. True for the lanes
// among the K best (score descending, index ascending), keyed relative to `ref` (wave-uniform). keys:
// this wave's 64-entry LDS slice. n, K are wave-uniform.
__device__ __forceinline__ bool topk_keep_ref(float score, int n, int K, uint32_t* keys, float ref) {
  const int lane = lane_id();
  const uint32_t mine = lane < n ? topk_key(score - ref, lane) : 0u;
  keys[lane] = mine;
  __threadfence_block();
  int rank = 0;
  for (int c = 0; c < n; c += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(keys + c);
    rank += (v.x > mine) + (v.y > mine) + (v.z > mine) + (v.w > mine);
  }
  __threadfence_block();
  return lane < n && rank < K;
}

// The same, keyed relative to the first candidate's score.
__device__ __forceinline__ bool topk_keep(float score, int n, int K, uint32_t* keys) {
  return topk_keep_ref(score, n, K, keys, topk_ref(score));
}

// Same, with the scores already in s[0, n) (LDS).
__device__ __forceinline__ bool topk_keep_lds(const float* s, int n, int K, uint32_t* keys) {
  const int lane = lane_id();
  return topk_keep(s[lane < n ? lane : 0], n, K, keys);
}

// Stable compaction: lanes with keep move to [0, count) in lane order, the others after them.
// Returns the value that lands on this lane.
__device__ __forceinline__ int compact_lanes(bool keep, int value, int* count) {
  const int lane = lane_id();
  const unsigned long long m = __ballot(keep);
  const unsigned long long below = lane ? (m & ((~0ull) >> (64 - lane))) : 0ull;
  const int pos = __popcll(below);
  const int total = __popcll(m);
  const int dst = keep ? pos : total + (lane - pos);
  *count = total;
  return __builtin_amdgcn_ds_permute(dst << 2, value);
}

// A run of up to 256 consecutive entries of a bucket-sorted (unit << 5 | slot) pair list, held four
// per lane (entry x in register x / 64 of lane x % 64), with each pair's bucket key.
struct PairRun {
  uint32_t pr[4];
  long long key[4];
  long long base, end;  // entries [base, end)
  // pair at absolute index x (base <= x < base + 256); every lane may ask for a different x
  __device__ __forceinline__ uint32_t pair(long long x) const {
    const int idx = (int)(x - base);
    const int src = idx & 63, which = idx >> 6;
    const uint32_t v0 = (uint32_t)__shfl((int)pr[0], src), v1 = (uint32_t)__shfl((int)pr[1], src);
    const uint32_t v2 = (uint32_t)__shfl((int)pr[2], src), v3 = (uint32_t)__shfl((int)pr[3], src);
    return which == 0 ? v0 : which == 1 ? v1 : which == 2 ? v2 : v3;
  }
  // first index >= from whose key differs from `key_at_from` (end if none); wave-uniform
  __device__ __forceinline__ long long run_end(long long from, long long key_at_from) const {
    const int lane = lane_id();
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const long long x = base + 64 * w + lane;
      const bool diff = x >= from && x < end && key[w] != key_at_from;
      const unsigned long long m = __ballot(diff);
      if (m) return base + 64 * w + __ffsll((long long)m) - 1;
    }
    return end;
  }
};

// Work-group index remapped so that consecutive logical indices run on the same XCD (dispatch
// places work-group w on XCD w % 8), keeping each XCD's L2 on a contiguous slice of the work.
__device__ __forceinline__ int xcd_logical_block(int nblocks) {
  const int w = blockIdx.x;
  const int per = (nblocks + 7) >> 3;
  const int xcd = w & 7;
  const int idx = w >> 3;
  const int full = nblocks & 7 ? (nblocks & 7) : 8;  // XCDs that get `per` blocks
  return xcd < full ? xcd * per + idx : full * per + (xcd - full) * (per - 1) + idx;
}

}  // namespace pisa
