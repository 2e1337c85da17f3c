// Fused decode step ("Block Sparse Attention with Log-Linear Complexity" digest, 工作参考价值 second
// bullet and 方法关键点 Kernel bullet: decode keeps a cached mean pyramid, updates only the new
// token's ancestor path, amortised O(log N) per step, and one kernel covers every level so that no
// further launches are paid).
//
// One work-group (8 waves) per (sequence b, KV head r), i.e. per decode unit; p = cached length:
//   1. append k_new, v_new at position p; add k_new to the sum of each ancestor of leaf p / C (every
//      level of the capacity layout) and refresh that node's mean = sum / tokens held;
//   2. walk the levels for query i = p: per scored level all threads stage the candidates' child
//      means into LDS (bf16 hi/lo, or fp32 for fp32 inputs), each wave scores one M-tile on MFMA
//      (8 candidates), and wave 0 keeps the Top-K;
//   3. leaf stage: the kept level-1 nodes' leaf pairs are spread over the 8 waves (exact per-head
//      LSE with the causal mask), wave 0 takes the leaf Top-K;
//   4. attention: the selected leaves are spread over the waves; each wave merges its leaves'
//      partial outputs with running LSE weights, and the 8 wave results are merged at the end.
// The update lands before the walk reads it: writes are fenced (work-group scope) and the work-group
// synchronises, and a work-group only reads its own (b, r) cache and pyramid.
#include "attn_tiles.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "walk_tiles.hpp"

namespace pisa {

template <typename T>
struct DecodeParams {
  const T* q_new;
  const T* k_new;
  const T* v_new;
  T* k_cache;
  T* v_cache;
  float* pyr_sum;
  float* pyr_mean;
  T* o;
  int* sel_out;
  int B, Hq, Hkv, G, Nmax, K;
  float scale;
  Levels lv;
  LensArg lens;
};

constexpr int kDecodeWaves = 8;

template <typename T, int D, int C, int KM>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_kernel(DecodeParams<T> p) {
  constexpr int NW = kDecodeWaves;
  constexpr int NT = NW * 64;
  constexpr int LOG2C = C == 64 ? 6 : 5;
  constexpr int ROWB = sizeof(T) == 2 ? 2 * D * 2 : D * 4;  // bytes per staged child row
  constexpr int STAGE = 16 * KM * ROWB;                     // 2K candidates x 2 children
  constexpr int VTB = NW * D * (C + 8) * 2;                 // per-wave transposed V tiles
  constexpr int OB = NW * 16 * D * 4;                       // per-wave outputs for the final merge
  constexpr int UNION = STAGE > VTB ? (STAGE > OB ? STAGE : OB) : (VTB > OB ? VTB : OB);
  constexpr int MO = D / 16;
  static_assert(KM <= NW, "one M-tile per wave");
  __shared__ __align__(16) unsigned char s_buf[UNION];
  __shared__ __align__(16) float s_sc[64];
  __shared__ __align__(16) uint32_t s_key[64];
  __shared__ float s_ell[64][17];
  __shared__ int s_kept[64];
  __shared__ int s_sel[64];
  __shared__ int s_n[2];
  __shared__ float s_lse[NW][16];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const int pos = p.lens.len[b];
  const int len = pos + 1;
  const long long head_row = (long long)bh * p.lv.nodes;
  // ---- 1. append and ancestor-path update
  if (tid < D) {
    const T kv = p.k_new[(long long)bh * D + tid];
    p.k_cache[((long long)bh * p.Nmax + pos) * D + tid] = kv;
    p.v_cache[((long long)bh * p.Nmax + pos) * D + tid] = p.v_new[(long long)bh * D + tid];
    const float kf = to_f32<T>(kv);
    // all ancestor sums are read first (independent loads), then updated
    float old_sum[kMaxLevels];
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l)
      if (l < p.lv.n_levels) old_sum[l] = p.pyr_sum[(head_row + p.lv.off[l] + (pos >> (LOG2C + l))) * D + tid];
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {
      if (l < p.lv.n_levels) {
        const long long j = pos >> (LOG2C + l);
        const long long row = (head_row + p.lv.off[l] + j) * D + tid;
        const float sm = old_sum[l] + kf;
        p.pyr_sum[row] = sm;
        const long long lo = j << (LOG2C + l);
        const long long hi = (j + 1) << (LOG2C + l);
        const float cnt = (float)((hi < len ? hi : (long long)len) - lo);
        p.pyr_mean[row] = sm / cnt;
      }
    }
  }
  // Only this work-group reads these writes during the step (its own cache rows and pyramid path),
  // so a work-group-scope fence orders them before the barrier; the next step is a new launch.
  __threadfence_block();
  __syncthreads();
  // query fragments: columns = the group's heads
  Frag<T> qf[D / 32];
  const bool hv = r16 < p.G;
  {
    const T* qrow = p.q_new + ((long long)b * p.Hq + (long long)r * p.G + (hv ? r16 : 0)) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      if (hv)
        qf[s].load(qrow + 32 * s);
      else
        qf[s].zero();
    }
  }
  const int i = pos;
  const int K = p.K;
  // ---- 2. walk to level 1
  int lstar = 0;
  for (int l = p.lv.n_levels - 1; l >= 1; --l) {
    if ((i >> (LOG2C + l)) + 1 > K) {
      lstar = l;
      break;
    }
  }
  int nk;
  if (lstar == 0) {
    nk = (i >> (LOG2C + 1)) + 1;
    if (tid < 64) s_kept[tid] = tid < nk ? tid : -1;
  } else {
    nk = (i >> (LOG2C + lstar + 1)) + 1;
    if (tid < 64) s_kept[tid] = tid < nk ? tid : -1;
    __syncthreads();
    for (int l = lstar; l >= 1; --l) {
      const int e_l = (i >> (LOG2C + l)) + 1;
      const int e_child = (i >> (LOG2C + l - 1)) + 1;
      int n_cand = 2 * nk;
      const int last = 2 * s_kept[nk - 1] + 1;
      if (last >= e_l) --n_cand;
      if (n_cand <= K) {
        __syncthreads();
        if (tid < 64) s_kept[tid] = tid < n_cand ? 2 * s_kept[tid >> 1] + (tid & 1) : -1;
        __syncthreads();
        nk = n_cand;
        continue;
      }
      const bool last_two = 2 * (2 * s_kept[(n_cand - 1) >> 1] + ((n_cand - 1) & 1)) + 1 < e_child;
      const int n_full = last_two ? n_cand : n_cand - 1;
      // stage child rows 2c + bit (child node 4 kept[c/2] + 2(c&1) + bit) of the level-(l-1) means
      const int n_rows = 2 * n_cand;
      const long long lvl_row = head_row + p.lv.off[l - 1];
      // all of this thread's row loads are issued before any is used
      constexpr int SPT = (16 * KM * (D / 4) + NT - 1) / NT;  // staging items per thread
      float4 mv[SPT];
#pragma unroll
      for (int it = 0; it < SPT; ++it) {
        const int x = tid + NT * it;
        mv[it] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (x < n_rows * (D / 4)) {
          const int rho = x / (D / 4), q4 = x % (D / 4);
          const int c = rho >> 1, bit = rho & 1;
          const int child = 4 * s_kept[c >> 1] + 2 * (c & 1) + bit;
          if (bit == 0 || c < n_full) mv[it] = *reinterpret_cast<const float4*>(p.pyr_mean + (lvl_row + child) * D + 4 * q4);
        }
      }
#pragma unroll
      for (int it = 0; it < SPT; ++it) {
        const int x = tid + NT * it;
        if (x >= n_rows * (D / 4)) continue;
        const int rho = x / (D / 4), q4 = x % (D / 4);
        const float4 m = mv[it];
        if constexpr (sizeof(T) == 2) {
          uint16_t* row = reinterpret_cast<uint16_t*>(s_buf) + rho * 2 * D + 4 * q4;
          const float v4[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t h16 = f32_to_bf16(v4[e]);
            row[e] = h16;
            row[D + e] = f32_to_bf16(v4[e] - bf16_to_f32(h16));
          }
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(s_buf) + rho * D + 4 * q4) = m;
        }
      }
      __syncthreads();
      if (wave < (2 * n_cand + 15) >> 4) {  // one M-tile (8 candidates) per wave
        StagedRows<T, D> rows;
        rows.base = reinterpret_cast<const T*>(s_buf);
        score_staged_mtile<T, D>(rows, qf, wave, n_full, p.G, p.scale, s_sc);
      }
      __syncthreads();
      if (wave == 0) {
        const int cn = lane < n_cand ? 2 * s_kept[lane >> 1] + (lane & 1) : -1;
        const bool keep = topk_keep_lds(s_sc, n_cand, K, s_key);
        int cnt;
        const int nxt = compact_lanes(keep, cn, &cnt);
        s_kept[lane] = lane < cnt ? nxt : -1;
        if (lane == 0) s_n[0] = cnt;
      }
      __syncthreads();
      nk = s_n[0];
    }
  }
  __syncthreads();
  // ---- 3. leaf stage: pairs of leaves under the kept level-1 nodes
  const T* kbh = p.k_cache + (long long)bh * p.Nmax * D;
  const T* vbh = p.v_cache + (long long)bh * p.Nmax * D;
  for (int slot = wave; slot < nk; slot += NW) {
    const long long pn = s_kept[slot];
    Frag<T> kf[C / 8][D / 32];
    load_leaf_pair<T, D, C>(kbh, 2 * pn * C, len, kf);
    float l0, l1;
    leaf_pair_lse<T, D, C>(kf, qf, 2 * pn * C, i, p.scale, l0, l1);
    if (grp == 0 && hv) {
      s_ell[2 * slot][r16] = l0;
      s_ell[2 * slot + 1][r16] = l1;
    }
  }
  __syncthreads();
  if (wave == 0) {
    int n_cand = 2 * nk;
    if (((2 * s_kept[nk - 1] + 1) << LOG2C) > i) --n_cand;
    const int leaf_c = lane < 2 * nk ? 2 * s_kept[lane >> 1] + (lane & 1) : -1;
    bool keep = lane < n_cand;
    if (n_cand > K) {
      float sc = 0.f;
      if (lane < n_cand)
        for (int h = 0; h < p.G; ++h) sc += s_ell[lane][h];
      keep = topk_keep(sc, n_cand, K, s_key);
    }
    int nsel;
    const int leaf = compact_lanes(keep, leaf_c, &nsel);
    s_sel[lane] = lane < nsel ? leaf : -1;
    if (lane == 0) s_n[1] = nsel;
    if (p.sel_out && lane < K) p.sel_out[(long long)bh * K + lane] = lane < nsel ? leaf : -1;
  }
  __syncthreads();
  const int nsel = s_n[1];
  // ---- 4. attention over the selected leaves
  f32x4 run_o[MO];
#pragma unroll
  for (int mt = 0; mt < MO; ++mt) run_o[mt] = zero4();
  float run_lse = kNegInf;
  uint16_t(*vt)[C + 8] = reinterpret_cast<uint16_t(*)[C + 8]>(s_buf) + wave * D;
  for (int k = wave; k < nsel; k += NW) {
    const long long t0 = (long long)s_sel[k] * C;
    Frag<T> kf[C / 16][D / 32];
    load_attn_k<T, D, C>(kbh, t0, len, kf);
    Frag<T> vf[D / 16][C / 32];
    load_attn_vt<T, D, C>(vbh, t0, len, vt, vf);
    f32x4 oacc[MO];
    float lse, inv;
    attend_tile<T, D, C>(kf, vf, qf, t0, hv ? i : -1, p.scale, oacc, lse, inv);
    const float m = fmaxf(run_lse, lse);
    if (m != kNegInf) {
      const float wa = run_lse == kNegInf ? 0.f : fast_exp2((run_lse - m) * kLog2e);
      const float wb = lse == kNegInf ? 0.f : fast_exp2((lse - m) * kLog2e);
      const float den = wa + wb;
      const float fa = wa / den, fb = wb * inv / den;
#pragma unroll
      for (int mt = 0; mt < MO; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) run_o[mt][j] = run_o[mt][j] * fa + oacc[mt][j] * fb;
      run_lse = m + kLn2 * fast_log2(den);
    }
  }
  __syncthreads();  // every wave is done with its transposed V tiles: s_buf now holds the outputs
  float(*s_o)[16][D] = reinterpret_cast<float(*)[16][D]>(s_buf);
#pragma unroll
  for (int mt = 0; mt < MO; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_o[wave][r16][attn_out_dim<D>(mt, grp, j)] = run_o[mt][j];
  if (grp == 0) s_lse[wave][r16] = run_lse;
  __syncthreads();
  for (int x = tid; x < p.G * D; x += NT) {
    const int h = x / D, d = x % D;
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = fmaxf(m, s_lse[w][h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float lw = s_lse[w][h];
      const float wt = lw == kNegInf ? 0.f : fast_exp2((lw - m) * kLog2e);
      num += wt * s_o[w][h][d];
      den += wt;
    }
    p.o[((long long)b * p.Hq + (long long)r * p.G + h) * D + d] = from_f32<T>(num / den);
  }
}

template <typename T, int D, int C>
static hipError_t decode_t(const DecodeArgs& da, const void* q_new, const void* k_new, const void* v_new,
                           void* k_cache, void* v_cache, float* pyr_sum, float* pyr_mean, void* o, int* sel_out,
                           hipStream_t st) {
  DecodeParams<T> p;
  p.q_new = (const T*)q_new;
  p.k_new = (const T*)k_new;
  p.v_new = (const T*)v_new;
  p.k_cache = (T*)k_cache;
  p.v_cache = (T*)v_cache;
  p.pyr_sum = pyr_sum;
  p.pyr_mean = pyr_mean;
  p.o = (T*)o;
  p.sel_out = sel_out;
  p.B = da.B;
  p.Hq = da.Hq;
  p.Hkv = da.Hkv;
  p.G = da.G;
  p.Nmax = da.Nmax;
  p.K = da.K;
  p.scale = da.scale;
  p.lv = da.lv;
  p.lens = da.lens;
  const int grid = da.B * da.Hkv;
  if (da.K <= 16)
    hipLaunchKernelGGL((decode_kernel<T, D, C, 4>), dim3(grid), dim3(kDecodeWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, C, 8>), dim3(grid), dim3(kDecodeWaves * 64), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& da, const void* q_new, const void* k_new, const void* v_new, void* k_cache,
                         void* v_cache, float* pyr_sum, float* pyr_mean, void* o, int* sel_out, hipStream_t st) {
#define PISA_DEC(T, D, C) return decode_t<T, D, C>(da, q_new, k_new, v_new, k_cache, v_cache, pyr_sum, pyr_mean, o, sel_out, st)
  if (da.bf16) {
    if (da.D == 128) {
      if (da.C == 64) PISA_DEC(uint16_t, 128, 64);
      PISA_DEC(uint16_t, 128, 32);
    }
    if (da.C == 64) PISA_DEC(uint16_t, 64, 64);
    PISA_DEC(uint16_t, 64, 32);
  }
  if (da.D == 128) {
    if (da.C == 64) PISA_DEC(float, 128, 64);
    PISA_DEC(float, 128, 32);
  }
  if (da.C == 64) PISA_DEC(float, 64, 64);
  PISA_DEC(float, 64, 32);
#undef PISA_DEC
}

}  // namespace pisa
