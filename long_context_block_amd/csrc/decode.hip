// Fused decode step ("Block Sparse Attention with Log-Linear Complexity" digest, 工作参考价值 second
// bullet and 方法关键点 Kernel bullet: decode keeps a cached mean pyramid, updates only the new
// token's ancestor path, amortised O(log N) per step, and one kernel covers every level so that no
// further launches are paid).
//
// One launch per step, S work-groups of 8 waves per decode unit (sequence b, KV head r), S = 2K / 8,
// so that a batch of a few units still spreads over every CU (a unit's work-groups are consecutive
// logical blocks on one XCD, sharing its L2). With p = cached length and i = p:
//   1. walk (every work-group, redundantly; the waves share a level's M-tiles, one barrier per
//      level, and every wave takes the same Top-K by counting ranks over LDS): from the top scored
//      level down to level 1, each candidate's child means come straight from memory into MFMA
//      fragments (fp32, split into bf16 hi + lo for bf16 inputs). The new token's ancestors are read
//      as (stored sum + k_new) / tokens held, the value the step writes back at its end, so the walk
//      sees the updated pyramid without anyone having written it yet;
//   2. leaf stage and attention, fused and split: the <= 2K candidate leaves (children of the kept
//      level-1 nodes) are dealt one per wave over the unit's S x 8 waves; a wave loads its leaf's K
//      and V once and computes, per head of the group, the leaf's exact LSE over t <= i (the
//      selection score term) and the leaf's normalised attention output, both to the workspace;
//   3. the last work-group of the unit to finish (an arrival counter) ranks the candidate leaves by
//      their head-summed LSEs (Top-K), merges the selected leaves' outputs with LSE weights, writes
//      o and sel, appends k_new / v_new at position p and adds k_new to each ancestor's sum and mean.
// Every work-group of a unit reads only the old pyramid and the old cache rows (the leaf holding p is
// completed by the wave that takes it), and the writes of step 3 happen after every other work-group
// of the unit has arrived, so no work-group reads what another writes during the step. Attention
// outputs of candidate leaves that the Top-K drops are computed and discarded: at most K extra V
// tiles per unit, in exchange for reading each candidate's K tile once and for no second pass.
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
  int* ticket;      // [U] arrival counters (zero between steps)
  float* part_o;    // [U, maxc, G, D] normalised attention output of each candidate leaf
  float* part_lse;  // [U, maxc, G] per-head LSE of each candidate leaf
  int B, Hq, Hkv, G, Nmax, K, S, maxc;
  float scale;
  Levels lv;
  LensArg lens;
};

// Mean of a node after the new token is added to it: (stored sum + k_new) / tokens it then holds. The
// walk and the final write-back evaluate the same expression, so both see the same value.
__device__ __forceinline__ float grown_mean(float sum, float knew, float held) { return (sum + knew) / held; }

// Tokens held by node j of a level whose nodes span 2^shift tokens, in a sequence of len tokens.
__device__ __forceinline__ float node_tokens(long long j, int shift, int len) {
  const long long lo = j << shift, hi = (j + 1) << shift;
  return (float)((hi < (long long)len ? hi : (long long)len) - lo);
}

// Dot products of one M-tile of fp32 child-mean rows (lane (r16, grp): row r16's elements
// 32 s + 8 grp .. +8) with the query columns: bf16 inputs split each element into bf16 hi + lo
// (hardware round-to-nearest-even) and accumulate both on the bf16 MFMA; fp32 inputs use the fp32
// MFMA directly.
template <typename T, int D>
__device__ __forceinline__ void dot_mean_rows(f32x4& acc, const float4 (&x)[D / 32][2], const Frag<T> (&qf)[D / 32]) {
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    if constexpr (sizeof(T) == 2) {
      const float v[8] = {x[s][0].x, x[s][0].y, x[s][0].z, x[s][0].w, x[s][1].x, x[s][1].y, x[s][1].z, x[s][1].w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hw[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
        const float r0 = v[2 * e] - __uint_as_float(hw[e] << 16), r1 = v[2 * e + 1] - __uint_as_float(hw[e] & 0xffff0000u);
        lw[e] = pack_bf16x2(r0, r1);
      }
      Frag<uint16_t> hi, lo;
      hi.u = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      lo.u = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      mma(acc, hi, qf[s]);
      mma(acc, lo, qf[s]);
    } else {
      Frag<float> f;
      f.a = x[s][0];
      f.b = x[s][1];
      mma(acc, f, qf[s]);
    }
  }
}

// Device-scope (all XCDs) store and load of one float: written through to, and read from, the level
// where the XCDs' caches are coherent.
__device__ __forceinline__ void store_device(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum over the 64 lanes (every lane gets it): row sums by DPP rotations, then the four rows.
__device__ __forceinline__ float wave_sum(float v) {
  v = row_sum16(v);
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

constexpr int kDecodeWaves = 8;
constexpr int kDecodeMaxG = 16;  // query heads per KV head (the 16 MFMA columns)

template <typename T, int D, int C, int KM>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_kernel(DecodeParams<T> p) {
  constexpr int NW = kDecodeWaves;
  constexpr int NT = NW * 64;
  constexpr int LOG2C = C == 64 ? 6 : 5;
  constexpr int MO = D / 16;
  constexpr int MW = (KM + NW - 1) / NW;  // M-tiles per wave at a scored level
  // per-wave LDS tile: the transposed V tile (bf16), later the leaf's output for the coalesced stores
  constexpr int VTW = sizeof(T) == 2 ? D * (C + 8) * 2 : 0;
  constexpr int TILE = VTW > kDecodeMaxG * D * 4 ? VTW : kDecodeMaxG * D * 4;
  __shared__ __align__(16) unsigned char s_vt[NW * TILE];
  __shared__ __align__(16) float s_sc[2][64];
  __shared__ float s_knew[D];
  __shared__ float s_w[64][17];
  __shared__ __align__(16) uint32_t s_keys[NW][64];  // each wave's Top-K keys (rank counting)
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  // unit and split: a unit's S work-groups are consecutive logical blocks, which share an XCD
  const int lb = xcd_logical_block(p.B * p.Hkv * p.S);
  const int bh = lb / p.S, split = lb % p.S;
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const int pos = p.lens.len[b];
  const int len = pos + 1;
  const int i = pos;
  const int K = p.K;
  const long long head_row = (long long)bh * p.lv.nodes;
  if (tid < D) s_knew[tid] = to_f32<T>(p.k_new[(long long)bh * D + tid]);
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
  __syncthreads();
  // ---- 1. walk to level 1. Every wave keeps the kept list in registers; a level's M-tiles are
  // dealt to the waves, the scores meet in LDS (double-buffered by level parity, so one barrier per
  // level suffices) and every wave takes the same Top-K.
  int lstar = 0;
  for (int l = p.lv.n_levels - 1; l >= 1; --l) {
    if ((i >> (LOG2C + l)) + 1 > K) {
      lstar = l;
      break;
    }
  }
  // kept nodes of the level above the walk's current one, ascending, one per lane
  int nk = (i >> (LOG2C + lstar + 1)) + 1;
  int kept = lane < nk ? lane : -1;
  for (int l = lstar; l >= 1; --l) {
    const int e_l = (i >> (LOG2C + l)) + 1;
    const int e_child = (i >> (LOG2C + l - 1)) + 1;
    const int last = 2 * readlane(kept, nk - 1) + 1;
    const int n_cand = 2 * nk - (last >= e_l ? 1 : 0);
    const int cn = lane < n_cand ? 2 * __shfl(kept, (lane >> 1) & 63) + (lane & 1) : -1;
    if (n_cand <= K) {
      kept = cn;
      nk = n_cand;
      continue;
    }
    float* sc = s_sc[l & 1];
    const int MT = (2 * n_cand + 15) >> 4;
    const bool last_two = 2 * readlane(cn, n_cand - 1) + 1 < e_child;
    const int n_full = last_two ? n_cand : n_cand - 1;
    const long long lvl_row = head_row + p.lv.off[l - 1];
    const int anc = i >> (LOG2C + l - 1);  // the new token's ancestor at level l - 1
    float4 x[MW][D / 32][2];
    int child[MW];
#pragma unroll
    for (int mw = 0; mw < MW; ++mw) {
      const int m = wave + NW * mw;
      const int row = 16 * m + r16;
      const int cidx = row >> 1;
      const int cnode = __shfl(cn, cidx & 63);
      const bool valid = m < MT && cidx < n_cand && ((row & 1) == 0 || cidx < n_full);
      child[mw] = valid ? 2 * cnode + (row & 1) : 0;
      if (m < MT) {
        // the new token's ancestor is read as its sum, and grown below
        const float* src = (valid && child[mw] == anc ? p.pyr_sum : p.pyr_mean) + lvl_row * D +
                           (unsigned)(child[mw] * D + 8 * grp);
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          x[mw][s][0] = *reinterpret_cast<const float4*>(src + 32 * s);
          x[mw][s][1] = *reinterpret_cast<const float4*>(src + 32 * s + 4);
        }
      }
      child[mw] = valid ? child[mw] : -1;
    }
#pragma unroll
    for (int mw = 0; mw < MW; ++mw) {
      const int m = wave + NW * mw;
      if (m < MT) {
        if (child[mw] == anc) {
          const float held = node_tokens(anc, LOG2C + l - 1, len);
#pragma unroll
          for (int s = 0; s < D / 32; ++s) {
            const float* kn = s_knew + 32 * s + 8 * grp;
            float4& a = x[mw][s][0];
            float4& c = x[mw][s][1];
            a = make_float4(grown_mean(a.x, kn[0], held), grown_mean(a.y, kn[1], held), grown_mean(a.z, kn[2], held),
                            grown_mean(a.w, kn[3], held));
            c = make_float4(grown_mean(c.x, kn[4], held), grown_mean(c.y, kn[5], held), grown_mean(c.z, kn[6], held),
                            grown_mean(c.w, kn[7], held));
          }
        }
        f32x4 acc = zero4();
        dot_mean_rows<T, D>(acc, x[mw], qf);
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = 8 * m + 2 * grp + a;
          const float x0 = p.scale * acc[2 * a], x1 = p.scale * acc[2 * a + 1];
          float lv = c < n_full ? lse2(x0, x1) : x0;
          lv = row_sum16(r16 < p.G ? lv : 0.f);
          if (r16 == 0) sc[c] = lv;
        }
      }
    }
    __syncthreads();
    const bool keep = topk_keep(sc[lane < n_cand ? lane : 0], n_cand, K, s_keys[wave]);
    int cnt;
    kept = compact_lanes(keep, cn, &cnt);
    kept = lane < cnt ? kept : -1;
    nk = cnt;
  }
  __syncthreads();  // every wave is past the walk before the leaf stage reuses LDS
  // ---- 2. leaf LSE and attention of this work-group's share of the candidate leaves
  const int n_leaf = 2 * nk - ((((2 * readlane(kept, nk - 1) + 1) << LOG2C) > i) ? 1 : 0);
  const T* kbh = p.k_cache + (long long)bh * p.Nmax * D;
  const T* vbh = p.v_cache + (long long)bh * p.Nmax * D;
  float* po = p.part_o + (long long)bh * p.maxc * p.G * D;
  float* pl = p.part_lse + (long long)bh * p.maxc * p.G;
  uint16_t(*vt)[C + 8] = reinterpret_cast<uint16_t(*)[C + 8]>(s_vt + wave * TILE);
  const int jnew = i >> LOG2C;  // the leaf that receives the new token
  for (int c = split * NW + wave; c < n_leaf; c += p.S * NW) {
    const int leaf = 2 * readlane(kept, c >> 1) + (c & 1);
    if (leaf == jnew) {
      // this wave completes the leaf: the new token's cache rows first (the step's end rewrites them)
      for (int e = lane; e < D; e += 64) {
        p.k_cache[((long long)bh * p.Nmax + pos) * D + e] = p.k_new[(long long)bh * D + e];
        p.v_cache[((long long)bh * p.Nmax + pos) * D + e] = p.v_new[(long long)bh * D + e];
      }
      __threadfence_block();
    }
    const long long t0 = (long long)leaf * C;
    Frag<T> kf[C / 16][D / 32];
    // the step reads each candidate leaf's K and V once: non-temporal loads, so that they pass through
    // the caches without displacing the pyramid rows the next step's walk reads
    load_attn_k<T, D, C, true>(kbh, t0, len, kf);
    Frag<T> vf[D / 16][C / 32];
    load_attn_vt<T, D, C, true>(vbh, t0, len, vt, vf);
    f32x4 oacc[MO];
    float lse, inv;
    attend_tile<T, D, C>(kf, vf, qf, t0, hv ? i : -1, p.scale, oacc, lse, inv);
    // the normalised output goes through this wave's LDS tile (free once the V^T fragments are in
    // registers), so that the device-scope stores are coalesced: lane x writes floats x, x + 64, ...
    float* s_o = reinterpret_cast<float*>(vt);
    if (hv) {
#pragma unroll
      for (int mt = 0; mt < MO; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_o[r16 * D + attn_out_dim<D>(mt, grp, j)] = oacc[mt][j] * inv;
      if (grp == 0) store_device(pl + c * p.G + r16, lse);
    }
    __threadfence_block();
    float* dst = po + (long long)c * p.G * D;
    for (int x = lane; x < p.G * D; x += 64) store_device(dst + x, s_o[x]);
    __threadfence_block();  // the tile is reused by this wave's next leaf
  }
  // ---- 3. arrival; the last work-group of the unit finishes the step. The partials are written
  // and read with device-scope accesses, which are coherent across the XCDs' L2s by themselves, so
  // the hand-over needs no L2 write-back: each wave waits until its partial stores have completed,
  // then one thread counts the work-group in.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): every store of this wave has completed
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(p.ticket + bh, 1) == p.S - 1;
  __syncthreads();
  if (!s_last) return;
  // Finishing work-group. Wave 0 loads the candidate leaves' LSEs first and ranks them; every thread
  // loads the candidate leaves' partial outputs of its first two output elements meanwhile, and
  // o = sum over the candidates of weight x output, weight 0 for the leaves the Top-K drops. The
  // append and the ancestor-path update come last: nothing waits for them.
  // wave 0, lane c: candidate leaf c's per-head LSEs, first in its load queue (the ranking needs them)
  float lh[kDecodeMaxG];
#pragma unroll
  for (int h = 0; h < kDecodeMaxG; ++h)
    lh[h] = (wave == 0 && h < p.G && lane < n_leaf) ? load_device(pl + lane * p.G + h) : kNegInf;
  constexpr int NC = 8 * KM;  // candidate leaves at most (2K)
  const int GD = p.G * D;
  float v0[NC], v1[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    v0[c] = (c < n_leaf && tid < GD) ? load_device(po + (long long)c * GD + tid) : 0.f;
    v1[c] = (c < n_leaf && tid + NT < GD) ? load_device(po + (long long)c * GD + tid + NT) : 0.f;
  }
  // waves 1-2: the new token's ancestors' sums, loaded now and written back at the very end
  const bool updater = tid >= 64 && tid < 64 + D;
  const int e = tid - 64;
  float old_sum[kMaxLevels];
  if (updater) {
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l)
      if (l < p.lv.n_levels) old_sum[l] = p.pyr_sum[(head_row + p.lv.off[l] + (pos >> (LOG2C + l))) * D + e];
  }
  if (wave == 0) {
    bool keep = lane < n_leaf;
    if (n_leaf > K) {
      float sc = 0.f;  // heads in index order
#pragma unroll
      for (int h = 0; h < kDecodeMaxG; ++h)
        if (h < p.G) sc += lh[h];
      keep = topk_keep(sc, n_leaf, K, s_keys[wave]);
    }
    int nsel;
    const int csel = compact_lanes(keep, lane, &nsel);
    const int leaf = 2 * __shfl(kept, (csel >> 1) & 63) + (csel & 1);
    if (p.sel_out && lane < K) p.sel_out[(long long)bh * K + lane] = lane < nsel ? leaf : -1;
    // merge weights per head, in candidate order: softmax of the kept leaves' LSEs, 0 elsewhere
#pragma unroll
    for (int h = 0; h < kDecodeMaxG; ++h) {
      if (h < p.G) {
        const float l = keep ? lh[h] : kNegInf;
        const float m = wave_max(l);
        const float w = keep ? fast_exp2((l - m) * kLog2e) : 0.f;
        const float den = wave_sum(w);
        if (lane < NC) s_w[lane][h] = keep ? w / den : 0.f;
      }
    }
  }
  __syncthreads();
  T* orow = p.o + ((long long)b * p.Hq + (long long)r * p.G) * D;
  {
    const int h0 = tid / D, h1 = (tid + NT) / D;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c < n_leaf) {
        if (tid < GD) a0 += s_w[c][h0] * v0[c];
        if (tid + NT < GD) a1 += s_w[c][h1] * v1[c];
      }
    }
    if (tid < GD) orow[tid] = from_f32<T>(a0);
    if (tid + NT < GD) orow[tid + NT] = from_f32<T>(a1);
  }
  for (int x = tid + 2 * NT; x < GD; x += NT) {  // more than 2 output elements per thread (large groups)
    const int h = x / D;
    float acc = 0.f;
    for (int c = 0; c < n_leaf; ++c) acc += s_w[c][h] * load_device(po + (long long)c * GD + x);
    orow[x] = from_f32<T>(acc);
  }
  // append the new token and add it to each ancestor's sum and mean
  if (updater) {
    const T kv = p.k_new[(long long)bh * D + e];
    p.k_cache[((long long)bh * p.Nmax + pos) * D + e] = kv;
    p.v_cache[((long long)bh * p.Nmax + pos) * D + e] = p.v_new[(long long)bh * D + e];
    const float kf = to_f32<T>(kv);
#pragma unroll
    for (int l = 0; l < kMaxLevels; ++l) {
      if (l < p.lv.n_levels) {
        const long long j = pos >> (LOG2C + l);
        const long long row = (head_row + p.lv.off[l] + j) * D + e;
        p.pyr_sum[row] = old_sum[l] + kf;
        p.pyr_mean[row] = grown_mean(old_sum[l], kf, node_tokens(j, LOG2C + l, len));
      }
    }
  }
  if (tid == 0) p.ticket[bh] = 0;  // every work-group of the unit has arrived: ready for the next step
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
  p.ticket = da.ticket;
  p.part_o = da.part_o;
  p.part_lse = da.part_lse;
  p.B = da.B;
  p.Hq = da.Hq;
  p.Hkv = da.Hkv;
  p.G = da.G;
  p.Nmax = da.Nmax;
  p.K = da.K;
  p.S = decode_splits(da.K);
  p.maxc = 2 * da.K;
  p.scale = da.scale;
  p.lv = da.lv;
  p.lens = da.lens;
  const int grid = da.B * da.Hkv * p.S;
  if (da.K <= 16)
    hipLaunchKernelGGL((decode_kernel<T, D, C, 4>), dim3(grid), dim3(kDecodeWaves * 64), 0, st, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, C, 8>), dim3(grid), dim3(kDecodeWaves * 64), 0, st, p);
  return hipGetLastError();
}

int decode_splits(int K) { return (2 * K + kDecodeWaves - 1) / kDecodeWaves; }

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
