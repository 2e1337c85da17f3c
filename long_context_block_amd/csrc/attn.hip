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
// Partial rows are stored in sorted-pair order (pair x owns rows x G .. x G + G - 1), so a work-group
// writes one contiguous range; the regroup leaves each pair's sorted index in pos[u K + slot].
// attn_merge combines a unit's K partials with weights exp(lse_k - LSE), LSE = LSE_k lse_k.
#include "attn_tiles.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "pair_runs.hpp"

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
  T* part;         // [pairs, G, D], rows in sorted-pair order
  float* part_lse; // [pairs, G]
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
      long long u, at;  // unit, sorted index of the pair
    };
    // A column past the run repeats the run's first pair: it computes that pair's result again and
    // stores the same bytes to the same place. Loads and stores are therefore unconditional and the
    // tile loop is straight-line code, which lets the query prefetch stay in flight across tiles.
    auto fetch = [&](Tile& t, long long tp) {
      const long long pi = tp + r16 / p.G;
      t.at = pi < seg ? pi : pos;
      const uint32_t pc = run.pair(t.at);
      t.u = pc >> 5;
      const T* qrow = qhead + (t.u - ubase) * D;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) t.qf[s].load(qrow + 32 * s);
    };
    auto attend = [&](const Tile& cur) {
      Frag<T> qf[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) qf[s] = cur.qf[s];
      f32x4 oacc[MO];
      float lse, inv;
      attend_tile<T, D, C>(kf, vf, qf, t0, cur.u - ubase, p.scale, oacc, lse, inv);
      const long long prow = cur.at * p.G + h;
      // lane group grp holds dimensions 32 c + 8 grp .. +8 in oacc[2c], oacc[2c + 1]
      T* dst = p.part + prow * D + 8 * grp;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int c = 0; c < MO / 2; ++c) {
          uint4 w;
          w.x = pack_bf16x2(oacc[2 * c][0] * inv, oacc[2 * c][1] * inv);
          w.y = pack_bf16x2(oacc[2 * c][2] * inv, oacc[2 * c][3] * inv);
          w.z = pack_bf16x2(oacc[2 * c + 1][0] * inv, oacc[2 * c + 1][1] * inv);
          w.w = pack_bf16x2(oacc[2 * c + 1][2] * inv, oacc[2 * c + 1][3] * inv);
          *reinterpret_cast<uint4*>((uint16_t*)dst + 32 * c) = w;
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MO; ++mt)
          *reinterpret_cast<float4*>((float*)dst + 32 * (mt >> 1) + 4 * (mt & 1)) =
              make_float4(oacc[mt][0] * inv, oacc[mt][1] * inv, oacc[mt][2] * inv, oacc[mt][3] * inv);
      }
      p.part_lse[prow] = lse;  // the column's 4 lanes hold the same value
    };
    // ring of R tiles in groups of R: the query fragments of tile t + R are requested as tile t
    // finishes
    constexpr int R = 2;
    const long long step = tile_units;
    // the run length is wave-uniform; readfirstlane lets the compiler see it (a scalar loop)
    const int run_len = __builtin_amdgcn_readfirstlane((int)(seg - pos));
    const int ntiles = (run_len + tile_units - 1) / tile_units;
    const int ngroups = (ntiles + R - 1) / R;
    Tile X[R];
#pragma unroll
    for (int r = 0; r < R; ++r) fetch(X[r], pos + r * step);
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        attend(X[r]);
        fetch(X[r], pos + (long long)((gi + 1) * R + r) * step);
      }
    }
    pos = seg;
  }
}

// bf16, work-group cooperative. A work-group task is kWgTask consecutive sorted pairs; its runs (one
// leaf each) are found once. For each run the 256 threads stage the leaf's K (swizzled) and V^T into
// LDS, then the four waves take the run's tiles of 16/G units x G heads round-robin, reading every
// MFMA fragment of K and V^T from LDS. Sharing the tiles keeps registers low (three waves per SIMD
// hide the query-gather latency) and loads each leaf's K/V once per work-group instead of per wave.
constexpr int kWgTask = 1024;

template <int D, int C>
__global__ __launch_bounds__(256, 3) void attn_leaf_wg_kernel(AttnParams<uint16_t> p) {
  constexpr int MO = D / 16;
  __shared__ __align__(16) uint16_t s_k[C][D];
  __shared__ __align__(16) uint16_t s_vt[D][C + 8];
  __shared__ uint32_t s_pair[kWgTask];
  __shared__ long long s_key[kWgTask];
  __shared__ int s_run[kWgTask + 1];
  __shared__ int s_wcount[4];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long total = *p.total;
  const long long base = (long long)xcd_logical_block(gridDim.x) * kWgTask;
  if (base >= total) return;  // whole work-group
  const int n = (int)(total - base < kWgTask ? total - base : kWgTask);
  const long long nch = ((long long)p.N + (1LL << p.chunk_log2) - 1) >> p.chunk_log2;
  // pairs, their bucket keys (KV head, position chunk, leaf) and the runs of equal keys
  const int nrun = stage_pair_runs<kWgTask>(
      p.pairs, base, n,
      [&](uint32_t pr) {
        const long long u = pr >> 5;
        const unsigned bh = (unsigned)u / (unsigned)p.N, i = (unsigned)u - bh * (unsigned)p.N;  // u < 2^27
        return ((long long)bh * nch + (i >> p.chunk_log2)) * (1LL << 32) + p.sel[u * p.K + (pr & 31)];
      },
      s_pair, s_key, s_run, s_wcount);
  const int tile_units = 16 / p.G;
  const int h = r16 % p.G;
  for (int r = 0; r < nrun; ++r) {
    const int a = s_run[r], b = s_run[r + 1];
    const long long u0 = s_pair[a] >> 5;
    const long long bh = u0 / p.N;
    const int leaf = (int)(s_key[a] & 0xffffffffLL);
    const long long t0 = (long long)leaf * C;
    const uint16_t* kbh = p.k + bh * (long long)p.N * D;
    const uint16_t* vbh = p.v + bh * (long long)p.N * D;
    stage_kv_wg<D, C>(kbh, vbh, t0, p.N, s_k, s_vt);
    __syncthreads();
    const int bi = (int)(bh / p.Hkv), ri = (int)(bh % p.Hkv);
    const int qr = quad_row(), hq = qr % p.G;
    const uint16_t* qhead = p.q + (((long long)bi * p.Hq + (long long)ri * p.G + hq) * p.N) * D + 8 * quad_chunk();
    const long long ubase = bh * p.N;
    const int ntiles = (b - a + tile_units - 1) / tile_units;
    // The query fragments of tile t + 4 (this wave's next tile) are requested before tile t is
    // computed. A column past the run, or past the wave's last tile, repeats the run's first pair:
    // same result, same bytes, same place. The loads are quad-coalesced (lane 4 r + g reads row r);
    // quad_rows_to_mfma() before use.
    // xc is the column's pair (its index in the task)
    auto fetch = [&](int t, Frag<uint16_t> (&qf)[D / 32], int& xc) {
      int xl = a + t * tile_units + qr / p.G;
      xl = (t < ntiles && xl < b) ? xl : a;
      const uint16_t* qrow = qhead + ((long long)(s_pair[xl] >> 5) - ubase) * D;
#pragma unroll
      for (int s2 = 0; s2 < D / 32; ++s2) qf[s2].load(qrow + 32 * s2);
      const int x = a + t * tile_units + r16 / p.G;
      xc = (t < ntiles && x < b) ? x : a;
    };
    struct Out {
      f32x4 o[MO];
      float lse, inv;
      int xc;
    };
    auto attend = [&](Frag<uint16_t> (&qf)[D / 32], int xc, Out& out) {
      out.xc = xc;
      quad_rows_to_mfma(qf);
      attend_tile_kv<uint16_t, D, C, true>([&](int m, int s2) { return k_frag_wg<D>(s_k, m, s2); },
                                           [&](int mt, int ks) { return vt_frag<C>(s_vt, mt, ks); }, qf, t0,
                                           (long long)(s_pair[xc] >> 5) - ubase, p.scale, out.o, out.lse, out.inv);
    };
    // partial rows in sorted-pair order: a tile's rows are contiguous
    auto store = [&](const Out& out) {
      const long long prow = (base + out.xc) * p.G + h;
      const long long prow_o = (base + row_partner(out.xc)) * p.G + (r16 ^ 8) % p.G;  // row r16 ^ 8
      // lane group grp holds dimensions 32 c + 8 grp .. +8 in o[2c], o[2c + 1]
      const float inv = out.inv;
      uint4 w[MO / 2];
#pragma unroll
      for (int c = 0; c < MO / 2; ++c) {
        w[c].x = pack_bf16x2(out.o[2 * c][0] * inv, out.o[2 * c][1] * inv);
        w[c].y = pack_bf16x2(out.o[2 * c][2] * inv, out.o[2 * c][3] * inv);
        w[c].z = pack_bf16x2(out.o[2 * c + 1][0] * inv, out.o[2 * c + 1][1] * inv);
        w[c].w = pack_bf16x2(out.o[2 * c + 1][2] * inv, out.o[2 * c + 1][3] * inv);
      }
      store_rows_lines<D>(p.part + prow * D + 8 * grp, p.part + prow_o * D + 8 * grp, w);
      if (grp == 0) p.part_lse[prow] = out.lse;  // the column's 4 lanes hold the same value
    };
    if (wave < ntiles) {
      // two register sets in turn: this wave's tiles t and t + 4 are computed while the queries of
      // t + 8 and t + 12 are in flight (a tile past the end repeats the run's first pair); each
      // prefetch is issued before the stores of the tile just computed
      Frag<uint16_t> qa[D / 32], qb[D / 32];
      int pa, pb;
      fetch(wave, qa, pa);
      fetch(wave + 4, qb, pb);
      opaque_frags(qa);
      opaque_frags(qb);
      for (int t = wave; t < ntiles; t += 8) {
        Out out;
        attend(qa, pa, out);
        fetch(t + 8, qa, pa);
        store(out);
        attend(qb, pb, out);
        fetch(t + 12, qb, pb);
        store(out);
      }
    }
    __syncthreads();  // every wave is done with this leaf's tiles before they are restaged
  }
}

template <typename T>
struct MergeParams {
  const int* sel;
  const int* pos;  // [U, K]: sorted index of the pair (u, slot), the row block of its partials
  const T* part;
  const float* part_lse;
  int B, Hq, Hkv, G, N, K;
  T* o;
  float* o_lse;
};

// Merge. A (unit, head) output row is one task, handled by DC = D / E lanes (E elements per 16-byte
// chunk); a wave takes 64 / DC consecutive tasks, so for G >= 64 / DC its loads of one slot cover the
// unit's G heads in one contiguous run. Per task: M = max_k lse_k, S = sum_k exp(lse_k - M),
// o = sum_k (exp(lse_k - M) / S) partial_k, LSE = M + ln S. Slots k < nsel hold the selected leaves
// (selections are left-packed), so only those partial rows are read, found through pos.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams<T> p) {
  constexpr int E = 16 / (int)sizeof(T);  // elements per chunk
  constexpr int DC = D / E;               // lanes per task
  constexpr int KJ = (32 + DC - 1) / DC;  // lse registers per lane (K <= 32)
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int li = lane % DC, base = lane - li;
  const long long U = (long long)p.B * p.Hkv * p.N;
  const long long task = ((long long)xcd_logical_block(gridDim.x) * 4 + wave) * (64 / DC) + lane / DC;
  const bool live = task < U * p.G;
  const long long u = live ? task / p.G : 0;
  const int h = (int)(task % p.G);
  // selected slots of u (left-packed)
  int nsel = 0;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int kk = li + j * DC;
    const bool has = live && kk < p.K && p.sel[u * p.K + kk] >= 0;
    const uint64_t m = __ballot(has);
    nsel += __popcll((m >> base) & (DC == 64 ? ~0ull : ((1ull << DC) - 1)));
  }
  float lv[KJ];
  int at[KJ];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    const int kk = li + j * DC;
    at[j] = kk < nsel ? p.pos[u * p.K + kk] : 0;
    lv[j] = kk < nsel ? p.part_lse[(long long)at[j] * p.G + h] : kNegInf;
    mx = fmaxf(mx, lv[j]);
  }
#pragma unroll
  for (int o = 1; o < DC; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float ws = 0.f;
#pragma unroll
  for (int j = 0; j < KJ; ++j) {
    lv[j] = lv[j] == kNegInf ? 0.f : fast_exp2((lv[j] - mx) * kLog2e);
    ws += lv[j];
  }
#pragma unroll
  for (int o = 1; o < DC; o <<= 1) ws += __shfl_xor(ws, o);
  const float rs = ws > 0.f ? 1.f / ws : 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  // the wave's tasks may have different nsel: loop to the wave's largest, lanes past theirs add 0
  int nmax = nsel;
#pragma unroll
  for (int o = DC; o < 64; o <<= 1) nmax = max(nmax, __shfl_xor(nmax, o));
  const T* src = p.part + (long long)h * D + li * E;
  for (int kk = 0; kk < nmax; ++kk) {
    float w = __shfl(lv[0], base + (kk % DC));
    int ak = __shfl(at[0], base + (kk % DC));
#pragma unroll
    for (int j = 1; j < KJ; ++j) {
      const float wj = __shfl(lv[j], base + (kk % DC));
      const int aj = __shfl(at[j], base + (kk % DC));
      w = (kk / DC == j) ? wj : w;
      ak = (kk / DC == j) ? aj : ak;
    }
    if (kk < nsel) {
      w *= rs;
      const T* row = src + (long long)ak * p.G * D;
      if constexpr (sizeof(T) == 2) {
        const uint4 x = *reinterpret_cast<const uint4*>(row);
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += w * __uint_as_float(xs[e] << 16);
          acc[2 * e + 1] += w * __uint_as_float(xs[e] & 0xffff0000u);
        }
      } else {
        const float4 x = *reinterpret_cast<const float4*>(row);
        acc[0] += w * x.x;
        acc[1] += w * x.y;
        acc[2] += w * x.z;
        acc[3] += w * x.w;
      }
    }
  }
  if (!live) return;
  const long long bh = u / p.N, i = u % p.N;
  const int b = (int)(bh / p.Hkv), r = (int)(bh % p.Hkv);
  const long long orow = ((long long)b * p.Hq + (long long)r * p.G + h) * p.N + i;
  T* dst = p.o + orow * D + li * E;
  if constexpr (sizeof(T) == 2) {
    uint4 w;
    w.x = pack_bf16x2(acc[0], acc[1]);
    w.y = pack_bf16x2(acc[2], acc[3]);
    w.z = pack_bf16x2(acc[4], acc[5]);
    w.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(dst) = w;
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  if (p.o_lse && li == 0) p.o_lse[orow] = ws > 0.f ? mx + kLn2 * fast_log2(ws) : kNegInf;
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
  if constexpr (sizeof(T) == 2) {
    const long long wg = (max_pairs + kWgTask - 1) / kWgTask;
    p.tasks = (int)wg;
    hipLaunchKernelGGL((attn_leaf_wg_kernel<D, C>), dim3((unsigned)wg), dim3(256), 0, st, p);
  } else {
    const long long tasks = (max_pairs + kAttnTask - 1) / kAttnTask;
    p.tasks = (int)tasks;
    hipLaunchKernelGGL((attn_leaf_kernel<T, D, C>), dim3((unsigned)((tasks + 3) / 4)), dim3(256), 0, st, p);
  }
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
static hipError_t merge_t(const SelDims& sd, const int* sel, const int* pos, const void* part,
                          const float* part_lse, void* o, float* o_lse, hipStream_t st) {
  MergeParams<T> p;
  p.sel = sel;
  p.pos = pos;
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
  const long long tasks = (long long)sd.B * sd.Hkv * sd.N * sd.G;
  constexpr int per_wave = 64 / (D / (16 / (int)sizeof(T)));
  const long long waves = (tasks + per_wave - 1) / per_wave;
  hipLaunchKernelGGL((attn_merge_kernel<T, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_attn_merge(const SelDims& sd, const int* sel, const int* pos, const void* part,
                             const float* part_lse, void* o, float* o_lse, hipStream_t st) {
  if (sd.bf16) return sd.D == 128 ? merge_t<uint16_t, 128>(sd, sel, pos, part, part_lse, o, o_lse, st)
                                  : merge_t<uint16_t, 64>(sd, sel, pos, part, part_lse, o, o_lse, st);
  return sd.D == 128 ? merge_t<float, 128>(sd, sel, pos, part, part_lse, o, o_lse, st)
                     : merge_t<float, 64>(sd, sel, pos, part, part_lse, o, o_lse, st);
}

}  // namespace pisa
