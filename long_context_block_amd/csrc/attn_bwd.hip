// Backward of block-sparse attention ("Block Sparse Attention with Log-Linear Complexity" digest, 工作参考
// 价值 fourth bullet: in training the gradients pass only through the selected attention, the discrete
// selection is not differentiated; the arxiv abstract: kernels for training and inference).
//
// For each (b, h, i) with T = the selected leaves' tokens t <= i, p_t = exp(s q . k_t - lse) (lse from the
// forward), dp_t = dO . v_t, D = dO . o, ds_t = p_t (dp_t - D):
//   dq = s sum_t ds_t k_t,   dk_t += s ds_t q,   dv_t += p_t dO   (summed over heads and queries).
// Leaf-major, on the forward's regroup (pairs bucketed by selected leaf):
//   prep:  D per query row; the fp32 dK / dV accumulators cleared.
//   dq:    the forward's work-group schedule: per run (one leaf) K, V (row tiles) and K^T are staged in
//          LDS; per tile of 16 (unit, head) columns S = K q^T and dP = V dO^T on MFMA, dS = P (dP - D),
//          dq^T = K^T dS; one unscaled partial row per (pair, head) in sorted-pair order.
//   dkdv:  per run, wave w owns tokens 16 w .. 16 w + 15 of the leaf (C = 32: two waves per slice, on
//          alternate tile pairs); tiles of 32 columns (q, dO rows and their transposes staged in LDS);
//          S^T = q K_w^T with the column rows permuted so that P^T and dS^T come out in the B-operand layout
//          of the next products; dv^T += dO^T P^T, dk^T += q^T dS^T in registers (C = 32: the two waves of
//          a slice add theirs through LDS). At the end of the run the sums go to the fp32 accumulators when
//          no other task holds pairs of the leaf, else to one of the task's two slots, which bwd_kv_reduce
//          adds up per leaf in task order (no atomics: they took a third of the backward's time).
//   merge: dq = s * sum of the unit's partial rows; finish: the accumulators in the output type.
#include "attn_tiles.hpp"
#include "common.hpp"
#include "internal.hpp"
#include "pair_runs.hpp"

namespace pisa {

constexpr int kWgTaskBwd = 1024;  // sorted pairs per work-group task (dq)
// dkdv: 512-pair tasks, so that two work-groups (77 KiB of LDS each) share a CU
constexpr int kWgTaskDkdv = 512;

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* d_o;
  const float* o_lse;
  const int* sel;
  const uint32_t* pairs;
  const int* total;
  const float* dsum;  // [B, Hq, N]: dO . o
  int B, Hq, Hkv, G, N, K, chunk_log2;
  float scale;
  uint16_t* part;  // [pairs, G, D] unscaled dq partials (dq pass)
  float* dk_acc;   // [B, Hkv, N, D]
  float* dv_acc;
  float* kv_part;  // [dkdv tasks, 2 slots, 2 (dk, dv), C, D] sums of runs shared with another task
};

// ------------------------------------------------------------------------------------------ prep
// D = dO . o per query row (16 lanes per row of D = 128, 8 per row of 64); clears the accumulators.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ d_o,
                                                       long long rows, float* __restrict__ dsum, float* __restrict__ acc,
                                                       long long acc_n) {
  constexpr int LPR = D / 8;  // lanes per row
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / LPR;
  const int li = (int)(gid % LPR);
  float x = 0.f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + 8 * li);
    const uint4 b = *reinterpret_cast<const uint4*>(d_o + row * D + 8 * li);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x = fmaf(__uint_as_float(av[e] << 16), __uint_as_float(bv[e] << 16), x);
      x = fmaf(__uint_as_float(av[e] & 0xffff0000u), __uint_as_float(bv[e] & 0xffff0000u), x);
    }
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) x += __shfl_xor(x, off);
  if (row < rows && li == 0) dsum[row] = x;
  for (long long j = gid; j < acc_n; j += (long long)gridDim.x * blockDim.x) acc[j] = 0.f;
}

// ------------------------------------------------------------------------------------------ dq pass
template <int D, int C>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdParams p) {
  constexpr int MS = C / 16, KS = C / 32, MO = D / 16;
  __shared__ __align__(16) uint16_t s_k[C][D];
  __shared__ __align__(16) uint16_t s_v[C][D];
  __shared__ __align__(16) uint16_t s_kt[D][C + 8];
  __shared__ uint32_t s_pair[kWgTaskBwd];
  __shared__ long long s_key[kWgTaskBwd];
  __shared__ int s_run[kWgTaskBwd + 1];
  __shared__ int s_wcount[4];
  const int lane = lane_id(), wave = threadIdx.x >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long total = *p.total;
  const long long base = (long long)xcd_logical_block(gridDim.x) * kWgTaskBwd;
  if (base >= total) return;
  const int n = (int)(total - base < kWgTaskBwd ? total - base : kWgTaskBwd);
  const long long nch = ((long long)p.N + (1LL << p.chunk_log2) - 1) >> p.chunk_log2;
  const int nrun = stage_pair_runs<kWgTaskBwd>(
      p.pairs, base, n,
      [&](uint32_t pr) {
        const long long u = pr >> 5;
        const unsigned bh = (unsigned)u / (unsigned)p.N, i = (unsigned)u - bh * (unsigned)p.N;
        return ((long long)bh * nch + (i >> p.chunk_log2)) * (1LL << 32) + p.sel[u * p.K + (pr & 31)];
      },
      s_pair, s_key, s_run, s_wcount);
  const int tile_units = 16 / p.G;
  const int h = r16 % p.G;
  const float c2 = p.scale * kLog2e;
  for (int r = 0; r < nrun; ++r) {
    const int a = s_run[r], b = s_run[r + 1];
    const long long u0 = s_pair[a] >> 5;
    const long long bh = u0 / p.N;
    const int leaf = (int)(s_key[a] & 0xffffffffLL);
    const long long t0 = (long long)leaf * C;
    const uint16_t* kbh = p.k + bh * (long long)p.N * D;
    const uint16_t* vbh = p.v + bh * (long long)p.N * D;
    stage_kv_wg<D, C>(kbh, kbh, t0, p.N, s_k, s_kt);  // K rows and K^T
    stage_rows_wg<D, C>(vbh, t0, p.N, s_v);           // V rows
    __syncthreads();
    const int bi = (int)(bh / p.Hkv), ri = (int)(bh % p.Hkv);
    const long long hrow = (long long)bi * p.Hq + (long long)ri * p.G;  // first query head of the group
    const int qr = quad_row(), hq = qr % p.G;
    const uint16_t* qhead = p.q + ((hrow + hq) * p.N) * D + 8 * quad_chunk();
    const uint16_t* ohead = p.d_o + ((hrow + hq) * p.N) * D + 8 * quad_chunk();
    const long long ubase = bh * p.N;
    const int ntiles = (b - a + tile_units - 1) / tile_units;
    for (int t = wave; t < ntiles; t += 4) {
      // columns past the run repeat the run's first pair: same values, same place
      int xl = a + t * tile_units + qr / p.G;
      xl = xl < b ? xl : a;
      const long long uq = (long long)(s_pair[xl] >> 5) - ubase;
      Frag<uint16_t> qf[D / 32], of[D / 32];
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        qf[s].load(qhead + uq * D + 32 * s);
        of[s].load(ohead + uq * D + 32 * s);
      }
      quad_rows_to_mfma(qf);
      quad_rows_to_mfma(of);
      int xc = a + t * tile_units + r16 / p.G;
      xc = xc < b ? xc : a;
      const long long ic = (long long)(s_pair[xc] >> 5) - ubase;  // the column's position
      const long long crow = (hrow + h) * p.N + ic;
      const float lse = p.o_lse[crow] * kLog2e, dsum = p.dsum[crow];
      f32x4 sacc[MS], dacc[MS];
#pragma unroll
      for (int m = 0; m < MS; ++m) {
        sacc[m] = zero4();
        dacc[m] = zero4();
      }
      // S, then dP: one operand set live at a time
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
#pragma unroll
        for (int m = 0; m < MS; ++m) mma(sacc[m], k_frag_wg<D>(s_k, m, s), qf[s]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
#pragma unroll
        for (int m = 0; m < MS; ++m) mma(dacc[m], k_frag_wg<D>(s_v, m, s), of[s]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const long long lim = ic - t0;
#pragma unroll
      for (int m = 0; m < MS; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool vis = attn_token(m, grp, j) <= lim;
          const float pr = vis ? fast_exp2(fmaf(sacc[m][j], c2, -lse)) : 0.f;
          sacc[m][j] = pr * (dacc[m][j] - dsum);  // dS
        }
      Frag<uint16_t> df[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        df[ks].u.x = pack_bf16x2(sacc[2 * ks][0], sacc[2 * ks][1]);
        df[ks].u.y = pack_bf16x2(sacc[2 * ks][2], sacc[2 * ks][3]);
        df[ks].u.z = pack_bf16x2(sacc[2 * ks + 1][0], sacc[2 * ks + 1][1]);
        df[ks].u.w = pack_bf16x2(sacc[2 * ks + 1][2], sacc[2 * ks + 1][3]);
      }
      f32x4 qacc[MO];
#pragma unroll
      for (int mt = 0; mt < MO; ++mt) {
        qacc[mt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) mma(qacc[mt], vt_frag<C>(s_kt, mt, ks), df[ks]);
      }
      // lane group grp holds dimensions 32 c + 8 grp .. +8 in qacc[2c], qacc[2c + 1]
      uint4 w[MO / 2];
#pragma unroll
      for (int c = 0; c < MO / 2; ++c) {
        w[c].x = pack_bf16x2(qacc[2 * c][0], qacc[2 * c][1]);
        w[c].y = pack_bf16x2(qacc[2 * c][2], qacc[2 * c][3]);
        w[c].z = pack_bf16x2(qacc[2 * c + 1][0], qacc[2 * c + 1][1]);
        w[c].w = pack_bf16x2(qacc[2 * c + 1][2], qacc[2 * c + 1][3]);
      }
      const long long prow = (base + xc) * p.G + h;
      const long long prow_o = (base + row_partner(xc)) * p.G + (r16 ^ 8) % p.G;  // row r16 ^ 8
      store_rows_lines<D>(p.part + prow * D + 8 * grp, p.part + prow_o * D + 8 * grp, w);
    }
    __syncthreads();  // every wave is done with this leaf's tiles before they are restaged
  }
}

// ------------------------------------------------------------------------------------------ dkdv pass
constexpr int kBwdCols = 32;  // columns per tile pair

// The transposed column tiles (row = dimension, 32 columns): 16-byte chunk k of row r is stored at chunk
// k ^ ((r >> 5) & 3), so that the staging writes of one wave, which span dimensions 32 apart, fall on
// different banks. colt_frag reads the B-operand fragment of rows 16 mt .. 16 mt + 15 (k = the columns).
__device__ __forceinline__ int colt_chunk(int row, int k) { return k ^ ((row >> 5) & 3); }
__device__ __forceinline__ Frag<uint16_t> colt_frag(const uint16_t (*t)[kBwdCols + 8], int mt) {
  const int r16 = lane_id() & 15, grp = lane_id() >> 4;
  const int row = 16 * mt + r16;
  Frag<uint16_t> f;
  f.u = *reinterpret_cast<const uint4*>(&t[row][8 * colt_chunk(row, grp)]);
  return f;
}

template <int D, int C>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_kernel(BwdParams p) {
  constexpr int MO = D / 16;
  constexpr int NSL = C / 16;  // token slices of 16
  __shared__ __align__(16) uint16_t s_k[C][D];
  __shared__ __align__(16) uint16_t s_v[C][D];
  __shared__ __align__(16) uint16_t s_q[kBwdCols][D];
  __shared__ __align__(16) uint16_t s_do[kBwdCols][D];
  __shared__ __align__(16) uint16_t s_qt[D][kBwdCols + 8];
  __shared__ __align__(16) uint16_t s_dot[D][kBwdCols + 8];
  __shared__ float s_lse[kBwdCols], s_dsum[kBwdCols];
  __shared__ long long s_pos[kBwdCols];
  __shared__ uint32_t s_pair[kWgTaskDkdv];
  __shared__ long long s_key[kWgTaskDkdv];
  __shared__ uint16_t s_run[kWgTaskDkdv + 1];
  __shared__ int s_wcount[4];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6, r16 = lane & 15, grp = lane >> 4;
  const long long total = *p.total;
  const long long base = (long long)xcd_logical_block(gridDim.x) * kWgTaskDkdv;
  if (base >= total) return;
  const int n = (int)(total - base < kWgTaskDkdv ? total - base : kWgTaskDkdv);
  const long long nch = ((long long)p.N + (1LL << p.chunk_log2) - 1) >> p.chunk_log2;
  auto key_of = [&](uint32_t pr) {
    const long long u = pr >> 5;
    const unsigned bh = (unsigned)u / (unsigned)p.N, i = (unsigned)u - bh * (unsigned)p.N;
    return ((long long)bh * nch + (i >> p.chunk_log2)) * (1LL << 32) + p.sel[u * p.K + (pr & 31)];
  };
  const int nrun = stage_pair_runs<kWgTaskDkdv>(p.pairs, base, n, key_of, s_pair, s_key, s_run, s_wcount);
  // A run whose leaf has pairs in no other task stores its sums straight to the accumulators; the task's
  // first run, if its leaf began in an earlier task, and its last run, if its leaf goes on in a later one,
  // store them to the task's slots 0 and 1 (the first run takes slot 0 when it is also the last), and
  // bwd_kv_reduce adds a leaf's slots in task order.
  __shared__ int s_cont[2];  // the first run continues an earlier task's; the last run goes on
  if (tid == 0) {
    s_cont[0] = base > 0 && key_of(p.pairs[base - 1]) == s_key[0];
    s_cont[1] = base + n < total && key_of(p.pairs[base + n]) == s_key[n - 1];
  }
  // this wave's token slice, and (C = 32) which tile pairs it takes
  const int slice = wave % NSL, phase = wave / NSL, nphase = 4 / NSL;
  const int units_per_pair = kBwdCols / p.G;
  const float c2 = p.scale * kLog2e;
  constexpr int CHR = D / 8;  // 16-byte chunks per row
  for (int r = 0; r < nrun; ++r) {
    const int a = s_run[r], b = s_run[r + 1];
    const long long u0 = s_pair[a] >> 5;
    const long long bh = u0 / p.N;
    const int leaf = (int)(s_key[a] & 0xffffffffLL);
    const long long t0 = (long long)leaf * C;
    stage_rows_wg<D, C>(p.k + bh * (long long)p.N * D, t0, p.N, s_k);
    stage_rows_wg<D, C>(p.v + bh * (long long)p.N * D, t0, p.N, s_v);
    __syncthreads();
    // B operands of this wave's tokens (lane (t, g): row 16 slice + t, chunk 4 s + g)
    Frag<uint16_t> bk[D / 32], bv[D / 32];
    {
      const int tt = 16 * slice + r16;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        bk[s].u = *reinterpret_cast<const uint4*>(&s_k[tt][8 * ((4 * s + grp) ^ kswz<D>(tt))]);
        bv[s].u = *reinterpret_cast<const uint4*>(&s_v[tt][8 * ((4 * s + grp) ^ kswz<D>(tt))]);
      }
    }
    f32x4 dva[MO], dka[MO];
#pragma unroll
    for (int mt = 0; mt < MO; ++mt) {
      dva[mt] = zero4();
      dka[mt] = zero4();
    }
    const int bi = (int)(bh / p.Hkv), ri = (int)(bh % p.Hkv);
    const long long hrow = (long long)bi * p.Hq + (long long)ri * p.G;
    const long long ubase = bh * p.N;
    const int npairs = (b - a + units_per_pair - 1) / units_per_pair;
    // A tile pair's 32 columns: column c = (unit a + tp * 32 / G + c / G, head c % G); a column past the
    // run has position -1 (every score masked) and zero rows. Its q and dO rows, LSE and D are fetched
    // into registers one tile pair ahead, so that the gathers are in flight while the previous tile pair
    // computes. A thread takes chunk ch of the rows of the column pair (2 cp, 2 cp + 1), item
    // x = tid + 256 it, so that it writes the transposed tiles as 32-bit column pairs.
    constexpr int CP = kBwdCols / 2;
    constexpr int SIT = (CP * CHR + 255) / 256;
    uint4 fq[SIT][2], fo[SIT][2];
    long long fpos = -1;
    float fl = 0.f, fds = 0.f;
    auto fetch = [&](int tp) {
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int x = tid + 256 * it;
        const int cp = x / CHR, ch = x % CHR;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int c = 2 * cp + k2;
          const int xu = a + tp * units_per_pair + c / p.G;
          fq[it][k2] = fo[it][k2] = make_uint4(0u, 0u, 0u, 0u);
          if (x < CP * CHR && xu < b) {
            const long long row = (hrow + c % p.G) * p.N + ((long long)(s_pair[xu] >> 5) - ubase);
            fq[it][k2] = *reinterpret_cast<const uint4*>(p.q + row * D + 8 * ch);
            fo[it][k2] = *reinterpret_cast<const uint4*>(p.d_o + row * D + 8 * ch);
          }
        }
      }
      if (tid < kBwdCols) {
        const int xu = a + tp * units_per_pair + tid / p.G;
        fpos = -1;
        fl = fds = 0.f;
        if (xu < b) {
          fpos = (long long)(s_pair[xu] >> 5) - ubase;
          const long long row = (hrow + tid % p.G) * p.N + fpos;
          fl = p.o_lse[row];
          fds = p.dsum[row];
        }
      }
    };
    fetch(0);
    for (int tp = 0; tp < npairs; ++tp) {
      // stage the fetched tile pair: rows (swizzled), and the transposes for the dV / dK products
#pragma unroll
      for (int it = 0; it < SIT; ++it) {
        const int x = tid + 256 * it;
        if (x >= CP * CHR) continue;
        const int cp = x / CHR, ch = x % CHR;
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int c = 2 * cp + k2;
          *reinterpret_cast<uint4*>(&s_q[c][8 * (ch ^ kswz<D>(c))]) = fq[it][k2];
          *reinterpret_cast<uint4*>(&s_do[c][8 * (ch ^ kswz<D>(c))]) = fo[it][k2];
        }
        const uint32_t q0[4] = {fq[it][0].x, fq[it][0].y, fq[it][0].z, fq[it][0].w};
        const uint32_t q1[4] = {fq[it][1].x, fq[it][1].y, fq[it][1].z, fq[it][1].w};
        const uint32_t o0[4] = {fo[it][0].x, fo[it][0].y, fo[it][0].z, fo[it][0].w};
        const uint32_t o1[4] = {fo[it][1].x, fo[it][1].y, fo[it][1].z, fo[it][1].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // element e of both columns: the low half from column 2 cp, the high half from 2 cp + 1
          const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
          const int dr = attn_vt_row<D>(8 * ch + e);
          const int col = 8 * colt_chunk(dr, cp >> 2) + 2 * (cp & 3);
          *reinterpret_cast<uint32_t*>(&s_qt[dr][col]) = __builtin_amdgcn_perm(q1[e >> 1], q0[e >> 1], sel);
          *reinterpret_cast<uint32_t*>(&s_dot[dr][col]) = __builtin_amdgcn_perm(o1[e >> 1], o0[e >> 1], sel);
        }
      }
      if (tid < kBwdCols) {
        s_pos[tid] = fpos;
        s_lse[tid] = fl * kLog2e;
        s_dsum[tid] = fds;
      }
      __syncthreads();
      if (tp + 1 < npairs) fetch(tp + 1);
      if (tp % nphase == phase) {
        // S^T and dP^T: rows = the 32 columns (permuted so that lane group g ends up with columns
        // 8 g .. 8 g + 7), columns = this wave's 16 tokens
        f32x4 sacc[2], dacc[2];
        sacc[0] = sacc[1] = dacc[0] = dacc[1] = zero4();
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            mma(sacc[m], k_frag_wg<D>(s_q, m, s), bk[s]);
            mma(dacc[m], k_frag_wg<D>(s_do, m, s), bv[s]);
          }
        const long long tok = t0 + 16 * slice + r16;
        Frag<uint16_t> pf, df;
        float pv[8], dv[8];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = attn_token(m, grp, j);  // 8 grp + 4 m + j
            const bool vis = tok <= s_pos[c];
            const float pr = vis ? fast_exp2(fmaf(sacc[m][j], c2, -s_lse[c])) : 0.f;
            pv[4 * m + j] = pr;
            dv[4 * m + j] = pr * (dacc[m][j] - s_dsum[c]);
          }
        pf.u = make_uint4(pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3]), pack_bf16x2(pv[4], pv[5]),
                          pack_bf16x2(pv[6], pv[7]));
        df.u = make_uint4(pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3]), pack_bf16x2(dv[4], dv[5]),
                          pack_bf16x2(dv[6], dv[7]));
#pragma unroll
        for (int mt = 0; mt < MO; ++mt) {
          mma(dva[mt], colt_frag(s_dot, mt), pf);
          mma(dka[mt], colt_frag(s_qt, mt), df);
        }
      }
      __syncthreads();  // the tile pair is consumed before the next one is staged
    }
    // the run's contributions: lane (t, g) holds dims attn_out_dim(mt, g, j) of token 16 slice + t
    // (4 consecutive dimensions per M-tile)
    const long long tok = t0 + 16 * slice + r16;
    if constexpr (NSL == 2) {
      // C = 32: the phase-1 wave of each slice hands its sums to the phase-0 wave through the staging
      // tiles, which the tile pairs no longer use (16 D floats per array and wave, the same lane layout)
      float* xv = reinterpret_cast<float*>(slice == 0 ? (void*)&s_q[0][0] : (void*)&s_qt[0][0]);
      float* xk = reinterpret_cast<float*>(slice == 0 ? (void*)&s_do[0][0] : (void*)&s_dot[0][0]);
      if (phase == 1) {
#pragma unroll
        for (int mt = 0; mt < MO; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            xv[(mt * 4 + j) * 64 + lane] = dva[mt][j];
            xk[(mt * 4 + j) * 64 + lane] = dka[mt][j];
          }
      }
      __syncthreads();
      if (phase == 0) {
#pragma unroll
        for (int mt = 0; mt < MO; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            dva[mt][j] += xv[(mt * 4 + j) * 64 + lane];
            dka[mt][j] += xk[(mt * 4 + j) * 64 + lane];
          }
      }
    }
    if (phase == 0) {
      const bool shared = (a == 0 && s_cont[0]) || (b == n && s_cont[1]);
      float* dkr;
      float* dvr;
      if (shared) {
        const long long task = base / kWgTaskDkdv;
        float* slot = p.kv_part + (task * 2 + (a == 0 ? 0 : 1)) * 2 * C * D;
        dkr = slot + (16 * slice + r16) * D;
        dvr = dkr + C * D;
      } else {
        dkr = p.dk_acc + (bh * p.N + tok) * D;
        dvr = p.dv_acc + (bh * p.N + tok) * D;
      }
      if (shared || tok < p.N) {
#pragma unroll
        for (int mt = 0; mt < MO; ++mt) {
          const int dim = attn_out_dim<D>(mt, grp, 0);
          *reinterpret_cast<float4*>(dvr + dim) = make_float4(dva[mt][0], dva[mt][1], dva[mt][2], dva[mt][3]);
          *reinterpret_cast<float4*>(dkr + dim) = make_float4(p.scale * dka[mt][0], p.scale * dka[mt][1],
                                                              p.scale * dka[mt][2], p.scale * dka[mt][3]);
        }
      }
    }
    __syncthreads();  // K and V of this leaf are consumed before the next run restages them
  }
}

// ------------------------------------------------------------------------------------------ merge, finish
// dq row of (unit, head): scale * sum over the unit's selected slots of the partial rows (16 lanes per row
// of D = 128, 8 bf16 each).
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_merge_kernel(const int* __restrict__ sel, const int* __restrict__ pos,
                                                           const uint16_t* __restrict__ part, int B, int Hq, int Hkv,
                                                           int G, int N, int K, float scale, uint16_t* __restrict__ dq) {
  constexpr int LPR = D / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long task = gid / LPR;  // (unit, head)
  const int li = (int)(gid % LPR);
  const long long U = (long long)B * Hkv * N;
  if (task >= U * G) return;
  const long long u = task / G;
  const int h = (int)(task % G);
  // the unit's slots first (selections are left-packed: nsel leading entries), then its partial rows
  // eight at a time, so that many loads are in flight; the sum runs over the slots in order
  constexpr int KMAX = 32;
  int at[KMAX];
  int nsel = 0;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    const bool in = s < K && sel[u * K + s] >= 0;
    at[s] = in ? pos[u * K + s] : 0;
    nsel += in ? 1 : 0;
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < KMAX; s0 += 8) {
    if (s0 >= nsel) break;
    uint4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < nsel) x[j] = *reinterpret_cast<const uint4*>(part + ((long long)at[s0 + j] * G + h) * D + 8 * li);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < nsel) {
        const uint32_t xs[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(xs[e] << 16);
          acc[2 * e + 1] += __uint_as_float(xs[e] & 0xffff0000u);
        }
      }
    }
  }
  const long long bh = u / N, i = u % N;
  const int b = (int)(bh / Hkv), r = (int)(bh % Hkv);
  const long long row = ((long long)b * Hq + (long long)r * G + h) * N + i;
  uint4 w;
  w.x = pack_bf16x2(scale * acc[0], scale * acc[1]);
  w.y = pack_bf16x2(scale * acc[2], scale * acc[3]);
  w.z = pack_bf16x2(scale * acc[4], scale * acc[5]);
  w.w = pack_bf16x2(scale * acc[6], scale * acc[7]);
  *reinterpret_cast<uint4*>(dq + row * D + 8 * li) = w;
}

// dK / dV of the leaves whose pairs span several dkdv tasks: one work-group per (sequence, KV
// head, leaf) bucket of the attention regroup (pairs [off[x], off[x + 1]) of the sorted list); the sum of
// the leaf's slots over its tasks, in task order, to the accumulators. A leaf within one task was stored
// by that task; a leaf without pairs keeps the cleared zeros.
template <int D, int C>
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const int* __restrict__ off, const float* __restrict__ kv_part,
                                                            int leaves, int N, float* __restrict__ dk_acc,
                                                            float* __restrict__ dv_acc) {
  const int x = blockIdx.x;
  const long long start = off[x], end = off[x + 1];
  if (end <= start) return;
  const long long t0 = start / kWgTaskDkdv, t1 = (end - 1) / kWgTaskDkdv;
  if (t1 == t0) return;
  const long long bh = x / leaves;
  const int leaf = x % leaves;
  constexpr int Q = C * D / 4;  // float4 items per array
  const int s0 = start % kWgTaskDkdv == 0 ? 0 : 1;  // the leaf's slot in its first task
  for (int it = threadIdx.x; it < 2 * Q; it += 256) {
    const int arr = it / Q, rem = it % Q;  // arr 0: dk, 1: dv
    const int tok_off = rem / (D / 4);
    const float4* src = reinterpret_cast<const float4*>(kv_part) + arr * Q + rem;
    float4 acc = src[(t0 * 2 + s0) * 2 * Q];
    for (long long t = t0 + 1; t <= t1; ++t) {
      const float4 v = src[t * 2 * 2 * Q];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const long long tok = (long long)leaf * C + tok_off;
    if (tok < N) {
      float* dst = (arr ? dv_acc : dk_acc) + (bh * N + tok) * D + 4 * (rem % (D / 4));
      *reinterpret_cast<float4*>(dst) = acc;
    }
  }
}

__global__ __launch_bounds__(256) void bwd_finish_kernel(const float* __restrict__ acc, long long n,
                                                         uint16_t* __restrict__ out) {
  const long long j = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 2;
  if (j < n) *reinterpret_cast<uint32_t*>(out + j) = pack_bf16x2(acc[j], acc[j + 1]);
}

// ------------------------------------------------------------------------------------------ launchers
template <int D, int C>
static hipError_t bwd_t(const SelDims& sd, const BwdParams& p0, const int* pos, const int* offsets, void* d_q,
                        void* d_k, void* d_v, hipStream_t st) {
  BwdParams p = p0;
  const long long rows = (long long)sd.B * sd.Hq * sd.N;
  const long long kv = (long long)sd.B * sd.Hkv * sd.N * D;
  // dk_acc and dv_acc are adjacent: one clear
  const long long pt = rows * (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((pt + 255) / 256)), dim3(256), 0, st, p.o, p.d_o, rows,
                     (float*)p.dsum, p.dk_acc, 2 * kv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long max_pairs = (long long)sd.B * sd.Hkv * sd.N * sd.K;
  const long long wg = (max_pairs + kWgTaskBwd - 1) / kWgTaskBwd;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, C>), dim3((unsigned)wg), dim3(256), 0, st, p);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, C>), dim3((unsigned)((max_pairs + kWgTaskDkdv - 1) / kWgTaskDkdv)),
                     dim3(256), 0, st, p);
  {
    const int leaves = sd.lv.n[0];
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<D, C>), dim3((unsigned)((long long)sd.B * sd.Hkv * leaves)), dim3(256),
                       0, st, offsets, p.kv_part, leaves, sd.N, p.dk_acc, p.dv_acc);
  }
  const long long mt = rows * (D / 8);
  hipLaunchKernelGGL((bwd_dq_merge_kernel<D>), dim3((unsigned)((mt + 255) / 256)), dim3(256), 0, st, p.sel, pos,
                     p.part, sd.B, sd.Hq, sd.Hkv, sd.G, sd.N, sd.K, sd.scale, (uint16_t*)d_q);
  hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)((kv / 2 + 255) / 256)), dim3(256), 0, st, p.dk_acc, kv,
                     (uint16_t*)d_k);
  hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)((kv / 2 + 255) / 256)), dim3(256), 0, st, p.dv_acc, kv,
                     (uint16_t*)d_v);
  return hipGetLastError();
}

hipError_t launch_attn_backward(const SelDims& sd, const void* q, const void* k, const void* v, const int* sel,
                                const void* o, const float* o_lse, const void* d_o, const uint32_t* pairs,
                                const int* total, const int* pos, const int* offsets, float* dsum, float* dk_acc,
                                float* dv_acc, float* kv_part, void* part, void* d_q, void* d_k, void* d_v,
                                hipStream_t st) {
  BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.d_o = (const uint16_t*)d_o;
  p.o_lse = o_lse;
  p.sel = sel;
  p.pairs = pairs;
  p.total = total;
  p.dsum = dsum;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.G = sd.G;
  p.N = sd.N;
  p.K = sd.K;
  p.chunk_log2 = sd.chunk_log2;
  p.scale = sd.scale;
  p.part = (uint16_t*)part;
  p.dk_acc = dk_acc;
  p.dv_acc = dv_acc;
  p.kv_part = kv_part;
  if (sd.D == 128) {
    if (sd.C == 64) return bwd_t<128, 64>(sd, p, pos, offsets, d_q, d_k, d_v, st);
    return bwd_t<128, 32>(sd, p, pos, offsets, d_q, d_k, d_v, st);
  }
  if (sd.C == 64) return bwd_t<64, 64>(sd, p, pos, offsets, d_q, d_k, d_v, st);
  return bwd_t<64, 32>(sd, p, pos, offsets, d_q, d_k, d_v, st);
}

size_t attn_backward_kv_part_bytes(const SelDims& sd) {
  const long long tasks = ((long long)sd.B * sd.Hkv * sd.N * sd.K + kWgTaskDkdv - 1) / kWgTaskDkdv;
  return (size_t)tasks * 2 * 2 * sd.C * sd.D * sizeof(float);
}

}  // namespace pisa
