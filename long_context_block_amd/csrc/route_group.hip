// Pyramid Top-K routing for several query units per wave ("Block Sparse Attention with Log-Linear
// Complexity" digest, 方法关键点: pyramid bullet -- coarse-to-fine walk keeping the Top-K of at most
// g*K candidates per level and expanding only their children; scoring bullet -- an intermediate node
// scores the LSE over its children's mean keys, summed over the GQA heads of the KV head).
//
// One work-group of 16 waves per CU (12 for K > 16) serves one KV head: the fp16 hi plane (and row
// bounds) of the upper pyramid levels is staged into LDS once, then each wave walks UG = 16 / G
// consecutive query positions at once (an aligned block, so at the top scored level the units share
// their candidates and one pass over the rows serves them all). Matrix column col = x G + h is head h
// of unit x, so all 16 columns carry data. At a scored
// level, row 16 m + r of unit x's M-tile m is child (r & 1) of candidate 8 m + (r >> 1); all lanes load
// and multiply every unit's rows, and the lanes of unit x keep the accumulators of their own M-tiles. A
// lane (col, g) then holds both children of candidates 8 m + 2 g + {0, 1} for its head, so the per-head
// LSE is lane-local and a butterfly over the unit's G columns (strides G/2 .. 1) sums the heads.
// Candidate 8 m + 2 g + a is owned by the lane with h = m mod G, which ranks it against its unit's keys
// in LDS and, if kept, places it in the unit's next kept list by a prefix count over an LDS bit mask.
//
// The arithmetic per candidate is the one-unit-per-wave walk's (same MFMA rows, k order, LSE, head-sum
// order, bounds, keys and tie-break), so both give the same kept sets bit for bit.
#include "common.hpp"
#include "internal.hpp"
#include "walk_tiles.hpp"

namespace pisa {

// waves per work-group: 16 (128 registers each) for the hot shape (d = 128, K <= 16, GQA 4); fewer where
// a wave's state grows (more candidate tiles, more units' heads per column block, or d = 64's longer
// per-row loops), so that no variant spills registers
template <int D, int G, int KM>
constexpr int group_waves() {
  return (KM > 4 || G == 16) ? 8 : (D == 128 && G == 4) ? 16 : 12;
}
constexpr int kGroupLdsBytes = 128 * 1024;
constexpr int kRowRound = 4;  // M-tiles of one unit whose hi rows are in flight together

struct GroupRouteParams {
  const uint16_t* q;
  const uint16_t* hilo;  // fp16 routing planes, Levels::rnodes rows per KV head (route_plane_chunk layout)
  const float* norms;    // per routing row: hi-plane bound
  const int* hexp;       // per KV head: planes hold 2^hexp mean
  int B, Hq, Hkv, N, K;
  float scale;
  Levels lv;
  int* kept;  // [U, K]
};

template <int D, int C, int G, int KM>
__global__ __launch_bounds__((group_waves<D, G, KM>() * 64)) void route_group_kernel(GroupRouteParams p, int lds_first,
                                                                      int wg_per_head) {
  constexpr int UG = 16 / G;             // units per wave
  constexpr int LOG2C = C == 64 ? 6 : 5;
  constexpr int NS = D / 32;             // k steps
  constexpr int OWN = (KM + G - 1) / G;  // owned M-tile slots per lane (x2 candidates)
  constexpr int NC = 8 * KM;             // candidate slots per unit (>= 2K)
  constexpr int kGroupWaves = group_waves<D, G, KM>();
  __shared__ __align__(16) uint16_t s_hi[kGroupLdsBytes / 2];
  __shared__ float s_bound[kGroupLdsBytes / 128];
  __shared__ int s_kept[kGroupWaves][2][UG][NC / 2];
  // a unit's keys (padded by 4 words: the units' 16-byte reads fall on different banks)
  __shared__ __align__(16) uint32_t s_key[kGroupWaves][UG][NC + 4];
  __shared__ unsigned long long s_mask[kGroupWaves][UG];
  __shared__ float s_ref[kGroupWaves][UG];  // per unit: the reference of its Top-K keys at this level
  const int lane = lane_id(), wave = threadIdx.x >> 6, col = lane & 15, g = lane >> 4;
  const int xo = col / G, h = col % G;  // this lane's unit and head
  const int cb = 2 * (col >> 2) + ((col >> 1) & 1);  // candidate of row col in M-tile 0
  const int BH = p.B * p.Hkv;
  const int bh = blockIdx.x % BH, w = blockIdx.x / BH;
  const int K = p.K;
  LdsHiRows<D> rows;
  rows.base = p.hilo + (long long)bh * p.lv.rnodes * 2 * D;
  const float* norms = p.norms + (long long)bh * p.lv.rnodes;
  rows.lds = s_hi;
  rows.lds_bound = s_bound;
  rows.first = lds_first;
  stage_hi_rows<D>(rows.base, norms, lds_first, (int)(p.lv.rnodes - lds_first), s_hi, s_bound);
  __syncthreads();
  const int hexp = p.hexp[bh];
  const int b = bh / p.Hkv, r = bh % p.Hkv;
  const int L = p.lv.n_levels - 1;
  const int groups = (p.N + UG - 1) / UG;
  for (int gi = w * kGroupWaves + wave; gi < groups; gi += wg_per_head * kGroupWaves) {
    // ---- units (positions) of this wave; past N: repeats of position N - 1, not stored
    int ix[UG];
#pragma unroll
    for (int x = 0; x < UG; ++x) ix[x] = gi * UG + x < p.N ? gi * UG + x : p.N - 1;
    int my_i = ix[0];
#pragma unroll
    for (int x = 1; x < UG; ++x) my_i = xo == x ? ix[x] : my_i;
    // ---- the column's query (bf16, then exactly scaled fp16) and sum_h |q_h| of its unit
    Frag<uint16_t> qf[NS], qh[NS];
    {
      const uint16_t* qrow = p.q + ((((long long)b * p.Hq + (long long)r * G + h) * p.N) + my_i) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < NS; ++s) qf[s].load(qrow + 32 * s);
    }
    float qn;
    {
      float sq = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = qf[s].get(e);
          sq += v * v;
        }
      qn = sqrtf(colgroup_sum(sq));
      qn = group_sum<G>(qn);
    }
    const int te = route_q_f16<D>(qf, qh);
    const float col_scale = ldexpf(p.scale, -(te + hexp));
    // ---- top of the walk: below the highest level where some unit has more than K eligible nodes
    int lw = 0;
#pragma unroll
    for (int x = 0; x < UG; ++x)
      for (int l = L; l > lw; --l)
        if ((ix[x] >> (LOG2C + l)) + 1 > K) {
          lw = l;
          break;
        }
    int nk[UG];
    int cur = 0;
#pragma unroll
    for (int x = 0; x < UG; ++x) {
      nk[x] = (ix[x] >> (LOG2C + lw + 1)) + 1;  // all eligible nodes of level lw + 1 (<= K when lw > 0)
      if (lane < nk[x]) s_kept[wave][0][x][lane] = lane;
    }
    __threadfence_block();
    for (int l = lw; l >= 1; --l) {
      const int off = (int)p.lv.roff[l - 1];  // routing row of the child level's node 0
      int n_cand[UG], n_full[UG];
      bool any_scored = false;
#pragma unroll
      for (int x = 0; x < UG; ++x) {
        // wave-uniform values (every lane reads the same LDS word), made scalar for uniform branches
        const int e_l = (ix[x] >> (LOG2C + l)) + 1, ec = (ix[x] >> (LOG2C + l - 1)) + 1;
        const int klast = __builtin_amdgcn_readfirstlane(s_kept[wave][cur][x][nk[x] - 1]);
        n_cand[x] = 2 * nk[x] - (2 * klast + 1 >= e_l ? 1 : 0);
        const int cn_last =
            2 * __builtin_amdgcn_readfirstlane(s_kept[wave][cur][x][(n_cand[x] - 1) >> 1]) + ((n_cand[x] - 1) & 1);
        n_full[x] = 2 * cn_last + 1 < ec ? n_cand[x] : n_cand[x] - 1;
        any_scored |= n_cand[x] > K;
      }
      int my_nc = n_cand[0], my_nf = n_full[0], my_nk = nk[0];
#pragma unroll
      for (int x = 1; x < UG; ++x) {
        my_nc = xo == x ? n_cand[x] : my_nc;
        my_nf = xo == x ? n_full[x] : my_nf;
        my_nk = xo == x ? nk[x] : my_nk;
      }
      const bool my_scored = my_nc > K;
      // row (col) of an M-tile m is valid iff its candidate 8 m + cb exists and, for a second child
      // (odd col), has two eligible children: 8 m + cb < lim[x]. Valid rows have kept index kj < nk.
      int lim[UG];
#pragma unroll
      for (int x = 0; x < UG; ++x) lim[x] = (col & 1) ? n_full[x] : n_cand[x];
      // candidate c: node 2 kept[c >> 1] + (c & 1) at level l
      auto cand_node = [&](int c) {
        const int kj = c >> 1;
        return 2 * s_kept[wave][cur][xo][kj < my_nk ? kj : 0] + (c & 1);
      };
      bool keep[OWN][2];
      if (any_scored) {
        // ---- pass 1 (hi) for every scored unit; lanes keep their own unit's accumulators. The level
        // is LDS-resident or not as a whole: one scalar branch picks the loader.
        f32x4 acc_own[KM];
        float own_e[OWN][2];
#pragma unroll
        for (int m = 0; m < KM; ++m) acc_own[m] = zero4();
        for_level_rows(rows, off, [&](const auto& ld) {
          if (l == lw) {
            // top scored level: the wave's units lie in one aligned block of 16 / G positions, so they
            // share the kept list (every eligible node of level lw + 1) and the candidate rows; one
            // pass serves all 16 columns
#pragma unroll
            for (int m = 0; m < KM; ++m) {
              const bool valid = 8 * m + cb < lim[0];
              const unsigned kn = (unsigned)s_kept[wave][cur][0][4 * m + (col >> 2)];  // any value if !valid
              Frag<uint16_t> hi[NS];
              ld.load_hi(hi, off + (valid ? (int)(4 * kn) + (col & 3) : 0), g);
              f32x4 a = zero4();
#pragma unroll
              for (int s = 0; s < NS; ++s) mma_f16(a, hi[s], qh[s]);
              acc_own[m] = a;
            }
          } else {
#pragma unroll
          for (int x = 0; x < UG; ++x) {
            if (n_cand[x] <= K) continue;
            // every M-tile is loaded (rows past the unit's candidates read row `off`, and their sums
            // are never used), so no branch separates the tiles' loads
            constexpr int MR = kRowRound < KM ? kRowRound : KM;
#pragma unroll
            for (int m0 = 0; m0 < KM; m0 += MR) {
#pragma unroll
              for (int m = m0; m < m0 + MR; ++m) {
                const bool valid = 8 * m + cb < lim[x];
                const unsigned kn = (unsigned)s_kept[wave][cur][x][4 * m + (col >> 2)];  // any value if !valid
                Frag<uint16_t> hi[NS];
                ld.load_hi(hi, off + (valid ? (int)(4 * kn) + (col & 3) : 0), g);
                f32x4 a = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s) mma_f16(a, hi[s], qh[s]);
                if (xo == x) acc_own[m] = a;
              }
              __builtin_amdgcn_sched_barrier(0);  // MR M-tiles' rows in flight at a time (register budget)
            }
          }
          }
          // the owned candidates' bounds: E = scale * sum_h |q_h| * max over the two children
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int m = h + j * G;
              const int c = 8 * m + 2 * g + a;
              float e = 0.f;
              if (m < KM && c < my_nc && my_scored) {
                const int r0 = off + 2 * cand_node(c);
                const float n0 = ld.bound(norms, r0), n1 = c < my_nf ? ld.bound(norms, r0 + 1) : 0.f;
                e = p.scale * qn * fmaxf(n0, n1);
              }
              own_e[j][a] = e;
            }
        });
        // ---- per-head candidate scores, summed over the unit's heads (strides G/2 .. 1)
        // tiles: bit m set = recompute M-tile m (wave-uniform)
        auto head_scores = [&](float (&sc)[KM][2], unsigned tiles) {
#pragma unroll
          for (int m = 0; m < KM; ++m)
            if ((tiles >> m) & 1u)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int c = 8 * m + 2 * g + a;
              const float x0 = col_scale * acc_own[m][2 * a], x1 = col_scale * acc_own[m][2 * a + 1];
              float v = c < my_nf ? lse2(x0, x1) : x0;
              sc[m][a] = group_sum<G>(v);
            }
        };
        float sc[KM][2];
        head_scores(sc, ~0u);
        // keys relative to the unit's first candidate's hi score (the reference topk_keep takes): lane
        // x G of lane group 0 holds the head sum of candidate 0 (m = 0, a = 0) of unit x
        float ref1 = __shfl(sc[0][0], xo * G);
        ref1 = __builtin_isfinite(ref1) ? ref1 : 0.f;
        if (h == 0 && g == 0) s_ref[wave][xo] = ref1;  // read back by pass 2
        // ---- owned candidates: hi score, hi Top-K
        float own_s[OWN][2];
        bool own_v[OWN][2], in[OWN][2];
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int m = h + j * G;
            float s = 0.f;
#pragma unroll
            for (int mm = 0; mm < KM; ++mm) s = mm == m ? sc[mm][a] : s;
            const int c = 8 * m + 2 * g + a;
            own_v[j][a] = m < KM && c < my_nc;
            own_s[j][a] = s;
          }
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int m = h + j * G;
            const int c = 8 * m + 2 * g + a;
            // every slot below NC has an owner: slots past the unit's candidates hold 0, which ranks
            // below every key (keys of finite and infinite scores are positive)
            if (m < KM) s_key[wave][xo][c] = own_v[j][a] ? topk_key(own_s[j][a] - ref1, c) : 0u;
          }
        __threadfence_block();
        // in-flags of the owned candidates (fewer than K of the unit's keys above theirs), all owned
        // keys ranked in one pass over the unit's keys in LDS
        auto owned_in = [&]() {
          uint32_t key[OWN][2];
          int rank[OWN][2];
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              // the owned candidate's own key, stored in its slot above (0 for a slot without one)
              const int m = h + j * G;
              key[j][a] = m < KM ? s_key[wave][xo][8 * m + 2 * g + a] : 0u;
              rank[j][a] = 0;
            }
#pragma unroll 2
          for (int c = 0; c < NC; c += 4) {  // every slot below NC holds a key or the padding 0
            const uint4 v = *reinterpret_cast<const uint4*>(&s_key[wave][xo][c]);
#pragma unroll
            for (int j = 0; j < OWN; ++j)
#pragma unroll
              for (int a = 0; a < 2; ++a)
                rank[j][a] += (v.x > key[j][a]) + (v.y > key[j][a]) + (v.z > key[j][a]) + (v.w > key[j][a]);
          }
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) in[j][a] = own_v[j][a] && rank[j][a] < K;
        };
        owned_in();
        float u_out = kNegInf, l_in = -kNegInf;
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            if (own_v[j][a] && !in[j][a]) u_out = fmaxf(u_out, own_s[j][a] + own_e[j][a]);
            if (in[j][a]) l_in = fminf(l_in, own_s[j][a] - own_e[j][a]);
          }
        // over the unit's lanes (its G columns in each of the 4 lane groups)
        u_out = group_max<G>(u_out);
        l_in = -group_max<G>(-l_in);
        u_out = colgroup_max(u_out);
        l_in = -colgroup_max(-l_in);
        bool refine[OWN][2];
        unsigned long long rb[OWN][2];  // wave-uniform: bit (x G + h) + 16 g = owner lane's flag
        unsigned long long ref_lanes = 0ull;
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const float lo_b = own_s[j][a] - own_e[j][a], hi_b = own_s[j][a] + own_e[j][a];
            refine[j][a] = my_scored && own_v[j][a] && ((in[j][a] && lo_b <= u_out) || (!in[j][a] && hi_b >= l_in));
            rb[j][a] = __ballot(refine[j][a]);
            ref_lanes |= rb[j][a];
          }
        if (ref_lanes) {
          // ---- pass 2 (lo) on the M-tiles holding undecided candidates; a row is read only if its
          // candidate is undecided. Candidate 8 m + 2 g' + a of unit x is owned by lane
          // (x G + m mod G) + 16 g' with flag set (m / G, a), so the tile and row flags come from the
          // owners' ballots.
          if (l == lw) {
            // shared rows (top scored level): a tile with an undecided candidate of any unit gets the lo
            // plane of all its valid rows; the sums of decided candidates are not used again
#pragma unroll
            for (int m = 0; m < KM; ++m) {
              unsigned long long tmask = 0ull;
#pragma unroll
              for (int x = 0; x < UG; ++x) tmask |= 0x0001000100010001ull << (x * G + (m % G));
              if (!((rb[m / G][0] | rb[m / G][1]) & tmask)) continue;
              const bool valid = 8 * m + cb < lim[0];
              const unsigned kn = (unsigned)s_kept[wave][cur][0][4 * m + (col >> 2)];  // any value if !valid
              Frag<uint16_t> lo[NS];
              rows.load_lo_any(lo, off + (valid ? (int)(4 * kn) + (col & 3) : 0), g);
#pragma unroll
              for (int s = 0; s < NS; ++s) mma_f16(acc_own[m], lo[s], qh[s]);
            }
          } else
#pragma unroll
          for (int x = 0; x < UG; ++x) {
#pragma unroll
            for (int m = 0; m < KM; ++m) {
              const int oc = x * G + (m % G);
              const unsigned long long tm = (rb[m / G][0] | rb[m / G][1]) & (0x0001000100010001ull << oc);
              if (!tm) continue;
              const bool valid = 8 * m + cb < lim[x];
              const unsigned long long fr = ((col >> 1) & 1) ? rb[m / G][1] : rb[m / G][0];
              // the owner's flag bit, computed here: hoisted out of the unit loop, the 16 shifted
              // 64-bit masks would hold 32 registers for the whole walk
              const int sh = opaque_int(oc + 16 * (col >> 2));
              const uint32_t fw = sh < 32 ? (uint32_t)fr : (uint32_t)(fr >> 32);
              const bool need = valid && ((fw >> (sh & 31)) & 1u);
              const unsigned kn = (unsigned)s_kept[wave][cur][x][4 * m + (col >> 2)];  // any value if !valid
              // rows of decided candidates read row `off` and add its lo plane: their sums are not used
              // again (a decided candidate's final key is +-inf), and other units' lanes drop `a`
              Frag<uint16_t> lo[NS];
              rows.load_lo_any(lo, off + (need ? (int)(4 * kn) + (col & 3) : 0), g);
              f32x4 a = acc_own[m];
#pragma unroll
              for (int s = 0; s < NS; ++s) mma_f16(a, lo[s], qh[s]);
              if (xo == x) acc_own[m] = a;
            }
          }
          // only tiles holding an undecided candidate of some unit change; the other tiles' scores
          // belong to decided candidates and are not read again
          unsigned rtiles = 0u;
#pragma unroll
          for (int m = 0; m < KM; ++m) {
            unsigned long long tmask = 0ull;
#pragma unroll
            for (int x = 0; x < UG; ++x) tmask |= 0x0001000100010001ull << (x * G + (m % G));
            if ((rb[m / G][0] | rb[m / G][1]) & tmask) rtiles |= 1u << m;
          }
          head_scores(sc, rtiles);
          __threadfence_block();
          // Decided candidates keep their flags: at most K were decided in (all ranked in by the hi
          // scores), and those together with the undecided hold every place, so the decided-out stay
          // out. An undecided candidate is in iff (decided in) + (undecided of its unit with a larger
          // hi+lo key) < K, i.e. its rank among all keys with the decided ones at +-inf. The undecided
          // keys of each unit are compacted to the front of its LDS key slots (0 after them), so the
          // ranking reads only those.
          const unsigned long long umask = (((1ull << G) - 1ull) << (xo * G)) * 0x0001000100010001ull;
          const unsigned long long below = lane ? (~0ull >> (64 - lane)) : 0ull;
          int n_in_dec = 0, n_ref = 0, pos[OWN][2];
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              n_in_dec += __popcll(__ballot(own_v[j][a] && in[j][a] && !refine[j][a]) & umask);
              pos[j][a] = n_ref + __popcll(rb[j][a] & umask & below);
              n_ref += __popcll(rb[j][a] & umask);
            }
          uint32_t rkey[OWN][2];
          const float ref2 = s_ref[wave][xo];  // pass 1's reference (keys of both passes share it)
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const int m = h + j * G;
              float sv = 0.f;
#pragma unroll
              for (int mm = 0; mm < KM; ++mm) sv = mm == m ? sc[mm][a] : sv;
              rkey[j][a] = topk_key(sv - ref2, 8 * m + 2 * g + a);
              if (refine[j][a]) s_key[wave][xo][pos[j][a]] = rkey[j][a];
            }
          if (h == 0 && g == 0) {  // one lane per unit pads the slots after its undecided keys
#pragma unroll
            for (int e = 0; e < 4; ++e) s_key[wave][xo][n_ref + e] = 0u;
          }
          __threadfence_block();
          int rank[OWN][2];
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a) rank[j][a] = n_in_dec;
          for (int c = 0; c < n_ref; c += 4) {
            const uint4 v = *reinterpret_cast<const uint4*>(&s_key[wave][xo][c]);
#pragma unroll
            for (int j = 0; j < OWN; ++j)
#pragma unroll
              for (int a = 0; a < 2; ++a)
                rank[j][a] += (v.x > rkey[j][a]) + (v.y > rkey[j][a]) + (v.z > rkey[j][a]) + (v.w > rkey[j][a]);
          }
#pragma unroll
          for (int j = 0; j < OWN; ++j)
#pragma unroll
            for (int a = 0; a < 2; ++a)
              if (refine[j][a]) in[j][a] = rank[j][a] < K;
        }
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) keep[j][a] = my_scored ? in[j][a] : own_v[j][a];
      } else {
#pragma unroll
        for (int j = 0; j < OWN; ++j)
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int m = h + j * G;
            keep[j][a] = m < KM && 8 * m + 2 * g + a < my_nc;
          }
      }
      // ---- next kept lists: kept candidates in ascending order
      if (lane < UG) s_mask[wave][lane] = 0ull;
      __threadfence_block();
#pragma unroll
      for (int j = 0; j < OWN; ++j)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = 8 * (h + j * G) + 2 * g + a;
          if (keep[j][a]) atomicOr(&s_mask[wave][xo], 1ull << c);
        }
      __threadfence_block();
      const unsigned long long my_mask = s_mask[wave][xo];
#pragma unroll
      for (int j = 0; j < OWN; ++j)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int c = 8 * (h + j * G) + 2 * g + a;
          if (keep[j][a]) s_kept[wave][cur ^ 1][xo][__popcll(my_mask & ((1ull << c) - 1))] = cand_node(c);
        }
      __threadfence_block();
#pragma unroll
      for (int x = 0; x < UG; ++x) nk[x] = __builtin_amdgcn_readfirstlane(__popcll(s_mask[wave][x]));
      cur ^= 1;
    }
    // ---- level-1 kept nodes (ascending), -1 past the count
#pragma unroll
    for (int x = 0; x < UG; ++x) {
      if (gi * UG + x >= p.N) break;
      const long long u = (long long)bh * p.N + gi * UG + x;
      if (lane < K) p.kept[u * K + lane] = lane < nk[x] ? s_kept[wave][cur][x][lane] : -1;
    }
    __threadfence_block();  // the next group rewrites this wave's LDS lists
  }
}

template <int D, int C, int G, int KM>
static hipError_t route_group_t(const SelDims& sd, const void* q, const void* hilo, const float* norms,
                                const int* hexp, int* kept, hipStream_t st) {
  GroupRouteParams p;
  p.q = (const uint16_t*)q;
  p.hilo = (const uint16_t*)hilo;
  p.norms = norms;
  p.hexp = hexp;
  p.B = sd.B;
  p.Hq = sd.Hq;
  p.Hkv = sd.Hkv;
  p.N = sd.N;
  p.K = sd.K;
  p.scale = sd.scale;
  p.lv = sd.lv;
  p.kept = kept;
  // LDS-resident upper levels: the smallest level whose rows up to the root fit
  int lcut = 0;
  while (lcut < sd.lv.n_levels - 1 && (sd.lv.rnodes - sd.lv.roff[lcut]) * D * 2 > kGroupLdsBytes) ++lcut;
  const int BH = sd.B * sd.Hkv;
  const long long groups = (sd.N + 16 / G - 1) / (16 / G);
  long long wph = 256 / BH;  // about one work-group per CU
  if (wph < 1) wph = 1;
  constexpr int kGroupWaves = group_waves<D, G, KM>();
  if (wph > (groups + kGroupWaves - 1) / kGroupWaves) wph = (groups + kGroupWaves - 1) / kGroupWaves;
  hipLaunchKernelGGL((route_group_kernel<D, C, G, KM>), dim3((unsigned)(BH * wph)), dim3(kGroupWaves * 64), 0, st, p,
                     (int)sd.lv.roff[lcut], (int)wph);
  return hipGetLastError();
}

template <int D, int C, int KM>
static hipError_t route_group_g(const SelDims& sd, const void* q, const void* hilo, const float* norms,
                                const int* hexp, int* kept, hipStream_t st) {
  if (sd.G == 4) return route_group_t<D, C, 4, KM>(sd, q, hilo, norms, hexp, kept, st);
  if (sd.G == 8) return route_group_t<D, C, 8, KM>(sd, q, hilo, norms, hexp, kept, st);
  return route_group_t<D, C, 16, KM>(sd, q, hilo, norms, hexp, kept, st);
}

bool route_group_supported(const SelDims& sd) {
  return sd.bf16 && (sd.G == 4 || sd.G == 8 || sd.G == 16) && sd.K <= 32;
}

hipError_t launch_route_group(const SelDims& sd, const void* q, const void* hilo, const float* norms, const int* hexp,
                              int* kept, hipStream_t st) {
  if (!route_group_supported(sd)) return hipErrorInvalidValue;
#define PISA_RG(D, C)                                                             \
  return sd.K <= 16 ? route_group_g<D, C, 4>(sd, q, hilo, norms, hexp, kept, st) \
                    : route_group_g<D, C, 8>(sd, q, hilo, norms, hexp, kept, st)
  if (sd.D == 128) {
    if (sd.C == 64) PISA_RG(128, 64);
    PISA_RG(128, 32);
  }
  if (sd.C == 64) PISA_RG(64, 64);
  PISA_RG(64, 32);
#undef PISA_RG
}

}  // namespace pisa
