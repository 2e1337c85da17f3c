// Work-group staging of a task of bucket-sorted (unit, slot) pairs, shared by the leaf stage of the
// selection and the leaf-major attention: the task's pairs and bucket keys go to LDS and the start of
// every run of equal keys is listed in order.
#pragma once
#include "common.hpp"

namespace pisa {

// kTask pairs per task, 256 threads. key(pair) is the pair's bucket key; runs are maximal ranges of
// equal keys. Returns the number of runs r; s_run[0..r] holds their starts and s_run[r] = n (RunT: any
// integer type that holds kTask).
template <int kTask, typename KeyFn, typename RunT>
__device__ __forceinline__ int stage_pair_runs(const uint32_t* __restrict__ pairs, long long base, int n, KeyFn key,
                                               uint32_t* s_pair, long long* s_key, RunT* s_run, int* s_wcount) {
  static_assert(kTask % 256 == 0, "task size");
  constexpr int J = kTask / 256;  // 64-entry chunks per wave
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  for (int x = tid; x < n; x += 256) {
    const uint32_t pr = pairs[base + x];
    s_pair[x] = pr;
    s_key[x] = key(pr);
  }
  __syncthreads();
  // wave w scans entries [w kTask / 4, (w + 1) kTask / 4)
  int cnt = 0;
  uint64_t masks[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int x = wave * (kTask / 4) + j * 64 + lane;
    const bool start = x < n && (x == 0 || s_key[x] != s_key[x - 1]);
    masks[j] = __ballot(start);
    cnt += __popcll(masks[j]);
  }
  if (lane == 0) s_wcount[wave] = cnt;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += s_wcount[w];
  const int nrun = s_wcount[0] + s_wcount[1] + s_wcount[2] + s_wcount[3];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int x = wave * (kTask / 4) + j * 64 + lane;
    if ((masks[j] >> lane) & 1) s_run[off + __popcll(masks[j] & ((1ull << lane) - 1))] = x;
    off += __popcll(masks[j]);
  }
  if (tid == 0) s_run[nrun] = n;
  __syncthreads();
  return nrun;
}

// Opaque copy of query fragments: keeps the compiler from folding a loop-carried prefetch (a phi of
// loads) into a single load placed right before its use.
template <typename F, int NF>
__device__ __forceinline__ void opaque_frags(F (&f)[NF]) {
#pragma unroll
  for (int s = 0; s < NF; ++s) asm volatile("" : "+v"(f[s].u.x), "+v"(f[s].u.y), "+v"(f[s].u.z), "+v"(f[s].u.w));
}

}  // namespace pisa
