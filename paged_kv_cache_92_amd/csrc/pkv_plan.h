// Work plan of the split-KV decode kernels.
//
// A sequence of L tokens splits into ceil(L / P) partitions of P tokens (the
// block-wise partial results that "vLLM: LLM 서빙 메모리 최적화의 교과서",
// velog.io, section 02 "Aggregation" combines).  The kernels run a persistent
// grid: every workgroup first builds, in LDS, the exclusive prefix sum of
// partitions per sequence, then walks the non-empty (sequence, partition,
// head) items round-robin.  No workgroup is launched for an empty partition
// and no host knowledge of the lengths is needed.
#pragma once

#include "pkv_device.h"

namespace pkv {

// Sequences per launch that the in-LDS plan supports; beyond it the kernels
// fall back to one workgroup per (partition, head, sequence) grid cell.
constexpr int kPlanMaxSeqs = 8192;

__device__ __forceinline__ int num_partitions_of(int L, int part_tokens) {
  return L > 0 ? (L + part_tokens - 1) / part_tokens : 0;
}

// Builds prefix[0..S] in LDS: prefix[s] = partitions of sequences 0..s-1.
// Every thread of the workgroup must call it; returns prefix[S].
// `scratch` is LDS for one int per wave (at most 16 waves).
__device__ inline int build_plan(int *prefix, int *scratch, const int32_t *__restrict__ context_lens,
                                 int S, int cap, int part_tokens) {
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const int chunk = (S + nthreads - 1) / nthreads;
  const int s0 = min(S, tid * chunk);
  const int s1 = min(S, s0 + chunk);
  int mine = 0;
  for (int s = s0; s < s1; ++s) mine += num_partitions_of(min(context_lens[s], cap), part_tokens);
  // Inclusive scan within the wave, then across waves.
  int x = mine;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) scratch[wv] = x;
  __syncthreads();
  int base = 0;
  for (int k = 0; k < wv; ++k) base += scratch[k];
  int run = base + x - mine;
  for (int s = s0; s < s1; ++s) {
    prefix[s] = run;
    run += num_partitions_of(min(context_lens[s], cap), part_tokens);
  }
  if (tid == nthreads - 1) prefix[S] = run;
  __syncthreads();
  return prefix[S];
}

// Sequence owning partition-list entry j: the s with prefix[s] <= j < prefix[s+1].
__device__ __forceinline__ int plan_sequence(const int *prefix, int S, int j) {
  int lo = 0, hi = S;  // invariant: prefix[lo] <= j < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= j) lo = mid;
    else hi = mid;
  }
  return lo;
}

}  // namespace pkv
