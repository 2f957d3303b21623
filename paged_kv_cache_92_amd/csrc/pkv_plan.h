// Work schedules of the decode kernels.
//
// Attention of one (sequence, head) over its blocks can be cut into pieces
// whose partial results (running max, denominator, weighted sum) combine
// exactly: the block-wise aggregation of "vLLM: LLM 서빙 메모리 최적화의
// 교과서" (velog.io), section 02 "Aggregation".  Three ways to hand the pieces
// to workgroups:
//
//   kSchedGrid  one workgroup per (partition, head unit, sequence) grid cell;
//   kSchedPlan  fixed partitions of P tokens, walked round-robin by a
//               persistent grid over the non-empty cells only: every
//               workgroup first builds in LDS the prefix sum of partitions
//               per sequence (from the device-side lengths);
//   kSchedFlat  balanced: all (sequence, head unit, block) units in one row,
//               cut into gridDim.x equal contiguous ranges, one per resident
//               workgroup.  A range covers at most two pieces that are not
//               whole (sequence, head unit) segments, its first and its last;
//               they go to workspace slots 2w and 2w+1, every whole segment
//               straight to the output.
//
// A "head unit" is what one item computes: a query head (wavefront kernel)
// or a KV head with its G query heads (matrix-core kernel).
//
// Every schedule covers only the tokens a sequence attends to: [lo, L) with
// lo = max(0, L - window) under a sliding window of `window` tokens (0: no
// window, lo = 0).  Partitions stay aligned to absolute positions 0, P, 2P,
// ...; those wholly before lo are neither counted nor visited, so blocks
// released from before the window are never read.
#pragma once

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {

constexpr int kSchedGrid = 0;
constexpr int kSchedPlan = 1;
constexpr int kSchedFlat = 2;

// Tokens [lo, hi) that sequence s attends to (hi = its length, capped by the
// table).
struct Span {
  int lo, hi;
};
__device__ __forceinline__ Span seq_span(const int32_t *__restrict__ context_lens, int s, int cap,
                                         int window) {
  const int L = min(context_lens[s], cap);
  return Span{window > 0 ? max(0, L - window) : 0, L};
}

// Partitions of P tokens (aligned to absolute positions) that overlap the
// span: first_part(...) .. first_part(...) + parts_in(...) - 1.
__device__ __forceinline__ int first_part(Span sp, int part_tokens) { return sp.lo / part_tokens; }
__device__ __forceinline__ int parts_in(Span sp, int part_tokens) {
  return sp.hi > sp.lo ? (sp.hi - 1) / part_tokens - sp.lo / part_tokens + 1 : 0;
}

// Builds prefix[0..S] in LDS: prefix[s] = sum over sequences 0..s-1 of
// mult * parts_in(span of s, part_tokens).  Every thread of the workgroup
// must call it; returns prefix[S].  `scratch` is LDS for one int per wave.
__device__ inline int build_plan(int *prefix, int *scratch, const int32_t *__restrict__ context_lens,
                                 int S, int cap, int window, int part_tokens, int mult) {
  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid >> 6;
  const int chunk = (S + nthreads - 1) / nthreads;
  const int s0 = min(S, tid * chunk);
  const int s1 = min(S, s0 + chunk);
  int mine = 0;
  for (int s = s0; s < s1; ++s) mine += mult * parts_in(seq_span(context_lens, s, cap, window), part_tokens);
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
    run += mult * parts_in(seq_span(context_lens, s, cap, window), part_tokens);
  }
  if (tid == nthreads - 1) prefix[S] = run;
  __syncthreads();
  return prefix[S];
}

// Sequence owning entry j: the s with prefix[s] <= j < prefix[s+1].
__device__ __forceinline__ int plan_sequence(const int *prefix, int S, int j) {
  int lo = 0, hi = S;  // invariant: prefix[lo] <= j < prefix[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= j) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Where an item's result goes: dest < 0 the output; otherwise head g of the
// item writes partial row dest + g * stride of the workspace.
struct Dest {
  int base;
  int stride;
};

// Hands this workgroup's items to item(s, hu, b0, b1, dest): blocks
// [b0, b1) of sequence s for head unit hu (the item masks positions outside
// the sequence's span).  `lds` holds S + 1 ints (plan and flat schedules);
// `scan` one int per wave.  HU head units per sequence, G heads per unit,
// P = part_tokens (plan and grid schedules).
template <int SCHED, typename Item>
__device__ __forceinline__ void run_schedule(Item &&item, int *lds, int *scan,
                                             const int32_t *__restrict__ context_lens, int S,
                                             int cap, int window, int BS, int HU, int G,
                                             int part_tokens, int nparts, int *__restrict__ ws_hdr) {
  const int part_blocks = part_tokens / BS;
  if constexpr (SCHED == kSchedGrid) {
    const int s = blockIdx.z, hu = blockIdx.y, part = blockIdx.x;
    const Span sp = seq_span(context_lens, s, cap, window);
    const int p0 = first_part(sp, part_tokens), np = parts_in(sp, part_tokens);
    if (part < p0 || part >= p0 + np) return;
    const int bs = sp.lo / BS, nb = (sp.hi + BS - 1) / BS;
    item(s, hu, max(bs, part * part_blocks), min(nb, (part + 1) * part_blocks),
         np == 1 ? Dest{-1, 0} : Dest{(s * HU + hu) * G * nparts + part, nparts});
  } else if constexpr (SCHED == kSchedPlan) {
    const int total = build_plan(lds, scan, context_lens, S, cap, window, part_tokens, 1);
    const int nitems = total * HU;
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
      const int hu = it % HU;
      const int j = it / HU;
      const int s = plan_sequence(lds, S, j);
      const Span sp = seq_span(context_lens, s, cap, window);
      const int part = first_part(sp, part_tokens) + (j - lds[s]);
      const int bs = sp.lo / BS, nb = (sp.hi + BS - 1) / BS;
      item(s, hu, max(bs, part * part_blocks), min(nb, (part + 1) * part_blocks),
           lds[s + 1] - lds[s] == 1 ? Dest{-1, 0} : Dest{(s * HU + hu) * G * nparts + part, nparts});
      __syncthreads();  // the item's LDS merge buffers are reused by the next one
    }
  } else {
    const int U = build_plan(lds, scan, context_lens, S, cap, window, BS, HU);
    const int W = gridDim.x;
    const int C = (U + W - 1) / W;
    const int w = blockIdx.x;
    if (w == 0) {
      for (int i = threadIdx.x; i <= S; i += blockDim.x) ws_hdr[kFlatPrefixAt + i] = lds[i];
      if (threadIdx.x == 0) {
        ws_hdr[0] = C;
        ws_hdr[1] = U;
      }
    }
    const int u0 = w * C, u1 = min(U, u0 + C);
    for (int u = u0; u < u1;) {
      const int s = plan_sequence(lds, S, u);
      const int nb = (lds[s + 1] - lds[s]) / HU;  // span blocks of one head unit of s
      const int bs = seq_span(context_lens, s, cap, window).lo / BS;
      const int r = u - lds[s];
      const int hu = r / nb, b = r - hu * nb;
      const int e = min(u1, u + (nb - b));
      const bool whole = b == 0 && e - u == nb;
      item(s, hu, bs + b, bs + b + (e - u),
           whole ? Dest{-1, 0} : Dest{(u == u0 ? 2 * w : 2 * w + 1) * G, 1});
      __syncthreads();
      u = e;
    }
  }
}

// Balanced schedule: which workgroup ranges touched segment (s, hu).  Their
// partial rows are slot * G + g with slot 2*w, except 2*w0 + 1 when the
// segment was w0's last piece; w0 == w1 means the segment went straight to
// the output.
struct FlatSegment {
  int w0, w1;     // workgroups whose ranges touch the segment
  bool w0_last;   // the segment is w0's last piece (slot 2*w0 + 1)
};
__device__ __forceinline__ FlatSegment flat_segment(const int *__restrict__ ws_hdr, int s, int hu,
                                                    int HU) {
  const int C = ws_hdr[0];
  const int p0 = ws_hdr[kFlatPrefixAt + s], p1 = ws_hdr[kFlatPrefixAt + s + 1];
  const int nb = (p1 - p0) / HU;
  FlatSegment f{0, 0, false};
  if (nb == 0 || C == 0) return f;
  const int a = p0 + hu * nb;
  f.w0 = a / C;
  f.w1 = (a + nb - 1) / C;
  f.w0_last = a > f.w0 * C;
  return f;
}

}  // namespace pkv
