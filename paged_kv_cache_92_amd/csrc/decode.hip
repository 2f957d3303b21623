// Paged decode attention on the vector ALUs: one workgroup (4 waves) per
// (partition, query head, sequence).  The block-by-block walk follows
// "vLLM — KV Cache와 PagedAttention 완전 해부" (hrletsgo.me), "부록": fetch
// each block through the block table, compute the partial scores, update the
// running softmax normaliser, accumulate the weighted values.  The result is
// the token-wise softmax attention of "vLLM: LLM 서빙 메모리 최적화의 교과서"
// (velog.io), section 01, rewritten block-wise as eq. (4) of section 02.
//
// Wave mapping of one block (B tokens):
//   key tile  [D/X][B][X] (X = 64 bytes of a key row): lane = 4*t + k holds
//             16-byte piece k of token t's X-wide slice, so one wave load
//             reads 16 tokens x 64 bytes = 1 KiB contiguous, and a block takes
//             KL = (D/X)*(B/16) loads per lane.  Each lane's partial dot
//             product covers D/4 dimensions; the 4 lanes of a quad are summed
//             with two DPP steps.
//   value tile [D][B] dimension-major: a 16-byte chunk is VEC consecutive
//             tokens of one dimension; CPR = B/VEC chunks per dimension row,
//             VL = D*CPR/64 loads per lane.  Each lane accumulates its
//             dimensions over its VEC tokens; the CPR lanes sharing a
//             dimension are summed at the end.
//   The B softmax weights move from the key layout to the value layout
//   through a per-wave LDS slot.
// The 4 waves take interleaved blocks of the partition and are merged
// through LDS at the end; every score lives in the log2 domain (scores
// scaled by scale*log2(e)) so that exp2 is a single instruction.
#include <algorithm>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_plan.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;

// Tokens one wave step covers: a whole block, or for 8-token blocks a pair of
// consecutive logical blocks (16 tokens), so the wave mapping below always
// sees groups of 16 tokens.
constexpr int group_tokens(int BS) { return BS == 8 ? 16 : BS; }

template <typename E, int D, int BS>
struct ValuCfg {
  static constexpr int EB = E::kBytes;
  static constexpr int VEC = 16 / EB;   // elements per 16-byte load
  static constexpr int X = 64 / EB;     // elements per 64-byte key piece
  static constexpr int NC = D / X;      // key pieces per row
  static constexpr int TG = BS / 16;    // 16-token groups per block
  static constexpr int KL = NC * TG;
  static constexpr int CPR = BS / VEC;
  static constexpr int VL = D * CPR / kWave;
  // VGPRs holding one block's key and value loads.
  static constexpr int kLoadRegs = 4 * (KL + VL);
  static_assert(D % X == 0 && BS % 16 == 0, "key tile mapping");
  static_assert(CPR >= 1 && kWave % CPR == 0 && (D * CPR) % kWave == 0, "value tile mapping");
};

template <typename E, int D, int BS>
struct ValuLds {
  float p[kWaves][BS] __attribute__((aligned(16)));
  float m[kWaves];
  float l[kWaves];
  float acc[kWaves][D];
};

// One work item: blocks [b0, b1) of sequence s for query head hq, positions
// before the sliding window's start (window > 0) masked; the merged result
// goes to the output or to a workspace partial row (dest).  E is the
// cache's element type, Q the query/output type (E itself, except over an
// 8-bit cache: there the key scale is folded into scale_log2 and the value
// scale multiplies the merged sums).  APPEND: the sequence's new token
// (position L-1) is taken from the input rows ap.k / ap.v, in cache format,
// instead of the pool, whose slot is written by the reduce kernel.
template <typename E, typename Q, int D, int BS, bool APPEND>
__device__ __forceinline__ void valu_item(
    ValuLds<E, D, group_tokens(BS)> &sh, int s, int hq, int b0, int b1, Dest dest,
    void *__restrict__ out,
    int out_f32, const typename Q::storage *__restrict__ q,
    const typename E::storage *__restrict__ kpool, const typename E::storage *__restrict__ vpool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    int64_t num_blocks, int Hkv, int Hq, int mbps, int cap, int window, float scale_log2,
    float v_scale, float *__restrict__ ws_ml, float *__restrict__ ws_acc, const Append<Q> &ap) {
  constexpr int GB = group_tokens(BS);
  constexpr bool kPair = GB == 2 * BS;      // two blocks per step
  using C = ValuCfg<E, D, GB>;
  using T = typename E::storage;
  constexpr bool kFP8 = E::kBytes == 1;
  constexpr bool kF64 = E::kBytes == 4;   // fp32 cache: scores in fp64
  const Span sp = seq_span(context_lens, s, cap, window);
  const int lo = sp.lo;                      // first attended position
  const int tok0 = max(b0 * BS, lo);
  const int tok1 = min(sp.hi, b1 * BS);
  if (tok0 >= tok1) return;
  const int blk0 = b0;
  const int nblk = b1 - b0;
  const int hkv = hq / (Hq / Hkv);

  int lane = threadIdx.x & (kWave - 1);
  const int w = uniform(threadIdx.x >> 6);
  int kq = lane & 3;         // 16-byte piece within a 64-byte key slice
  int kt = lane >> 2;        // token within a 16-token group
  int cp = lane % C::CPR;    // token chunk of the value row

  auto &lds_p = sh.p;
  auto &lds_m = sh.m;
  auto &lds_l = sh.l;
  auto &lds_acc = sh.acc;

  // The query dimensions this lane multiplies: kept in the packed input
  // format (dot2 products), or as fp32 over an 8-bit cache.
  u32x4 qc[kFP8 ? 1 : C::NC];
  float qf[kFP8 ? C::NC : 1][kFP8 ? C::VEC : 1];
  {
    const typename Q::storage *qrow = q + ((size_t)s * Hq + hq) * D + kq * C::VEC;
    if constexpr (kFP8) {
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        unpack16<Q>(load16(qrow + c * C::X), &qf[c][0]);
        unpack16<Q>(load16(qrow + c * C::X + 8), &qf[c][8]);
      }
    } else {
#pragma unroll
      for (int c = 0; c < C::NC; ++c) qc[c] = load16(qrow + c * C::X);
    }
  }
  // q.k of this lane's slice against one 16-byte key load of piece c.
  auto dot = [&](const u32x4 &k, int c) -> float {
    if constexpr (kFP8) {
      float kf[16];
      unpack16<FP8>(k, kf);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) d = fmaf(qf[c][i], kf[i], d);
      return d;
    } else {
      return dot16<E>(k, qc[c]);
    }
  };

  float m = -INFINITY;
  float l = 0.f;
  float acc[C::VL];
#pragma unroll
  for (int i = 0; i < C::VL; ++i) acc[i] = 0.f;

  const int32_t *bt = block_tables + (size_t)s * mbps;
  constexpr int STEP = kPair ? 2 : 1;
  // One step of a wave: block b of the item (and b+1 for a pair).  `app`
  // (std::true_type) marks the step that appends the new token.
  auto step = [&](const int b, auto app) {
    constexpr bool kApp = decltype(app)::value;
    const int lb = blk0 + b;
    // Appending step: the new token's index in the step, and (cache in the
    // model dtype) its key row, which the lanes holding that token load in
    // place of the pool's slot.
    const int j = kApp ? sp.hi - 1 - lb * BS : -1;
    const T *knew = nullptr;
    if constexpr (kApp && !kFP8) knew = (const T *)ap.k + ((size_t)s * Hkv + hkv) * D + kq * C::VEC;
    auto kld = [&](const T *p, int t, int c) -> u32x4 {
      if constexpr (kApp && !kFP8) {
        if (t == j) p = knew + c * C::X;
      }
      return load16_stream(p);
    };
    int64_t phys = uniform(bt[lb]);
    int64_t phys2 = phys;
    bool ok1 = true, ok2 = true;   // table entries in range (a pair's second: if covered)
    u32x4 kr[C::KL];
    u32x4 vr[C::VL];
    if constexpr (!kPair) {
      if (phys < 0 || phys >= num_blocks) return;
      const T *ktile = kpool + ((size_t)phys * Hkv + hkv) * (BS * D);
      const T *vtile = vpool + ((size_t)phys * Hkv + hkv) * (D * BS);
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int r = 0; r < C::TG; ++r)
          kr[c * C::TG + r] = kld(ktile + (c * BS + 16 * r + kt) * C::X + kq * C::VEC, 16 * r + kt, c);
#pragma unroll
      for (int i = 0; i < C::VL; ++i) vr[i] = load16_stream(vtile + (size_t)(kWave * i + lane) * C::VEC);
    } else {
      // Blocks lb and lb+1 (the second only if the item covers it; past the
      // item its tokens are masked and block lb is read in its place).  An
      // out-of-range id reads block 0 instead of faulting.
      phys2 = b + 1 < nblk ? uniform(bt[lb + 1]) : phys;
      ok1 = phys >= 0 && phys < num_blocks;
      ok2 = phys2 >= 0 && phys2 < num_blocks;
      if (!ok1) phys = 0;
      if (!ok2) phys2 = 0;
      const T *kt0 = kpool + ((size_t)phys * Hkv + hkv) * (BS * D);
      const T *kt1 = kpool + ((size_t)phys2 * Hkv + hkv) * (BS * D);
      const T *vt0 = vpool + ((size_t)phys * Hkv + hkv) * (D * BS);
      const T *vt1 = vpool + ((size_t)phys2 * Hkv + hkv) * (D * BS);
      // Token t of the step lies in block t / BS of the pair.
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int r = 0; r < C::TG; ++r) {
          const int t = 16 * r + kt;
          kr[c * C::TG + r] = kld((t < BS ? kt0 : kt1) + (c * BS + t % BS) * C::X + kq * C::VEC, t, c);
        }
#pragma unroll
      for (int i = 0; i < C::VL; ++i) {
        const int idx = kWave * i + lane;           // chunk: dimension idx / CPR, tokens VEC*(idx % CPR)..
        const int dim = idx / C::CPR, tok = (idx % C::CPR) * C::VEC;
        if constexpr (C::VEC <= BS) {
          vr[i] = load16_stream((tok < BS ? vt0 : vt1) + dim * BS + tok % BS);
        } else {
          // 16 codes of one dimension: 8 from each block's row.
          const u32x2 a = load8_stream(vt0 + dim * BS), c2 = load8_stream(vt1 + dim * BS);
          vr[i] = u32x4{a[0], a[1], c2[0], c2[1]};
        }
      }
    }

    // The new token in cache format: its key pieces replace the pool's (an
    // 8-bit cache quantises them here; otherwise they were loaded from the
    // input row above) and its value element replaces the pool's as the
    // values are unpacked.  The pool's slot is never read; the reduce kernel
    // that follows stores the rows into it.
    uint32_t vnew[C::VL];   // the new token's value bits, one per chunk of this lane
    int vj = -1;            // its element within this lane's chunks (-1: none)
    const size_t row = ((size_t)s * Hkv + hkv) * D;
    if constexpr (kApp) {
#pragma unroll
      for (int i = 0; i < C::VL; ++i) vnew[i] = 0u;
      if (j >= 0 && j < GB) {
        if constexpr (kFP8) {
#pragma unroll
          for (int r = 0; r < C::TG; ++r) {
            if (16 * r + kt != j) continue;
#pragma unroll
            for (int c = 0; c < C::NC; ++c)
              kr[c * C::TG + r] = cache_piece<E, Q>(ap.k + row + c * C::X + kq * C::VEC, ap.k_scale);
          }
        }
        // A lane's value chunks all start at token (lane % CPR) * VEC.
        const int t0 = (lane % C::CPR) * C::VEC;
        if (j >= t0 && j < t0 + C::VEC) {
          vj = j - t0;
#pragma unroll
          for (int i = 0; i < C::VL; ++i)
            vnew[i] = cache_elem<E, Q>(ap.v[row + (kWave * i + lane) / C::CPR], ap.v_scale);
        }
      }
    }

    const int tbase = lb * BS;
    // Only the last step can end past the length, only the first start
    // before the window.
    const bool partial = tbase + GB > tok1 || tbase < lo;
    // Scores.  Over an fp32 cache each score is formed in fp64 and kept
    // (sd) until its weight is taken: a score of a few hundred log2 units
    // rounded to fp32 would already move its weight by ~1e-5, so the weight
    // is 2^(sd - m) with the fp64 difference, and only the reference maximum
    // m is an fp32 value (the rounded score).
    float sc[C::TG];
    double sd[kF64 ? C::TG : 1];
#pragma unroll
    for (int r = 0; r < C::TG; ++r) {
      bool masked = partial && (unsigned)(tbase + 16 * r + kt - lo) >= (unsigned)(tok1 - lo);
      if constexpr (kF64) {
        double x = dot16_f64(kr[r], qc[0]);
#pragma unroll
        for (int c = 1; c < C::NC; ++c) x += dot16_f64(kr[c * C::TG + r], qc[c]);
        x = quad_sum_f64(x) * (double)scale_log2;
        if (masked) x = -INFINITY;
        sd[r] = x;
        sc[r] = (float)x;
      } else {
        float x = dot(kr[r], 0);
#pragma unroll
        for (int c = 1; c < C::NC; ++c) x += dot(kr[c * C::TG + r], c);
        x = group_sum<4>(x) * scale_log2;
        if (masked) x = -INFINITY;
        sc[r] = x;
      }
    }
    float mb = sc[0];
#pragma unroll
    for (int r = 1; r < C::TG; ++r) mb = fmaxf(mb, sc[r]);
    mb = quad_uniform_max(mb);
    const float mnew = fmaxf(m, mb);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    if (kq == 0) {
#pragma unroll
      for (int r = 0; r < C::TG; ++r) {
        if constexpr (kF64) lds_p[w][16 * r + kt] = fast_exp2((float)(sd[r] - (double)mnew));
        else lds_p[w][16 * r + kt] = fast_exp2(sc[r] - mnew);
      }
    }
    __builtin_amdgcn_wave_barrier();
    float p[C::VEC];
#pragma unroll
    for (int i = 0; i < C::VEC; i += 4) {
      const f32x4 pv = *(const f32x4 *)&lds_p[w][cp * C::VEC + i];
      p[i] = pv[0]; p[i + 1] = pv[1]; p[i + 2] = pv[2]; p[i + 3] = pv[3];
    }
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < C::VEC; ++e) psum += p[e];
    l = l * alpha + psum;
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      float vf[C::VEC];
      unpack16<E>(vr[i], vf);
      if constexpr (kApp) {
        if (vj >= 0) {
          const float nv = elem_value<E>(vnew[i]);
#pragma unroll
          for (int e = 0; e < C::VEC; ++e)
            if (e == vj) vf[e] = nv;
        }
      }
      float a = acc[i] * alpha;
      if (partial) {
        // Slots outside [lo, tok1) may hold anything (NaN included): their values count as 0.
#pragma unroll
        for (int e = 0; e < C::VEC; ++e) {
          const float ve =
              ((unsigned)(tbase + cp * C::VEC + e - lo) < (unsigned)(tok1 - lo)) ? vf[e] : 0.f;
          a = fmaf(p[e], ve, a);
        }
      } else {
#pragma unroll
        for (int e = 0; e < C::VEC; ++e) a = fmaf(p[e], vf[e], a);
      }
      acc[i] = a;
    }
    __builtin_amdgcn_wave_barrier();
  };
  // An appending item that ends the sequence takes its last step (the one
  // holding position L-1) out of the loop, so that the loop itself is the
  // plain decode's.
  int bmain = nblk, blast = -1;
  if constexpr (APPEND) {
    if (tok1 == sp.hi) {
      blast = (nblk - 1) / STEP * STEP;
      bmain = blast;
    }
  }
  for (int b = STEP * w; b < bmain; b += STEP * kWaves) step(b, std::false_type{});
  if constexpr (APPEND) {
    if (blast >= 0 && (blast / STEP) % kWaves == w) {
      // Opaque copies of the lane indices: the step recomputes its per-lane
      // addresses instead of keeping them live through the loop.
      asm volatile("" : "+v"(lane), "+v"(kq), "+v"(kt), "+v"(cp));
      step(blast, std::true_type{});
    }
  }

  // Sum each dimension over the CPR lanes that share it, and l over the same lanes.
  l = group_sum<C::CPR>(l);
#pragma unroll
  for (int i = 0; i < C::VL; ++i) acc[i] = group_sum<C::CPR>(acc[i]);
  if (cp == 0) {
#pragma unroll
    for (int i = 0; i < C::VL; ++i) lds_acc[w][(kWave * i + lane) / C::CPR] = acc[i];
  }
  if (lane == 0) {
    lds_m[w] = m;
    lds_l[w] = l;
  }
  __syncthreads();

  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float M = lds_m[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) M = fmaxf(M, lds_m[k]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float f = fast_exp2(lds_m[k] - M);  // 0 for a wave that saw no block
      num = fmaf(f, lds_acc[k][e], num);
      den = fmaf(f, lds_l[k], den);
    }
    if constexpr (kFP8) num *= v_scale;
    if (dest.base < 0) {
      store_out<Q>(out, ((size_t)s * Hq + hq) * D + e, num / den, out_f32);
    } else {
      const size_t pi = dest.base;
      ws_acc[pi * D + e] = num;
      if (e == 0) {
        ws_ml[2 * pi] = M;
        ws_ml[2 * pi + 1] = den;
      }
    }
  }
}

// SCHED: kSchedGrid (one workgroup per grid cell), kSchedPlan (fixed
// partitions over a persistent grid) or kSchedFlat (balanced ranges).  The
// grid schedule asks for 8 waves per SIMD (64 VGPRs) only where one block's
// loads plus the query slice fit that budget without spills; other variants
// keep the compiler's choice.  Appending variants of 16-bit caches with
// head_dim 128 and 16-token blocks ask for the 5 waves per SIMD their plain
// versions reach.
template <typename E, int D, int BS, int SCHED, bool APPEND>
constexpr int valu_min_waves() {
  if constexpr (APPEND) return E::kBytes == 2 && D == 128 && BS == 16 ? 5 : 1;
  return SCHED == kSchedGrid && E::kBytes >= 2 &&
                 ValuCfg<E, D, group_tokens(BS)>::kLoadRegs + 4 * ValuCfg<E, D, group_tokens(BS)>::NC <= 24
             ? 8
             : 1;
}
template <typename E, typename Q, int D, int BS, int SCHED, bool APPEND>
__global__ __launch_bounds__(256, (valu_min_waves<E, D, BS, SCHED, APPEND>())) void
decode_valu_kernel(
    void *__restrict__ out, int out_f32, const typename Q::storage *__restrict__ q,
    const typename E::storage *__restrict__ kpool, const typename E::storage *__restrict__ vpool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    int64_t num_blocks, int Hkv, int Hq, int S, int mbps, int cap, int window, float scale_log2,
    float v_scale, int part_tokens, int nparts, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int *__restrict__ ws_hdr, Append<Q> ap) {
  __shared__ ValuLds<E, D, group_tokens(BS)> sh;
  extern __shared__ int plan[];
  __shared__ int scan[16];
  run_schedule<SCHED>(
      [&](int s, int hq, int b0, int b1, Dest dest) {
        valu_item<E, Q, D, BS, APPEND>(sh, s, hq, b0, b1, dest, out, out_f32, q, kpool, vpool, block_tables,
                               context_lens, num_blocks, Hkv, Hq, mbps, cap, window, scale_log2,
                               v_scale, ws_ml, ws_acc, ap);
      },
      plan, scan, context_lens, S, cap, window, BS, Hq, 1, part_tokens, nparts, ws_hdr);
}

// Appending call: the reduce kernel (launched after the decode kernel, also
// when there is nothing to reduce) stores each sequence's new key and value
// rows into the cache slot of position L-1; the decode kernel took them from
// the input rows and never read that slot.  Stores in the middle of the
// decode kernel's read stream cost it far more than the bytes they move.
struct NewToken {
  const void *k = nullptr;   // [S][Hkv][D] model dtype; nullptr: nothing to store
  const void *v = nullptr;
  float k_scale = 1.f, v_scale = 1.f;
  void *kpool = nullptr;
  void *vpool = nullptr;
  const int32_t *block_tables = nullptr;
  int64_t num_blocks = 0;
  int Hkv = 1, BS = 16, mbps = 0;
  int cap = 0;   // lengths are clamped to it, as the decode kernel clamps them
};

// Rows of sequence s, KV head hkv, into the slot of position L-1 (none if
// the table entry is out of range), each element as pkv_reshape_and_cache
// stores it.  KV is the cache element, Q the model dtype.
template <typename KV, typename Q, int D>
__device__ __forceinline__ void store_new_token(const NewToken &nt,
                                                const int32_t *__restrict__ context_lens, int s,
                                                int hkv) {
  const int L = min(context_lens[s], nt.cap);
  if (L <= 0) return;
  const int64_t phys = nt.block_tables[(size_t)s * nt.mbps + (L - 1) / nt.BS];
  if (phys < 0 || phys >= nt.num_blocks) return;
  const int off = (L - 1) % nt.BS;
  constexpr int X = 64 / KV::kBytes;   // elements per 64-byte key piece
  using T = typename KV::storage;
  using TQ = typename Q::storage;
  const size_t row = ((size_t)s * nt.Hkv + hkv) * D;
  const size_t tile = ((size_t)phys * nt.Hkv + hkv) * ((size_t)nt.BS * D);
  T *kt = (T *)nt.kpool + tile;
  T *vt = (T *)nt.vpool + tile;
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    store_bits<KV::kBytes>(kt + (e / X) * (nt.BS * X) + off * X + e % X,
                           cache_elem<KV, Q>(((const TQ *)nt.k)[row + e], nt.k_scale));
    store_bits<KV::kBytes>(vt + (size_t)e * nt.BS + off,
                           cache_elem<KV, Q>(((const TQ *)nt.v)[row + e], nt.v_scale));
  }
}

// Cross-partition reduce over the partitions of the sequence's span:
// o = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p.
template <typename E, typename KV, int D>
__global__ __launch_bounds__(128) void decode_reduce_kernel(
    void *__restrict__ out, int out_f32, const int32_t *__restrict__ context_lens, int Hq,
    int mbps_tokens, int window, int part_tokens, int nparts, const float *__restrict__ ws_ml,
    const float *__restrict__ ws_acc, NewToken nt) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  const int G = Hq / nt.Hkv;
  if (nt.k != nullptr && hq % G == 0) store_new_token<KV, E, D>(nt, context_lens, s, hq / G);
  const Span sp = seq_span(context_lens, s, mbps_tokens, window);
  const int p0 = first_part(sp, part_tokens);
  const int np = min(parts_in(sp, part_tokens), nparts - p0);
  if (np <= 1) return;
  const size_t base = ((size_t)s * Hq + hq) * nparts + p0;
  float M = -INFINITY;
  for (int p = 0; p < np; ++p) M = fmaxf(M, ws_ml[2 * (base + p)]);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int p = 0; p < np; ++p) {
      const float f = fast_exp2(ws_ml[2 * (base + p)] - M);
      num = fmaf(f, ws_acc[(base + p) * D + e], num);
      den = fmaf(f, ws_ml[2 * (base + p) + 1], den);
    }
    store_out<E>(out, ((size_t)s * Hq + hq) * D + e, num / den, out_f32);
  }
}

// Balanced-schedule reduce: the partial rows of every segment that spans
// several workgroup ranges (see run_schedule), combined as above.  HU head
// units per sequence, G query heads per unit.
template <typename E, typename KV, int D>
__global__ __launch_bounds__(128) void decode_reduce_flat_kernel(
    void *__restrict__ out, int out_f32, const int *__restrict__ ws_hdr, int Hq, int HU, int G,
    const float *__restrict__ ws_ml, const float *__restrict__ ws_acc,
    const int32_t *__restrict__ context_lens, NewToken nt) {
  const int hq = blockIdx.x;
  const int s = blockIdx.y;
  if (nt.k != nullptr && hq % (Hq / nt.Hkv) == 0)
    store_new_token<KV, E, D>(nt, context_lens, s, hq / (Hq / nt.Hkv));
  const int g = hq % G;
  const FlatSegment f = flat_segment(ws_hdr, s, hq / G, HU);
  if (f.w1 <= f.w0) return;
  auto row = [&](int w) -> size_t {
    const int slot = (w == f.w0 && f.w0_last) ? 2 * w + 1 : 2 * w;
    return (size_t)slot * G + g;
  };
  float M = -INFINITY;
  for (int w = f.w0; w <= f.w1; ++w) M = fmaxf(M, ws_ml[2 * row(w)]);
  for (int e = threadIdx.x; e < D; e += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int w = f.w0; w <= f.w1; ++w) {
      const size_t r = row(w);
      const float fct = fast_exp2(ws_ml[2 * r] - M);
      num = fmaf(fct, ws_acc[r * D + e], num);
      den = fmaf(fct, ws_ml[2 * r + 1], den);
    }
    store_out<E>(out, ((size_t)s * Hq + hq) * D + e, num / den, out_f32);
  }
}

template <typename E, typename Q, int D, int BS, bool APPEND>
void launch_valu_ta(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  using T = typename E::storage;
  using TQ = typename Q::storage;
  const float sl = a.scale * kLog2e * c.k_scale;  // k_scale is 1 unless the cache is 8-bit
  const size_t lds = sizeof(int) * (a.S + 1);
  auto go = [&](auto kern, dim3 grid, size_t dyn) {
    hipLaunchKernelGGL(kern, grid, dim3(256), dyn, stream, a.out, (int)a.out_f32, (const TQ *)a.q,
                       (const T *)c.k, (const T *)c.v, a.block_tables, a.context_lens,
                       c.num_blocks, c.H, a.Hq, a.S, a.max_blocks_per_seq, a.cap_tokens, a.window,
                       sl, c.v_scale,
                       a.partition_tokens, a.num_partitions, a.ws_ml, a.ws_acc, a.ws_hdr,
                       Append<Q>{(const TQ *)a.new_k, (const TQ *)a.new_v, c.k_scale, c.v_scale});
  };
  // Fixed partitions run a persistent grid over the non-empty cells (a 3-D
  // grid would launch a workgroup for every empty partition); without a split
  // every grid cell has work and the hardware balances uneven lengths itself.
#ifndef PKV_GRID_FACTOR
#define PKV_GRID_FACTOR 4
#endif
  if (a.flat) {
    go(decode_valu_kernel<E, Q, D, BS, kSchedFlat, APPEND>, dim3(a.flat_grid), lds);
  } else if (a.num_partitions > 1 && a.S <= kPlanMaxSeqs) {
    auto kern = decode_valu_kernel<E, Q, D, BS, kSchedPlan, APPEND>;
    const int64_t cells = (int64_t)a.S * a.num_partitions * a.Hq;
    const int grid = (int)std::min<int64_t>(cells, PKV_GRID_FACTOR * (int64_t)resident_workgroups((const void *)kern, 256, lds));
    go(kern, dim3(grid), lds);
  } else {
    go(decode_valu_kernel<E, Q, D, BS, kSchedGrid, APPEND>,
       dim3((unsigned)a.num_partitions, (unsigned)a.Hq, (unsigned)a.S), 0);
  }
}

// Appending calls run their own instantiations, so that plain decode keeps
// its register budget.
template <typename E, typename Q, int D, int BS>
void launch_valu_t(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (a.new_k != nullptr) launch_valu_ta<E, Q, D, BS, true>(c, a, stream);
  else launch_valu_ta<E, Q, D, BS, false>(c, a, stream);
}

template <typename E, typename Q = E>
void launch_valu_e(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (c.D == 64 && c.B == 8) launch_valu_t<E, Q, 64, 8>(c, a, stream);
  else if (c.D == 128 && c.B == 8) launch_valu_t<E, Q, 128, 8>(c, a, stream);
  else if (c.D == 64 && c.B == 16) launch_valu_t<E, Q, 64, 16>(c, a, stream);
  else if (c.D == 64 && c.B == 32) launch_valu_t<E, Q, 64, 32>(c, a, stream);
  else if (c.D == 128 && c.B == 16) launch_valu_t<E, Q, 128, 16>(c, a, stream);
  else launch_valu_t<E, Q, 128, 32>(c, a, stream);
}

template <typename E, typename Q, int D, int BS>
int flat_grid_t(int S) {
  return resident_workgroups((const void *)decode_valu_kernel<E, Q, D, BS, kSchedFlat, false>, 256,
                             sizeof(int) * (S + 1));
}

template <typename E, typename Q = E>
int flat_grid_e(const CacheDesc &c, int S) {
  if (c.D == 64 && c.B == 8) return flat_grid_t<E, Q, 64, 8>(S);
  if (c.D == 128 && c.B == 8) return flat_grid_t<E, Q, 128, 8>(S);
  if (c.D == 64 && c.B == 16) return flat_grid_t<E, Q, 64, 16>(S);
  if (c.D == 64 && c.B == 32) return flat_grid_t<E, Q, 64, 32>(S);
  if (c.D == 128 && c.B == 16) return flat_grid_t<E, Q, 128, 16>(S);
  return flat_grid_t<E, Q, 128, 32>(S);
}

template <typename E, typename KV>
void launch_reduce_e(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  const dim3 grid((unsigned)a.Hq, (unsigned)a.S);
  const int mt = a.cap_tokens;
  const int G = a.Hq / c.H;
  const int HU = a.mfma ? c.H : a.Hq, GU = a.mfma ? G : 1;   // the decode kernel's work units
  NewToken nt;
  if (a.new_k != nullptr) {
    nt.k = a.new_k;
    nt.v = a.new_v;
    nt.k_scale = c.k_scale;
    nt.v_scale = c.v_scale;
    nt.kpool = c.k;
    nt.vpool = c.v;
    nt.block_tables = a.block_tables;
    nt.num_blocks = c.num_blocks;
    nt.BS = c.B;
    nt.mbps = a.max_blocks_per_seq;
    nt.cap = a.cap_tokens;
  }
  nt.Hkv = c.H;
  auto go = [&](auto kern_part, auto kern_flat, int threads) {
    if (a.flat)
      hipLaunchKernelGGL(kern_flat, grid, dim3(threads), 0, stream, a.out, (int)a.out_f32,
                         (const int *)a.ws_hdr, a.Hq, HU, GU, a.ws_ml, a.ws_acc, a.context_lens, nt);
    else
      hipLaunchKernelGGL(kern_part, grid, dim3(threads), 0, stream, a.out, (int)a.out_f32,
                         a.context_lens, a.Hq, mt, a.window, a.partition_tokens, a.num_partitions,
                         a.ws_ml, a.ws_acc, nt);
  };
  if (c.D == 64) go(decode_reduce_kernel<E, KV, 64>, decode_reduce_flat_kernel<E, KV, 64>, 64);
  else go(decode_reduce_kernel<E, KV, 128>, decode_reduce_flat_kernel<E, KV, 128>, 128);
}

}  // namespace

hipError_t launch_decode_valu(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (c.fp8()) {
    if (c.mdtype == 1) launch_valu_e<FP8, F16>(c, a, stream);
    else launch_valu_e<FP8, BF16>(c, a, stream);
  } else if (c.dtype == 0) {
    launch_valu_e<F32>(c, a, stream);
  } else if (c.dtype == 1) {
    launch_valu_e<F16>(c, a, stream);
  } else {
    launch_valu_e<BF16>(c, a, stream);
  }
  return hipGetLastError();
}

int decode_valu_flat_grid(const CacheDesc &c, int S) {
  if (c.fp8()) return c.mdtype == 1 ? flat_grid_e<FP8, F16>(c, S) : flat_grid_e<FP8, BF16>(c, S);
  if (c.dtype == 0) return flat_grid_e<F32>(c, S);
  if (c.dtype == 1) return flat_grid_e<F16>(c, S);
  return flat_grid_e<BF16>(c, S);
}

// The reduce writes the output, so it goes by the model dtype; an appending
// call's stores go by the cache's.
hipError_t launch_decode_reduce(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (c.mdtype == 0) launch_reduce_e<F32, F32>(c, a, stream);
  else if (c.mdtype == 1) c.fp8() ? launch_reduce_e<F16, FP8>(c, a, stream) : launch_reduce_e<F16, F16>(c, a, stream);
  else c.fp8() ? launch_reduce_e<BF16, FP8>(c, a, stream) : launch_reduce_e<BF16, BF16>(c, a, stream);
  return hipGetLastError();
}

}  // namespace pkv
