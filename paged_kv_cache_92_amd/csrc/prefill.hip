// Causal chunked prefill over the paged cache on the matrix cores.
//
// A chunk of a long prompt is processed as one step ("Sparse Computation and
// Memory Management for Efficient LLM Inference", pyy0715.github.io, section
// "Prefill-Decode Disaggregation"); all of its rows are known at once, so
// attention is a matrix-matrix product ("vLLM: LLM 서빙 메모리 최적화의 교과서",
// velog.io, section 01, prompt phase), causal over j <= i.
//
// Workgroup = 8 waves (two per SIMD) = one (sequence, query head, 256-row
// query tile); wave w owns 32 query rows.  The key/value positions
// 0..last row's position are walked in 64-token tiles gathered through the
// block table (staged in LDS once per workgroup) into LDS: three tile
// buffers, tile t+2 stored while tiles t and t+1 are read, one barrier per
// tile.  Each wave computes 32-token sub-tiles:
//
//   S^T (32 tokens x 32 rows) = K (32 x D) . Q^T (D x 32)
//   O^T (D x 32 rows)        += V^T (D x 32) . P^T (32 x 32)
//
// with 32x32x16 MFMAs.  The key rows are fed to the first product in a
// permuted order chosen so that each lane's 16 result rows are, per 16-token
// k-step of the second product, 8 consecutive tokens: the B operand P^T is
// built from the lane's own registers and the A operand V^T is one 16-byte
// LDS read from the dimension-major value tile.  Scores live in the log2
// domain.  Tiles wholly below a wave's first row take an unmasked loop; only
// the tiles that reach the diagonal are masked.
//
// Two routes.  The fast one keeps a fixed reference maximum per row (the
// maximum over its first 32 keys) for the whole walk, so accumulators are
// never rescaled, and runs P.V on the fp16 matrix cores (bf16 values are
// re-encoded to fp16 as tiles are staged).  If any row's accumulators or
// denominator come out non-finite (a weight beyond fp16 range, or a bf16
// value beyond it), the workgroup redoes the walk on the exact route: lazy
// rescaling of a running maximum, and bf16 products for bf16.  Workgroups
// are dispatched longest first (the (sequence, query tile) classes ranked by
// their tile counts on the device).
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// Query rows per wave: NG groups of 32 (the matrix-core tile's columns).
// Each key and value operand read from LDS feeds the products of all NG
// groups, and a wave's registers hold NG groups' queries and accumulators.
#ifndef PKV_PREFILL_NG
#define PKV_PREFILL_NG 1
#endif
constexpr int NG = PKV_PREFILL_NG;
constexpr int kWaves = 8 / NG;         // two waves per SIMD at NG = 1, one at NG = 2
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsW = 32 * NG;
constexpr int kQT = kRowsW * kWaves;   // 256 query rows per workgroup
constexpr int kKT = 64;               // key/value tokens per tile: two 32-token halves
constexpr int kNBuf = 3;              // LDS tile buffers
constexpr int kLptClasses = 256;      // (sequence, query tile) classes ranked in LDS

template <typename E>
struct Mfma32;
// kSplitP: bf16 softmax weights enter P.V as hi + lo pairs (see split_bf16x2).
template <>
struct Mfma32<F16> {
  static constexpr bool kSplitP = false;
  __device__ static f32x16 mma(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_f16x2(lo, hi); }
};
template <>
struct Mfma32<BF16> {
  static constexpr bool kSplitP = true;
  __device__ static f32x16 mma(const u32x4 &a, const u32x4 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
};

// Row i of a 32-token score product (i = 8a + 4h + b) holds token perm(i) of
// its half-tile.
__device__ __forceinline__ int perm_row(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}
// LDS row of tile token k.  Rows are D + 8 elements (an odd number of 16-byte
// bank groups), and bit 2 is flipped on odd 8-token groups: the 8 tokens that
// one 8-lane group of a score-operand read touches (perm rows 0-3 and 8-11,
// and the like) then sit in 8 distinct bank groups.
__device__ __forceinline__ int kslot(int k) { return k ^ (((k >> 3) & 1) << 2); }

// Lazy rescaling (exact route): a row keeps its reference maximum until a new
// score beats it by more than 2^kRescaleLog2; weights stay <= 2^kRescaleLog2
// meanwhile (no overflow in fp32, fp16 or bf16), and the final o = acc / l is
// unaffected.
constexpr float kRescaleLog2 = 8.f;
// Fixed reference (fast route): each row's reference is the maximum of its
// first 32 keys, kept for the whole walk.  Later weights 2^(s - ref) may
// exceed 1; the walk is valid as long as they fit fp16 (s - ref < 16).  A
// weight beyond that packs to an infinity, which makes that row's
// accumulators or denominator non-finite: the workgroup then redoes the walk
// on the exact route.

template <int R>
using Grp = std::integral_constant<int, R>;

// Max and sum of x over lanes l and l ^ 32.
__device__ __forceinline__ float pair_max(float x) { return __builtin_fmaxf(x, __shfl_xor(x, 32)); }
__device__ __forceinline__ float pair_sum(float x) { return x + __shfl_xor(x, 32); }

// E4M3 codes -> 16-bit values, exactly (every E4M3 value is an fp16 and a
// bf16 value): the 16 codes of c become two 8-element operands.
template <typename T>
__device__ __forceinline__ void widen16(const u32x4 &c, u32x4 &lo, u32x4 &hi) {
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // One scaled conversion (scale 1) per code pair: bytes 0-1, then 2-3.
    if constexpr (std::is_same<T, F16>::value) {
      w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.f, false));
      w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c[i], 1.f, true));
    } else {
      w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.f, false));
      w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[i], 1.f, true));
    }
  }
  lo = u32x4{w[0], w[1], w[2], w[3]};
  hi = u32x4{w[4], w[5], w[6], w[7]};
}

// E: the queries' and outputs' type (f16 or bf16).  KV: the cache's elements,
// E itself or FP8 (E4M3 codes: keys widened to E and values to fp16 as tiles
// are staged; the key scale is folded into scale_log2, the value scale
// multiplies the normalised output).
template <typename E, typename KV, int D, int BS>
__global__ __launch_bounds__(kThreads, 8 / kWaves) void prefill_kernel(
    void *__restrict__ out, int out_f32, const uint16_t *__restrict__ q,
    const void *__restrict__ kpool_, const void *__restrict__ vpool_,
    const int32_t *__restrict__ query_start_loc, const int32_t *__restrict__ context_lens,
    const int32_t *__restrict__ block_tables, int64_t num_blocks, int Hkv, int Hq, int mbps,
    int staged, int nqt, float scale_log2, float v_scale) {
  // staged: block-table entries per sequence that fit the dynamic LDS
  // (enough for max_context_len); positions beyond them are never walked.
  constexpr bool kFP8 = KV::kBytes == 1;
  constexpr int KS = D / 16;           // k-steps of the score product
  constexpr int DT = D / 32;           // 32-dimension tiles of the output
  constexpr int KX = 64 / KV::kBytes;  // elements per 64-byte key piece
  constexpr int KROW = D + 8;          // LDS key row (16-bit elements)
  constexpr int VROW = kKT + 8;        // LDS value row (16-bit elements)
  constexpr int KPR = kThreads / 256;  // key pieces per chunk round
  constexpr int NPC = D / KX;          // key pieces per row
  // 16-byte key chunks per thread (an 8-bit row of 64 dimensions has one
  // piece: half of the threads then load none).
  constexpr int KPT = NPC >= KPR ? NPC / KPR : 1;
  // Value chunks: 8 tokens (16-bit) or 16 tokens (8-bit) of one dimension.
  constexpr int VTC = 16 / KV::kBytes;           // tokens per chunk
  constexpr int VDR = kThreads / (kKT / VTC);    // value dimensions per chunk round
  constexpr int VPT = D >= VDR ? D / VDR : 1;    // chunks per thread
  static_assert((KPT * KPR * KX == D || (NPC < KPR && KX == D)) && (VPT * VDR == D || VDR == 2 * D),
                "whole rows per chunk round");
  const uint8_t *kpool = (const uint8_t *)kpool_;
  const uint8_t *vpool = (const uint8_t *)vpool_;

  // Work item.  The hardware hands out block ids in order as workgroups
  // finish, so the longest items go first (greedy longest-processing-time
  // order): the (sequence, query tile) classes are ranked by their number of
  // 64-token tiles, and block b takes head b % Hq of the class ranked b / Hq.
  // Every workgroup ranks the classes itself (in LDS, from the lengths); with
  // more than kLptClasses classes the order is the XCD-aware one instead,
  // which keeps the query tiles of one (sequence, head) on one XCD.
  const int tid = threadIdx.x;
  __shared__ int sLen[kLptClasses];
  __shared__ int sPick;
  int qt, hq, s;
  const int ncls = gridDim.x / Hq;  // S * nqt: the grid is S * Hq * nqt blocks
  if (ncls <= kLptClasses) {
    for (int c = tid; c < ncls; c += kThreads) {
      const int cs = c / nqt, cq = c % nqt;
      const int ql = query_start_loc[cs + 1] - query_start_loc[cs];
      const int h0 = min(context_lens[cs], staged * BS) - ql;
      sLen[c] = (cq * kQT < ql && h0 >= 0) ? (h0 + min(cq * kQT + kQT, ql) - 1) / kKT + 1 : 0;
    }
    __syncthreads();
    const int want = blockIdx.x / Hq;
    for (int c = tid; c < ncls; c += kThreads) {
      const int lc = sLen[c];
      int rank = 0;
      for (int o = 0; o < ncls; ++o) rank += sLen[o] > lc || (sLen[o] == lc && o < c);
      if (rank == want) sPick = c;
    }
    __syncthreads();
    const int c = sPick;
    s = c / nqt;
    qt = c % nqt;
    hq = blockIdx.x % Hq;
  } else {
    const int nwork = gridDim.x;
    int wid = blockIdx.x;
    if ((nwork & 7) == 0) wid = (wid & 7) * (nwork >> 3) + (wid >> 3);
    qt = nqt - 1 - wid % nqt;
    hq = (wid / nqt) % Hq;
    s = wid / (nqt * Hq);
  }

  const int qs = query_start_loc[s];
  const int qlen = query_start_loc[s + 1] - qs;
  if (qt * kQT >= qlen) return;
  const int ctx = min(context_lens[s], staged * BS);
  const int hist = ctx - qlen;
  if (hist < 0) return;
  const int hkv = hq / (Hq / Hkv);

  const int lane = tid & (kWave - 1);
  const int w = uniform(tid >> 6);
  const int j32 = lane & 31;  // query column of this lane within its group
  const int h = lane >> 5;    // k-half / row group of the MFMA layouts

  // Three LDS tile buffers: tile t+2 is stored while tiles t and t+1 are read.
  __shared__ __attribute__((aligned(16))) uint16_t sK[kNBuf][kKT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kNBuf][D * VROW];
  __shared__ int sBad;        // the fast route produced a non-finite result
  extern __shared__ int sBT[];  // block ids of the positions this workgroup reads

  const int wrow0 = qt * kQT + kRowsW * w;  // first chunk row of this wave
  const int wg_last = min(qt * kQT + kQT, qlen) - 1;
  const int ntiles = (hist + wg_last) / kKT + 1;
  // 32-token sub-tiles this wave computes (up to its rows' last position);
  // the workgroup's remaining tiles it only stages.
  const int nu_w = wrow0 < qlen ? (hist + min(wrow0 + kRowsW, qlen) - 1) / 32 + 1 : 0;
  // Position of this lane's query in each group, and of each group's first row.
  int qpos[NG], gmin[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    qpos[g] = hist + min(wrow0 + 32 * g + j32, qlen - 1);
    gmin[g] = hist + min(wrow0 + 32 * g, qlen - 1);
  }

  // Stage the block table once; tile loads then look block ids up in LDS.
  if (tid == 0) sBad = 0;
  {
    const int32_t *bt = block_tables + (size_t)s * mbps;
    const int nbt = min((ntiles * kKT + BS - 1) / BS, staged);
    for (int i = tid; i < nbt; i += kThreads) {
      const int32_t b = bt[i];
      sBT[i] = (b >= 0 && b < num_blocks) ? b : -1;
    }
  }

  // Q^T operands: query column j32 of group g, dimensions 16*ks + 8*h .. +8
  // (zero past the chunk).
  u32x4 qb[NG][KS];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int row = wrow0 + 32 * g + j32;
    const bool valid = row < qlen;
    const uint16_t *qrow = q + ((size_t)(qs + (valid ? row : 0)) * Hq + hq) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[g][ks] = valid ? load16(qrow + 16 * ks) : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // Global -> register staging of one tile.  Thread tid moves the 16-byte
  // column tid%4 of token (tid/4)%64's key row in pieces tid/256 + KPR*i (a
  // wave reads 16 tokens x 64 bytes contiguously per piece), and value
  // chunks (dimension tid/(64/VTC) + VDR*i, tokens VTC*(tid%(64/VTC))..+VTC).
  const int ktok = (tid >> 2) & (kKT - 1), ksub = tid & 3, kpc = tid >> 8;
  const int vtok = VTC * (tid % (kKT / VTC)), vdim = tid / (kKT / VTC);
  const bool kload = NPC >= KPR || kpc < NPC;   // this thread has key chunks
  const bool vload = D >= VDR || vdim < D;      // ... and value chunks
  // Byte offsets of this thread's chunks within one block's key / value tile
  // (for every tile: 64-token tiles start on block boundaries), and the bytes
  // between consecutive blocks of a pool.
  const uint32_t blk_bytes = (uint32_t)Hkv * D * BS * KV::kBytes;
  const uint8_t *kbase = kpool + ((size_t)hkv * D * BS + (ktok % BS) * KX) * KV::kBytes + 16 * ksub;
  const uint8_t *vbase = vpool + ((size_t)hkv * D * BS + vtok % BS) * KV::kBytes;
  const uint8_t *vbase2 = vpool + (size_t)hkv * D * BS * KV::kBytes;
  // FULL: the tile lies within the context (every tile but the last), so no
  // position needs a bounds check or a mask.
  auto load_rows = [&](int t0, auto full_t, u32x4 (&kreg)[KPT], u32x4 (&vreg)[VPT]) {
    constexpr bool FULL = decltype(full_t)::value;
    if (kload) {
      const int pos = t0 + ktok;
      // Positions past the context read a harmless in-pool address; their
      // scores are masked.  An invalid block id (a broken caller contract)
      // reads block 0 instead of faulting.
      const int blk = (FULL || pos < ctx) ? max(sBT[pos / BS], 0) : 0;
      const uint8_t *kb = kbase + (size_t)(uint32_t)blk * blk_bytes;
#pragma unroll
      for (int i = 0; i < KPT; ++i) kreg[i] = load16(kb + (size_t)(kpc + KPR * i) * BS * 64);
    }
    if (vload) {
      const int pos = t0 + vtok;
      const int blk = (FULL || pos < ctx) ? max(sBT[pos / BS], 0) : 0;
      const uint8_t *vblk = vbase + (size_t)(uint32_t)blk * blk_bytes;
      // 8-bit values in 8-token blocks: the chunk's second half is the next block's.
      const uint8_t *vblk2 = vblk;
      if constexpr (VTC > BS) {
        const int blk2 = (FULL || pos + BS < ctx) ? max(sBT[(pos + BS) / BS], 0) : 0;
        vblk2 = vbase2 + (size_t)(uint32_t)blk2 * blk_bytes;
      }
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const size_t row = (size_t)(vdim + VDR * i) * BS * KV::kBytes;
        u32x4 x;
        if constexpr (VTC > BS) {
          const u32x2 a = load8(vblk + row), b = load8(vblk2 + row);
          x = u32x4{a[0], a[1], b[0], b[1]};
        } else {
          x = load16(vblk + row);
        }
        if (!FULL && pos + VTC > ctx) {
          // Slots past the context may hold anything (NaN included): zero them.
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            uint32_t keep = 0;
#pragma unroll
            for (int e = 0; e < 4 / KV::kBytes; ++e)
              if (pos + (4 / KV::kBytes) * k + e < ctx) keep |= (KV::kBytes == 1 ? 0xffu : 0xffffu) << (8 * KV::kBytes * e);
            x[k] &= keep;
          }
        }
        vreg[i] = x;
      }
    }
  };
  auto load_tile = [&](int t, u32x4 (&kreg)[KPT], u32x4 (&vreg)[VPT]) {
    const int t0 = t * kKT;
    if (t0 + kKT <= ctx) load_rows(t0, std::true_type{}, kreg, vreg);
    else load_rows(t0, std::false_type{}, kreg, vreg);
  };
  // Registers -> LDS buffer buf.  CONV: bf16 values re-encoded to fp16 (exact
  // below 65536 in magnitude; larger ones become infinities, which the walk's
  // result check catches).  8-bit codes: keys widened to E, values to fp16.
  auto store_tile = [&](auto conv, int buf, const u32x4 (&kreg)[KPT], const u32x4 (&vreg)[VPT]) {
    constexpr bool CONV = decltype(conv)::value;
    uint16_t *kd = &sK[buf][kslot(ktok) * KROW + (16 / KV::kBytes) * ksub];
    if (kload) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if constexpr (kFP8) {
          u32x4 lo, hi;
          widen16<E>(kreg[i], lo, hi);
          *(u32x4 *)(kd + KX * (kpc + KPR * i)) = lo;
          *(u32x4 *)(kd + KX * (kpc + KPR * i) + 8) = hi;
        } else {
          *(u32x4 *)(kd + KX * (kpc + KPR * i)) = kreg[i];
        }
      }
    }
    if (vload) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        uint16_t *vd = &sV[buf][(vdim + VDR * i) * VROW + vtok];
        if constexpr (kFP8) {
          u32x4 lo, hi;
          widen16<F16>(vreg[i], lo, hi);
          *(u32x4 *)vd = lo;
          *(u32x4 *)(vd + 8) = hi;
        } else {
          u32x4 x = vreg[i];
          if constexpr (CONV) {
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = pack_f16x2(as_f32(x[k] << 16), as_f32(x[k] & 0xffff0000u));
          }
          *(u32x4 *)vd = x;
        }
      }
    }
  };

  // Per-lane LDS operand bases: key row kslot(perm(j32)) (half 1: +32 rows),
  // column 8*h; value row j32 (dimension tile dt: +32 rows), token 8*h.
  const int kop0 = kslot(perm_row(j32)) * KROW + 8 * h;
  const int vop0 = j32 * VROW + 8 * h;

  float m[NG], l[NG];   // reference max (scaled log2 units) and this lane's denominator share
  f32x16 acc[NG][DT];
  const f32x16 zero16 = {};

  // The whole walk over the key/value tiles.  CONV (bf16 only): P.V on the
  // fp16 matrix cores.  FIXED: the fast route with a fixed reference max per
  // row (no rescaling of the accumulators); otherwise the exact route with
  // lazy rescaling.  Compute runs in 32-token sub-tiles u = 2t + half.
  auto attend = [&](auto conv, auto fixed) {
    constexpr bool CONV = decltype(conv)::value;
    constexpr bool FIXED = decltype(fixed)::value;
    // Values in LDS are fp16 for an f16 cache, for bf16 on the fast route and
    // for 8-bit codes; bf16 on bf16's exact route.
    using PV = typename std::conditional<CONV || kFP8 || std::is_same<E, F16>::value, Mfma32<F16>,
                                         Mfma32<E>>::type;
    constexpr bool kSplit = PV::kSplitP;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[g][dt] = zero16;
    }

    // Scores of every row group against sub-tile `half` of tile buffer buf:
    // each key operand read from LDS feeds all groups' products.
    auto qk = [&](int buf, int half, f32x16 (&st)[NG]) {
      const uint16_t *kb = &sK[buf][kop0 + 32 * half * KROW];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 a = *(const u32x4 *)(kb + 16 * ks);
#pragma unroll
        for (int g = 0; g < NG; ++g) st[g] = Mfma32<E>::mma(a, qb[g][ks], ks == 0 ? zero16 : st[g]);
      }
    };
    // Causal mask of group g's scores (only on sub-tiles that reach past the
    // group's first row; MAYBE: the caller's tile may); u0 is the sub-tile's
    // first position.
    auto mask = [&](int g, int u0, f32x16 &st, auto maybe) {
      if (decltype(maybe)::value && u0 + 31 > gmin[g]) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int pos = u0 + 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
            if (pos > qpos[g]) st[4 * a + b] = -INFINITY;
          }
      }
    };
    // Row max of scores (log2 units).
    auto row_max = [&](const f32x16 &st) -> float {
      float mraw = __builtin_fmaxf(__builtin_fmaxf(st[0], st[1]), st[2]);
#pragma unroll
      for (int i = 3; i < 15; i += 2) mraw = __builtin_fmaxf(__builtin_fmaxf(mraw, st[i]), st[i + 1]);
      mraw = __builtin_fmaxf(mraw, st[15]);
      return pair_max(mraw) * scale_log2;  // scale > 0: the max commutes with scaling
    };
    // Exact route: running-max update and lazy rescale of group g.
    auto rescale = [&](int g, const f32x16 &st) {
      const float mb = row_max(st);
      if (__any(mb > m[g] + kRescaleLog2)) {
        const float mnew = __builtin_fmaxf(m[g], mb);
        const float alpha = fast_exp2(m[g] - mnew);  // 1 for rows that keep their reference
        m[g] = mnew;
        l[g] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[g][dt] *= alpha;
      }
    };
    // Weights of group g, packed as the P^T operands of the sub-tile's two
    // 16-token k-steps (c: tokens 16c .. 16c+15; this lane's 8 are
    // 16c + 8h .. +8), and the lane's share of the denominator.
    auto weights = [&](int g, const f32x16 &st, u32x4 (&pk)[2], u32x4 (&pl)[2]) {
      const float mr = m[g];
      float lsum = l[g];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) p[k] = fast_exp2(fmaf(st[8 * c + k], scale_log2, -mr));
        if constexpr (kSplit) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) split_bf16x2(p[2 * k], p[2 * k + 1], hi[k], lo[k]);
          pk[c] = u32x4{hi[0], hi[1], hi[2], hi[3]};
          pl[c] = u32x4{lo[0], lo[1], lo[2], lo[3]};
#pragma unroll
          for (int k = 0; k < 8; ++k) lsum += p[k];
        } else {
          // fp16 weights; the denominator sums the same rounded weights the
          // product uses (two per dot instruction, fp32 accumulation).
          const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t wv = pack_f16x2(p[2 * k], p[2 * k + 1]);
            pk[c][k] = wv;
            lsum = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, wv), one2, lsum, false);
          }
        }
      }
      l[g] = lsum;
    };
    // O^T of every group += V^T . P^T over sub-tile `half` of tile buffer
    // buf, each value operand read once for all groups.
    auto pv = [&](int buf, int half, const u32x4 (&pk)[NG][2], const u32x4 (&pl)[NG][2]) {
      const uint16_t *vb = &sV[buf][vop0 + 32 * half];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4 a = *(const u32x4 *)(vb + 32 * dt * VROW + 16 * c);
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            acc[g][dt] = PV::mma(a, pk[g][c], acc[g][dt]);
            if constexpr (kSplit) acc[g][dt] = PV::mma(a, pl[g][c], acc[g][dt]);
          }
        }
    };

    u32x4 kreg[KPT], vreg[VPT];
    // Prologue: tiles 0 and 1 in LDS, tile 2 in registers.
    load_tile(0, kreg, vreg);
    store_tile(conv, 0, kreg, vreg);
    if (ntiles > 1) {
      load_tile(1, kreg, vreg);
      store_tile(conv, 1, kreg, vreg);
    }
    if (ntiles > 2) load_tile(2, kreg, vreg);
    __syncthreads();

    f32x16 sc[NG];
    qk(0, 0, sc);
    if constexpr (FIXED) {
      // Reference max of each row: its first 32 keys (key 0 is always one of
      // them, so it is finite).
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        mask(g, 0, sc[g], std::true_type{});
        m[g] = row_max(sc[g]);
      }
    }
    // One 64-token tile t (buffer cur; nxt and aft hold tiles t+1 and t+2):
    // its two 32-token sub-tiles u = 2t + half, then tile t+2 goes from
    // registers to LDS and tile t+3 from HBM to registers.  A sub-tile
    // starts with its scores (computed by the previous one) masked and, on
    // the exact route, their maxima handled; then it computes the next
    // sub-tile's scores while its own weights are formed, then its P.V.  The
    // next scores are computed even past the wave's last sub-tile (then from
    // a stale buffer, and never used), so every sub-tile runs the same code.
    // MASKED: the tile may reach past the wave's first row (causal mask, and
    // sub-tiles past the wave's last row skipped).
    auto tile_step = [&](int t, int cur, int nxt, int aft, auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      auto sub = [&](auto hv) {
        constexpr int half = decltype(hv)::value;
        const int u0 = t * kKT + 32 * half;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          mask(g, u0, sc[g], masked);
          if constexpr (!FIXED) rescale(g, sc[g]);
        }
        f32x16 nx[NG];
        qk(half ? nxt : cur, half ^ 1, nx);
        u32x4 pk[NG][2], pl[NG][2];
#pragma unroll
        for (int g = 0; g < NG; ++g) weights(g, sc[g], pk[g], pl[g]);
        pv(cur, half, pk, pl);
#pragma unroll
        for (int g = 0; g < NG; ++g) sc[g] = nx[g];
      };
      if (!MASKED || 2 * t < nu_w) sub(Grp<0>{});
      if (!MASKED || 2 * t + 1 < nu_w) sub(Grp<1>{});
      if (t + 2 < ntiles) {
        store_tile(conv, aft, kreg, vreg);
        if (t + 3 < ntiles) load_tile(t + 3, kreg, vreg);
      }
      __syncthreads();
    };
    // Tiles before the first that reaches past the wave's first row need no
    // mask (and are all within the wave's sub-tiles).
    const int t_diag = nu_w > 0 ? min(ntiles, (gmin[0] + 1) / kKT) : 0;
    int t = 0, cur = 0;
    for (; t < t_diag; ++t) {
      const int nxt = cur == kNBuf - 1 ? 0 : cur + 1;
      tile_step(t, cur, nxt, nxt == kNBuf - 1 ? 0 : nxt + 1, std::false_type{});
      cur = nxt;
    }
    for (; t < ntiles; ++t) {
      const int nxt = cur == kNBuf - 1 ? 0 : cur + 1;
      tile_step(t, cur, nxt, nxt == kNBuf - 1 ? 0 : nxt + 1, std::true_type{});
      cur = nxt;
    }
  };

  // The fast route first: fixed reference maxima and, for bf16, P.V on the
  // fp16 matrix cores.  The workgroup redoes the walk on the exact route
  // (lazy rescaling, bf16 products for bf16) if any row's accumulators or
  // denominator came out non-finite: a weight beyond fp16 (a row whose max
  // outgrew its reference by 2^16), or for bf16 a value of magnitude >= 65536
  // (no fp16 encoding).  A non-finite input gives the same answer on both
  // routes.  The decision is the workgroup's (its waves share the barriers);
  // nothing was written meanwhile.
  constexpr bool kConvV = std::is_same<E, BF16>::value;
  attend(std::integral_constant<bool, kConvV>{}, std::true_type{});
  {
    bool bad = false;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      bad |= !__builtin_isfinite(pair_sum(l[g]));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) bad |= !__builtin_isfinite(acc[g][dt][i]);
    }
    if (__any(bad) && lane == 0) sBad = 1;
  }
  __syncthreads();
  if (sBad) attend(std::false_type{}, std::false_type{});

  // Lanes l and l^32 hold the two row halves of the same query column.
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float ltot = pair_sum(l[g]);
    const int row = wrow0 + 32 * g + j32;
    if (row < qlen) {
      const float inv = (kFP8 ? v_scale : 1.f) / ltot;
      const size_t orow = ((size_t)(qs + row) * Hq + hq) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int dim = 32 * dt + 8 * a + 4 * h;
          const float o0 = acc[g][dt][4 * a] * inv, o1 = acc[g][dt][4 * a + 1] * inv;
          const float o2 = acc[g][dt][4 * a + 2] * inv, o3 = acc[g][dt][4 * a + 3] * inv;
          if (out_f32) {
            *(f32x4 *)((float *)out + orow + dim) = f32x4{o0, o1, o2, o3};
          } else {
            *(u32x2 *)((uint16_t *)out + orow + dim) =
                u32x2{Mfma32<E>::pack2(o0, o1), Mfma32<E>::pack2(o2, o3)};
          }
        }
    }
  }
}

// Block-table entries staged per workgroup: the table's width, or fewer when
// max_context_len needs fewer.
int staged_entries(const PrefillArgs &a, int B) {
  return std::min(a.max_blocks_per_seq, (a.max_context_len + B - 1) / B);
}

template <typename E, typename KV, int D, int BS>
size_t lds_bytes_t(const PrefillArgs &a) {
  // The kernel's static LDS is a property of its code: asked once.
  static const size_t static_bytes = [] {
    hipFuncAttributes fa{};
    return hipFuncGetAttributes(&fa, (const void *)prefill_kernel<E, KV, D, BS>) == hipSuccess
               ? fa.sharedSizeBytes
               : SIZE_MAX;
  }();
  if (static_bytes == SIZE_MAX) return SIZE_MAX;
  return static_bytes + sizeof(int) * (size_t)staged_entries(a, BS);
}

template <typename E, typename KV>
size_t lds_bytes_e(const CacheDesc &c, const PrefillArgs &a) {
  if (c.D == 64 && c.B == 8) return lds_bytes_t<E, KV, 64, 8>(a);
  if (c.D == 128 && c.B == 8) return lds_bytes_t<E, KV, 128, 8>(a);
  if (c.D == 64 && c.B == 16) return lds_bytes_t<E, KV, 64, 16>(a);
  if (c.D == 64 && c.B == 32) return lds_bytes_t<E, KV, 64, 32>(a);
  if (c.D == 128 && c.B == 16) return lds_bytes_t<E, KV, 128, 16>(a);
  return lds_bytes_t<E, KV, 128, 32>(a);
}

template <typename E, typename KV, int D, int BS>
void launch_t(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  const int nqt = (a.max_query_len + kQT - 1) / kQT;
  const int64_t nwork = (int64_t)a.S * a.Hq * nqt;
  const int staged = staged_entries(a, BS);
  const size_t lds = sizeof(int) * (size_t)staged;   // staged block table
  // k_scale and v_scale are 1 unless the cache is 8-bit.
  hipLaunchKernelGGL((prefill_kernel<E, KV, D, BS>), dim3((unsigned)nwork), dim3(kThreads), lds, stream,
                     a.out, (int)a.out_f32, (const uint16_t *)a.q, (const void *)c.k, (const void *)c.v,
                     a.query_start_loc, a.context_lens, a.block_tables, c.num_blocks, c.H, a.Hq,
                     a.max_blocks_per_seq, staged, nqt, a.scale * kLog2e * c.k_scale, c.v_scale);
}

template <typename E, typename KV>
void launch_e(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  if (c.D == 64 && c.B == 8) launch_t<E, KV, 64, 8>(c, a, stream);
  else if (c.D == 128 && c.B == 8) launch_t<E, KV, 128, 8>(c, a, stream);
  else if (c.D == 64 && c.B == 16) launch_t<E, KV, 64, 16>(c, a, stream);
  else if (c.D == 64 && c.B == 32) launch_t<E, KV, 64, 32>(c, a, stream);
  else if (c.D == 128 && c.B == 16) launch_t<E, KV, 128, 16>(c, a, stream);
  else launch_t<E, KV, 128, 32>(c, a, stream);
}

}  // namespace

// The queries' and outputs' type is the cache's, or for an 8-bit cache the
// model dtype (f16 or bf16).
size_t prefill_lds_bytes(const CacheDesc &c, const PrefillArgs &a) {
  if (c.fp8()) return c.mdtype == 1 ? lds_bytes_e<F16, FP8>(c, a) : lds_bytes_e<BF16, FP8>(c, a);
  return c.dtype == 1 ? lds_bytes_e<F16, F16>(c, a) : lds_bytes_e<BF16, BF16>(c, a);
}

hipError_t launch_prefill(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  if (a.max_query_len == 0 || a.S == 0) return hipSuccess;
  if (c.fp8()) {
    if (c.mdtype == 1) launch_e<F16, FP8>(c, a, stream);
    else launch_e<BF16, FP8>(c, a, stream);
  } else if (c.dtype == 1) {
    launch_e<F16, F16>(c, a, stream);
  } else {
    launch_e<BF16, BF16>(c, a, stream);
  }
  return hipGetLastError();
}

}  // namespace pkv
