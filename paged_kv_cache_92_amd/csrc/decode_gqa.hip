// Grouped-query paged decode on the matrix cores (f16/bf16 queries over an
// f16, bf16 or 8-bit E4M3 cache).
//
// G query heads share one KV head ("Sparse Computation and Memory Management
// for Efficient LLM Inference", pyy0715.github.io, section "The Hidden Waste
// of KV Cache": 32 query heads over 8 KV heads).  A workgroup (8 waves) owns
// one (partition, KV head, sequence) at a time, its waves taking interleaved
// steps; the G queries are stacked into the N
// columns of 16x16 matrix products so each key/value tile is read once for
// the whole group.  Per 16-token sub-tile, each wave computes
//
//   S^T (16 tokens x 16 heads) = K (16 x D) . Q^T (D x 16)     16x16x32 MFMAs
//   O^T (D x 16 heads)        += V^T (D x 16) . P^T (16 x 16)  16x16x16 MFMAs
//
// Lane l holds column l%16 (a query head) of S^T with tokens 4*(l/16)+j, which
// is exactly the B-operand layout of P^T for the second product, so the
// softmax weights never leave their registers.  V^T comes straight from the
// dimension-major value tile (4 consecutive tokens of one dimension = 8
// bytes per lane; for 32-token blocks 8 tokens = 16 bytes and 16x16x32
// products).  K^T operands come from the key tile's 64-byte pieces: one
// k-step of 32 dimensions is one piece, so a wave load reads 16 tokens x 64
// bytes contiguously.  The running max and denominator are per head, i.e. per
// lane column, as in the block-wise walk of "vLLM — KV Cache와 PagedAttention
// 완전 해부" (hrletsgo.me), "부록".  Scores are kept in the log2 domain.
#include <algorithm>

#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"
#include "pkv_plan.h"

namespace pkv {
namespace {

// Waves per work item.  Eight (two workgroups of them resident per CU, as
// many waves as four of four) measured 3% faster per call than four at the
// grouped-query shape: each item's tiles stream through half as many steps
// per wave.
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

template <typename E>
struct Mfma;

// kSplitP: the softmax weights P enter the P.V product as hi + lo bf16 pairs
// (bf16 alone keeps 8 significant bits, too coarse for 2e-3 output accuracy);
// fp16 keeps 11 bits and goes in as one operand.
template <>
struct Mfma<F16> {
  static constexpr bool kSplitP = false;
  __device__ static f32x4 qk(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) {
    return (uint32_t)f32_to_f16_bits(lo) | ((uint32_t)f32_to_f16_bits(hi) << 16);
  }
};

template <>
struct Mfma<BF16> {
  static constexpr bool kSplitP = true;
  __device__ static f32x4 qk(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  __device__ static f32x4 pv(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }
};

// Token (within the block) that row i of score sub-tile sb holds.  For 32-token
// blocks, rows 4g..4g+3 of sub-tiles 0 and 1 are tokens 8g..8g+7, the k-range
// of lane group g in a 16x16x32 product.
template <int BS>
__device__ __forceinline__ int token_of_row(int sb, int i) {
  if constexpr (BS == 32) return 8 * (i >> 2) + 4 * sb + (i & 3);
  else return 16 * sb + i;
}

// E4M3 codes -> the matrix-core input type, exactly (every E4M3 value is an
// fp16 and a bf16 value): 4 codes of word w become two packed pairs.
template <typename E>
__device__ __forceinline__ u32x2 widen4(uint32_t w) {
  // One scaled conversion (scale 1, so exact) per code pair, bytes 0-1 then 2-3.
  if constexpr (std::is_same<E, F16>::value) {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, true))};
  } else {
    return u32x2{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true))};
  }
}

// One work item: blocks [b0, b1) of sequence s for the G query heads of KV
// head hkv, positions before the sliding window's start (window > 0)
// masked; head h's merged result goes to the output or to workspace
// partial row dest.base + h * dest.stride.  `lds_dyn` holds the cross-wave
// merge buffers.  E is the query / matrix-core type; KV the cache element
// (E itself, or FP8: key codes are widened to E and value codes to fp16
// right after the loads, so that P.V takes the weights as one fp16 operand
// instead of a bf16 hi + lo pair; the key scale is folded into scale_log2
// and v_scale multiplies the merged sums).
// APPEND: the sequence's new token (position L-1) is taken from the input
// rows ap.k / ap.v, in cache format, instead of the pool, whose slot is
// written by the reduce kernel.
template <typename E, typename KV, int D, int BS, bool APPEND>
__device__ __forceinline__ void mfma_item(
    float *lds_dyn, int s, int hkv, int b0, int b1, Dest dest, void *__restrict__ out,
    int out_f32, const uint16_t *__restrict__ q, const typename KV::storage *__restrict__ kpool,
    const typename KV::storage *__restrict__ vpool, const int32_t *__restrict__ block_tables,
    const int32_t *__restrict__ context_lens, int64_t num_blocks, int Hkv, int G, int mbps,
    int cap, int window, float scale_log2, float v_scale, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, const Append<E> &ap) {
  constexpr bool kFP8 = KV::kBytes == 1;
  using PVE = typename std::conditional<kFP8, F16, E>::type;   // the P.V product's type
  constexpr int KS = D / 32;    // k-steps of the score product
  constexpr int NT = D / 16;    // 16-dimension tiles of the output
  // 8- and 16-token blocks are taken two at a time: a step covers GB tokens,
  // and 32-token steps halve the fixed work per token (scores, softmax and
  // products are issued per step) and let P.V run as 16x16x32 products over
  // 16-byte value operands.
  constexpr bool kPair = BS == 8 || BS == 16;
  constexpr int GB = kPair ? 2 * BS : BS;
  constexpr int SUB = GB / 16;  // 16-token sub-tiles per step
  // 32-token steps: the two sub-tiles' score rows are interleaved so each
  // lane ends up with 8 consecutive tokens, and P.V runs as 16x16x32 products
  // over 16-byte V^T operands.
  constexpr bool kWide = GB == 32;
  const Span sp = seq_span(context_lens, s, cap, window);
  const int lo = sp.lo;                      // first attended position
  const int tok0 = max(b0 * BS, lo);
  const int tok1 = min(sp.hi, b1 * BS);
  if (tok0 >= tok1) return;
  const int blk0 = b0;
  const int nblk = b1 - b0;
  const int Hq = Hkv * G;

  int lane = threadIdx.x & (kWave - 1);
  const int w = uniform(threadIdx.x >> 6);
  int n16 = lane & 15;   // query head (column) / token row / dimension row
  int g4 = lane >> 4;    // k-group of the operands, row group of the result

  // Cross-wave merge buffers, sized for the G live heads:
  // m[kWaves][16], l[kWaves][16], acc[kWaves][G][D + 1].
  float *lds_m = lds_dyn;
  float *lds_l = lds_dyn + kWaves * 16;
  float *lds_acc = lds_dyn + 2 * kWaves * 16;
  auto acc_at = [&](int wv, int h, int e) -> float & { return lds_acc[(wv * G + h) * (D + 1) + e]; };

  // Q^T operand: head n16 of the group (zero past G); k-step ks covers
  // dimensions 32*ks + 8*g4 .. +8 (16-bit cache) or, over an 8-bit cache
  // whose loads bring 16 dimensions of a 64-dimension piece, 64*(ks/2) +
  // 16*g4 + 8*(ks%2) .. +8: the contraction order only has to match the
  // keys'.
  auto qdim = [&](int ks) { return kFP8 ? 64 * (ks >> 1) + 16 * g4 + 8 * (ks & 1) : 32 * ks + 8 * g4; };
  u32x4 qb[KS];
  {
    const bool valid = n16 < G;
    const uint16_t *qrow = q + ((size_t)s * Hq + hkv * G + (valid ? n16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = valid ? load16(qrow + qdim(ks)) : u32x4{0, 0, 0, 0};
  }

  float m = -INFINITY;  // running max of head n16 (log2 domain)
  float l = 0.f;        // this lane's share of the denominator of head n16
  f32x4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t *bt = block_tables + (size_t)s * mbps;
  constexpr int STEP = kPair ? 2 : 1;
  using TS = typename KV::storage;
  // One step of a wave: block b of the item (and b+1 for a pair).  `app`
  // (std::true_type) marks the step that appends the new token.
  auto step = [&](const int b, auto app) {
    constexpr bool kApp = decltype(app)::value;
    const int lb = blk0 + b;
    // Appending step: the new token's index in the step; over a 16-bit cache
    // the lanes holding its key rows load them from the input row in place
    // of the pool's slot.
    const int j = kApp ? sp.hi - 1 - lb * BS : -1;
    const TS *knew = nullptr;
    if constexpr (kApp && !kFP8) knew = (const TS *)ap.k + ((size_t)s * Hkv + hkv) * D + 8 * g4;
    int64_t phys = uniform(bt[lb]);
    // Key and value tiles this lane reads: one block's, or for a pair those of
    // block lb + t/BS for the lane's tokens t (key rows: block n16 / 8 of the
    // pair for every sub-tile; value tokens 4*g4..+4 or, 32-token steps,
    // 8*g4..+8: block g4 / 2).  The second block of a pair is read only if the
    // item covers it (past the item its tokens are masked and block lb is
    // read in its place); there an out-of-range id reads block 0 instead of
    // faulting, while a single block with such an id is skipped.
    const TS *kt, *vt;
    int64_t phys2 = phys;
    bool ok1 = true, ok2 = true;   // table entries in range (a pair's second: if covered)
    int krow;   // key row of this lane within its tile
    int vtok;   // first value token of this lane within its tile (non-wide)
    if constexpr (!kPair) {
      if (phys < 0 || phys >= num_blocks) return;
      kt = kpool + ((size_t)phys * Hkv + hkv) * (BS * D);
      vt = vpool + ((size_t)phys * Hkv + hkv) * (D * BS);
      krow = 0;
      vtok = 0;
    } else {
      phys2 = b + 1 < nblk ? uniform(bt[lb + 1]) : phys;
      ok1 = phys >= 0 && phys < num_blocks;
      ok2 = phys2 >= 0 && phys2 < num_blocks;
      if (!ok1) phys = 0;
      if (!ok2) phys2 = 0;
      const int64_t pk = n16 < 8 ? phys : phys2, pv = g4 < 2 ? phys : phys2;
      kt = kpool + ((size_t)pk * Hkv + hkv) * (BS * D);
      vt = vpool + ((size_t)pv * Hkv + hkv) * (D * BS);
      krow = -BS * (n16 >> 3);   // the lane's key rows sit BS*(n16/8) earlier in their tile
      vtok = -BS * (g4 >> 1);    // and its value tokens BS*(g4/2) earlier
    }
    u32x4 ka[SUB][KS];
    if constexpr (kFP8) {
      // One 16-byte load = 16 dimensions (64-byte piece c, quarter g4) of a
      // token: k-steps 2c and 2c+1.
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int c = 0; c < KS / 2; ++c) {
          const u32x4 raw = load16_stream(kt + (c * BS + token_of_row<GB>(sb, n16) + krow) * 64 + 16 * g4);
          const u32x2 a0 = widen4<E>(raw[0]), a1 = widen4<E>(raw[1]);
          const u32x2 a2 = widen4<E>(raw[2]), a3 = widen4<E>(raw[3]);
          ka[sb][2 * c] = u32x4{a0[0], a0[1], a1[0], a1[1]};
          ka[sb][2 * c + 1] = u32x4{a2[0], a2[1], a3[0], a3[1]};
        }
    } else {
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const TS *p = kt + (ks * BS + token_of_row<GB>(sb, n16) + krow) * 32 + 8 * g4;
          if constexpr (kApp) {
            if (token_of_row<GB>(sb, n16) == j) p = knew + 32 * ks;
          }
          ka[sb][ks] = load16_stream(p);
        }
    }
    // V^T operand: dimension row 16*nt + n16; tokens 8*g4 .. +8 (wide) or
    // 16*sb + 4*g4 .. +4 of sub-tile sb.
    u32x4 vw[kWide ? NT : 1];
    u32x2 va[kWide ? 1 : SUB][kWide ? 1 : NT];
    if constexpr (kWide) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (kFP8) {
          const u32x2 raw = load8_stream(vt + (16 * nt + n16) * BS + 8 * g4 + vtok);
          const u32x2 lo = widen4<PVE>(raw[0]), hi = widen4<PVE>(raw[1]);
          vw[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          vw[nt] = load16_stream(vt + (16 * nt + n16) * BS + 8 * g4 + vtok);
        }
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (kFP8)
            va[sb][nt] = widen4<PVE>(load4_stream(vt + (16 * nt + n16) * BS + 16 * sb + 4 * g4 + vtok));
          else
            va[sb][nt] = load8_stream(vt + (16 * nt + n16) * BS + 16 * sb + 4 * g4 + vtok);
        }
    }

    // The new token in cache format: over an 8-bit cache its key codes are
    // quantised here (a 16-bit cache loaded the key rows from the input
    // above); its value element is read here and patched into the V^T
    // operand just before the product.  The pool's slot is never read; the
    // reduce kernel that follows stores the rows into it.
    const bool has_new = kApp && j >= 0 && j < GB;
    const size_t row = ((size_t)s * Hkv + hkv) * D;
    uint32_t vnew[NT];   // cache bits of the new value, dimensions 16*nt + n16
    int vj = -1;         // its element in this lane's V^T operand (-1: none)
    int vsb = 0;         // ... and that operand's sub-tile (non-wide)
    if constexpr (kApp) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) vnew[nt] = 0u;
      if (has_new) {
        if constexpr (kFP8) {
#pragma unroll
          for (int sb = 0; sb < SUB; ++sb) {
            if (token_of_row<GB>(sb, n16) != j) continue;
#pragma unroll
            for (int c = 0; c < KS / 2; ++c) {
              const u32x4 codes = cache_piece<KV, E>(ap.k + row + 64 * c + 16 * g4, ap.k_scale);
              const u32x2 a0 = widen4<E>(codes[0]), a1 = widen4<E>(codes[1]);
              const u32x2 a2 = widen4<E>(codes[2]), a3 = widen4<E>(codes[3]);
              ka[sb][2 * c] = u32x4{a0[0], a0[1], a1[0], a1[1]};
              ka[sb][2 * c + 1] = u32x4{a2[0], a2[1], a3[0], a3[1]};
            }
          }
        }
        // This lane's value tokens: 8*g4 .. +8 (wide) or 16*sb + 4*g4 .. +4.
#pragma unroll
        for (int sb = 0; sb < (kWide ? 1 : SUB); ++sb) {
          const int t0 = kWide ? 8 * g4 : 16 * sb + 4 * g4;
          if (j >= t0 && j < t0 + (kWide ? 8 : 4)) {
            vj = j - t0;
            vsb = sb;
          }
        }
        if (vj >= 0) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) vnew[nt] = cache_elem<KV, E>(ap.v[row + 16 * nt + n16], ap.v_scale);
        }
      }
    }

    const int tbase = lb * BS;
    // Only the last block can end past the length, only the first start
    // before the window.
    const bool partial = tbase + GB > tok1 || tbase < lo;
    const unsigned span = (unsigned)(tok1 - lo);
    auto keep = [&](int t) { return (unsigned)(t - lo) < span; };
    f32x4 st[SUB];
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) x = Mfma<E>::qk(ka[sb][ks], qb[ks], x);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v = x[j] * scale_log2;
        if (partial && !keep(tbase + token_of_row<GB>(sb, 4 * g4 + j))) v = -INFINITY;
        x[j] = v;
      }
      st[sb] = x;
    }
    float mb = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) mb = fmaxf(mb, st[sb][j]);
    mb = xor_max<16, kWave>(mb);
    const float mnew = fmaxf(m, mb);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    // Softmax weights of this lane's tokens, packed as P^T operands (hi and,
    // for bf16, lo parts), in the token order of the lane's V^T rows.
    uint32_t ph[2 * SUB], plo[2 * SUB];
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < SUB; ++sb) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = fast_exp2(st[sb][j] - mnew);
        psum += p[j];
      }
      if constexpr (Mfma<PVE>::kSplitP) {
        split_bf16x2(p[0], p[1], ph[2 * sb], plo[2 * sb]);
        split_bf16x2(p[2], p[3], ph[2 * sb + 1], plo[2 * sb + 1]);
      } else {
        ph[2 * sb] = Mfma<PVE>::pack2(p[0], p[1]);
        ph[2 * sb + 1] = Mfma<PVE>::pack2(p[2], p[3]);
      }
    }
    l = l * alpha + psum;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] *= alpha;
    if (partial) {
      // Slots outside [lo, tok1) may hold anything (NaN included): zero their values.
      if constexpr (kWide) {
        const int t0 = tbase + 8 * g4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t mask = (keep(t0 + 2 * k) ? 0x0000ffffu : 0u) |
                                (keep(t0 + 2 * k + 1) ? 0xffff0000u : 0u);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) vw[nt][k] &= mask;
        }
      } else {
#pragma unroll
        for (int sb = 0; sb < SUB; ++sb) {
          const int t0 = tbase + 16 * sb + 4 * g4;
          const uint32_t keep01 = (keep(t0) ? 0x0000ffffu : 0u) | (keep(t0 + 1) ? 0xffff0000u : 0u);
          const uint32_t keep23 = (keep(t0 + 2) ? 0x0000ffffu : 0u) | (keep(t0 + 3) ? 0xffff0000u : 0u);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            va[sb][nt][0] &= keep01;
            va[sb][nt][1] &= keep23;
          }
        }
      }
    }
    if constexpr (kApp) {
      if (vj >= 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          // The element as the product reads it: an 8-bit code widened to E.
          uint32_t e = vnew[nt];
          if constexpr (kFP8) e = widen4<PVE>(e)[0] & 0xffffu;
          if constexpr (kWide) {
            vw[nt] = put_elem<2>(vw[nt], vj, e);
          } else {
#pragma unroll
            for (int sb = 0; sb < SUB; ++sb) {
              if (sb != vsb) continue;
              const u32x4 w4 = put_elem<2>(u32x4{va[sb][nt][0], va[sb][nt][1], 0u, 0u}, vj, e);
              va[sb][nt] = u32x2{w4[0], w4[1]};
            }
          }
        }
      }
    }
    if constexpr (kWide) {
      const u32x4 pw = {ph[0], ph[1], ph[2], ph[3]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        acc[nt] = Mfma<PVE>::qk(vw[nt], pw, acc[nt]);
        if constexpr (Mfma<PVE>::kSplitP) acc[nt] = Mfma<PVE>::qk(vw[nt], u32x4{plo[0], plo[1], plo[2], plo[3]}, acc[nt]);
      }
    } else {
#pragma unroll
      for (int sb = 0; sb < SUB; ++sb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[nt] = Mfma<PVE>::pv(va[sb][nt], u32x2{ph[2 * sb], ph[2 * sb + 1]}, acc[nt]);
          if constexpr (Mfma<PVE>::kSplitP)
            acc[nt] = Mfma<PVE>::pv(va[sb][nt], u32x2{plo[2 * sb], plo[2 * sb + 1]}, acc[nt]);
        }
    }
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
      asm volatile("" : "+v"(lane), "+v"(n16), "+v"(g4));
      step(blast, std::true_type{});
    }
  }

  // Denominator of head n16: sum over the 4 row groups.
  l = xor_sum<16, kWave>(l);
  if (g4 == 0) {
    lds_m[w * 16 + n16] = m;
    lds_l[w * 16 + n16] = l;
  }
  if (n16 < G) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc_at(w, n16, 16 * nt + 4 * g4 + j) = acc[nt][j];
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int e = idx - h * D;
    float M = lds_m[h];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) M = fmaxf(M, lds_m[k * 16 + h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      const float f = fast_exp2(lds_m[k * 16 + h] - M);
      num = fmaf(f, acc_at(k, h, e), num);
      den = fmaf(f, lds_l[k * 16 + h], den);
    }
    if constexpr (kFP8) num *= v_scale;
    const int hq = hkv * G + h;
    if (dest.base < 0) {
      store_out<E>(out, ((size_t)s * Hq + hq) * D + e, num / den, out_f32);
    } else {
      const size_t pi = (size_t)dest.base + (size_t)h * dest.stride;
      ws_acc[pi * D + e] = num;
      if (e == 0) {
        ws_ml[2 * pi] = M;
        ws_ml[2 * pi + 1] = den;
      }
    }
  }
}

// SCHED as for the wavefront kernel.  Dynamic LDS: [plan: S + 1 ints,
// padded to 16 bytes][merge buffers].
#ifndef PKV_MFMA_MIN_WAVES
#define PKV_MFMA_MIN_WAVES 4
#endif
#ifndef PKV_MFMA_MIN_WAVES_FP8
#define PKV_MFMA_MIN_WAVES_FP8 3
#endif
// The appending variants over 32-token steps (16- and 32-token blocks) give up
// one wave per SIMD rather than spill the new token's staging.
template <typename E, typename KV, int D, int BS, int SCHED, bool APPEND>
__global__ __launch_bounds__(kThreads, KV::kBytes == 1 ? PKV_MFMA_MIN_WAVES_FP8 : (APPEND && BS >= 16 ? 3 : PKV_MFMA_MIN_WAVES)) void decode_mfma_kernel(
    void *__restrict__ out, int out_f32, const uint16_t *__restrict__ q,
    const typename KV::storage *__restrict__ kpool, const typename KV::storage *__restrict__ vpool,
    const int32_t *__restrict__ block_tables, const int32_t *__restrict__ context_lens,
    int64_t num_blocks, int Hkv, int G, int S, int mbps, int cap, int window, float scale_log2,
    float v_scale, int part_tokens, int nparts, float *__restrict__ ws_ml,
    float *__restrict__ ws_acc, int *__restrict__ ws_hdr, Append<E> ap) {
  extern __shared__ __attribute__((aligned(16))) int dyn[];
  __shared__ int scan[16];
  int *plan = dyn;
  float *merge = (float *)(dyn + (SCHED == kSchedGrid ? 0 : ((S + 1 + 3) & ~3)));
  run_schedule<SCHED>(
      [&](int s, int hkv, int b0, int b1, Dest dest) {
        mfma_item<E, KV, D, BS, APPEND>(merge, s, hkv, b0, b1, dest, out, out_f32, q, kpool, vpool,
                                block_tables, context_lens, num_blocks, Hkv, G, mbps, cap, window,
                                scale_log2, v_scale, ws_ml, ws_acc, ap);
      },
      plan, scan, context_lens, S, cap, window, BS, Hkv, G, part_tokens, nparts, ws_hdr);
}

template <int D>
size_t merge_bytes(int G) {
  return sizeof(float) * (2 * kWaves * 16 + (size_t)kWaves * G * (D + 1));
}

template <typename E, typename KV, int D, int BS, bool APPEND>
void launch_ta(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  using T = typename KV::storage;
  const int G = a.Hq / c.H;
  const size_t merge = merge_bytes<D>(G);
  const size_t plan = sizeof(int) * (size_t)((a.S + 1 + 3) & ~3);
  const float sl = a.scale * kLog2e * c.k_scale;  // k_scale is 1 unless the cache is 8-bit
  auto go = [&](auto kern, dim3 grid, size_t dyn) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), dyn, stream, a.out, (int)a.out_f32,
                       (const uint16_t *)a.q, (const T *)c.k, (const T *)c.v, a.block_tables,
                       a.context_lens, c.num_blocks, c.H, G, a.S, a.max_blocks_per_seq, a.cap_tokens,
                       a.window,
                       sl, c.v_scale, a.partition_tokens, a.num_partitions, a.ws_ml, a.ws_acc,
                       a.ws_hdr,
                       Append<E>{(const uint16_t *)a.new_k, (const uint16_t *)a.new_v, c.k_scale,
                                 c.v_scale});
  };
  // Schedules as for the wavefront kernel.
#ifndef PKV_GRID_FACTOR
#define PKV_GRID_FACTOR 4
#endif
  if (a.flat) {
    go(decode_mfma_kernel<E, KV, D, BS, kSchedFlat, APPEND>, dim3(a.flat_grid), plan + merge);
  } else if (a.num_partitions > 1 && a.S <= kPlanMaxSeqs) {
    auto kern = decode_mfma_kernel<E, KV, D, BS, kSchedPlan, APPEND>;
    const int64_t cells = (int64_t)a.S * a.num_partitions * c.H;
    const int grid = (int)std::min<int64_t>(cells, PKV_GRID_FACTOR * (int64_t)resident_workgroups((const void *)kern, kThreads, plan + merge));
    go(kern, dim3(grid), plan + merge);
  } else {
    go(decode_mfma_kernel<E, KV, D, BS, kSchedGrid, APPEND>,
       dim3((unsigned)a.num_partitions, (unsigned)c.H, (unsigned)a.S), merge);
  }
}

// Appending calls run their own instantiations, so that plain decode keeps
// its register budget.
template <typename E, typename KV, int D, int BS>
void launch_t(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (a.new_k != nullptr) launch_ta<E, KV, D, BS, true>(c, a, stream);
  else launch_ta<E, KV, D, BS, false>(c, a, stream);
}

template <typename E, typename KV = E>
void launch_e(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (c.D == 64 && c.B == 8) launch_t<E, KV, 64, 8>(c, a, stream);
  else if (c.D == 128 && c.B == 8) launch_t<E, KV, 128, 8>(c, a, stream);
  else if (c.D == 64 && c.B == 16) launch_t<E, KV, 64, 16>(c, a, stream);
  else if (c.D == 64 && c.B == 32) launch_t<E, KV, 64, 32>(c, a, stream);
  else if (c.D == 128 && c.B == 16) launch_t<E, KV, 128, 16>(c, a, stream);
  else launch_t<E, KV, 128, 32>(c, a, stream);
}

template <typename E, typename KV, int D, int BS>
int flat_grid_t(int G, int S) {
  const size_t dyn = sizeof(int) * (size_t)((S + 1 + 3) & ~3) + merge_bytes<D>(G);
  return resident_workgroups((const void *)decode_mfma_kernel<E, KV, D, BS, kSchedFlat, false>, kThreads, dyn);
}

template <typename E, typename KV = E>
int flat_grid_e(const CacheDesc &c, int G, int S) {
  if (c.D == 64 && c.B == 8) return flat_grid_t<E, KV, 64, 8>(G, S);
  if (c.D == 128 && c.B == 8) return flat_grid_t<E, KV, 128, 8>(G, S);
  if (c.D == 64 && c.B == 16) return flat_grid_t<E, KV, 64, 16>(G, S);
  if (c.D == 64 && c.B == 32) return flat_grid_t<E, KV, 64, 32>(G, S);
  if (c.D == 128 && c.B == 16) return flat_grid_t<E, KV, 128, 16>(G, S);
  return flat_grid_t<E, KV, 128, 32>(G, S);
}

}  // namespace

// Over an 8-bit cache the matrix cores run in the model dtype.
hipError_t launch_decode_mfma(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream) {
  if (c.fp8()) {
    if (c.mdtype == 1) launch_e<F16, FP8>(c, a, stream);
    else launch_e<BF16, FP8>(c, a, stream);
  } else if (c.dtype == 1) {
    launch_e<F16>(c, a, stream);
  } else {
    launch_e<BF16>(c, a, stream);
  }
  return hipGetLastError();
}

int decode_mfma_flat_grid(const CacheDesc &c, int G, int S) {
  if (c.fp8()) return c.mdtype == 1 ? flat_grid_e<F16, FP8>(c, G, S) : flat_grid_e<BF16, FP8>(c, G, S);
  return c.dtype == 1 ? flat_grid_e<F16>(c, G, S) : flat_grid_e<BF16>(c, G, S);
}

}  // namespace pkv
