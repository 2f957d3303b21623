// Causal chunked prefill over the paged cache on the matrix cores (f16/bf16).
//
// A chunk of a long prompt is processed as one step ("Sparse Computation and
// Memory Management for Efficient LLM Inference", pyy0715.github.io, section
// "Prefill-Decode Disaggregation"); all of its rows are known at once, so
// attention is a matrix-matrix product ("vLLM: LLM 서빙 메모리 최적화의 교과서",
// velog.io, section 01, prompt phase), causal over j <= i.
//
// Workgroup = 8 waves = one (sequence, query head, 256-row query tile); wave
// w owns 32 rows.  The key/value positions 0..last row's position are walked
// in 64-token tiles gathered through the block table into LDS (the next
// tile's global loads are in flight while the current one is computed); each
// tile is two 32-token halves:
//
//   S^T (32 tokens x 32 rows) = K (32 x D) . Q^T (D x 32)     D/16 k-steps per half
//   O^T (D x 32 rows)        += V^T (D x 32) . P^T (32 x 32)   2 k-steps per half
//
// with 32x32x16 MFMAs.  The key rows are fed to the first product in a
// permuted order chosen so that each lane's 16 result rows are, per 16-token
// k-step of the second product, 8 consecutive tokens: the B operand P^T is
// then built from the lane's own registers and the A operand V^T is one
// 16-byte LDS read from the dimension-major value tile.  Online softmax per
// row, log2 domain.  Tiles entirely in a wave's future are skipped.
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
constexpr int kWaves = PKV_PREFILL_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 32 * kWaves;  // query rows per workgroup
constexpr int kKT = 64;           // key/value tokens per tile
constexpr int kVPad = 8;          // LDS row padding (elements) against bank conflicts

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

// bf16 inputs run P.V on the fp16 matrix cores: value tiles are re-encoded to
// fp16 when staged in LDS (exact over fp16's range) and the softmax weights
// pack to fp16 (11 significant bits, against 8 in bf16, so no hi + lo split).
// A tile holding a value outside fp16's range is flagged while staged and
// takes the exact bf16 route instead (values read from HBM, weights split).
#ifndef PKV_PREFILL_CONV_V
#define PKV_PREFILL_CONV_V 1
#endif

// Operand reads issued a whole product ahead (1) or next to each product (0).
#ifndef PKV_PREFILL_EARLY_LDS
#define PKV_PREFILL_EARLY_LDS 1
#endif

// Row i of a 32-token score product (i = 8a + 4h + b) holds token perm(i) of
// its half-tile.
__device__ __forceinline__ int perm_row(int i) {
  const int a = i >> 3, h = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
}

// Lazy rescaling: a row keeps its reference maximum until a new score beats it
// by more than 2^kRescaleLog2; weights stay <= 2^kRescaleLog2 meanwhile (no
// overflow in fp32 or bf16), and the final o = acc / l is unaffected.
constexpr float kRescaleLog2 = 8.f;

template <typename E, int D, int BS>
__global__ __launch_bounds__(kThreads, 512 / kThreads) void prefill_kernel(
    void *__restrict__ out, int out_f32, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ kpool, const uint16_t *__restrict__ vpool,
    const int32_t *__restrict__ query_start_loc, const int32_t *__restrict__ context_lens,
    const int32_t *__restrict__ block_tables, int64_t num_blocks, int Hkv, int Hq, int mbps,
    int staged, int nqt, float scale_log2) {
  // staged: block-table entries per sequence that fit the dynamic LDS
  // (enough for max_context_len); positions beyond them are never walked.
  constexpr int KS = D / 16;          // k-steps of the score product
  constexpr int DT = D / 32;          // 32-dimension tiles of the output
  constexpr int KCH = kKT * D / 8;    // 16-byte chunks of a key tile
  constexpr int VCH = D * kKT / 8;    // 16-byte chunks of a value tile
  constexpr int KPT = KCH / kThreads; // key chunks per thread
  constexpr int VPT = VCH / kThreads; // value chunks per thread
  static_assert(KCH % kThreads == 0 && VCH % kThreads == 0, "tile must split evenly over the workgroup");
  constexpr int KROW = D + kVPad;     // LDS key row (elements)
  constexpr int VROW = kKT + kVPad;   // LDS value row (elements)

  // Work item: XCD-aware order keeps the tiles of one (sequence, head) on one
  // XCD (consecutive block ids go round-robin over the 8 XCDs), longest tile first.
  const int nwork = gridDim.x;
  int wid = blockIdx.x;
  if ((nwork & 7) == 0) wid = (wid & 7) * (nwork >> 3) + (wid >> 3);
  const int qt = nqt - 1 - wid % nqt;
  const int hq = (wid / nqt) % Hq;
  const int s = wid / (nqt * Hq);

  const int qs = query_start_loc[s];
  const int qlen = query_start_loc[s + 1] - qs;
  if (qt * kQT >= qlen) return;
  const int ctx = min(context_lens[s], staged * BS);
  const int hist = ctx - qlen;
  if (hist < 0) return;
  const int hkv = hq / (Hq / Hkv);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int w = uniform(tid >> 6);
  const int j32 = lane & 31;  // query column of this lane
  const int h = lane >> 5;    // k-half / row group

  // Two LDS tile buffers: tile t+1 is stored while tile t is computed.
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKT * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][D * VROW];
  extern __shared__ int sBT[];  // block ids of the positions this workgroup reads

  const int wrow0 = qt * kQT + 32 * w;                  // first chunk row of this wave
  const int myrow = wrow0 + j32;
  const int qpos = hist + min(myrow, qlen - 1);         // position of this lane's query
  const int wave_min_pos = hist + min(wrow0, qlen - 1);
  const int wave_max_pos = hist + min(wrow0 + 31, qlen - 1);
  const int wg_max_pos = hist + min(qt * kQT + kQT - 1, qlen - 1);
  const int ntiles = (wg_max_pos + kKT) / kKT;

  // Stage the block table once; tile loads then look block ids up in LDS.
  __shared__ int sOvf;  // a staged value lay outside fp16's range
  if (tid == 0) sOvf = 0;
  {
    const int32_t *bt = block_tables + (size_t)s * mbps;
    const int nbt = min((ntiles * kKT + BS - 1) / BS, staged);
    for (int i = tid; i < nbt; i += kThreads) {
      const int32_t b = bt[i];
      sBT[i] = (b >= 0 && b < num_blocks) ? b : -1;
    }
  }

  // Q^T operand: query column j32, dimensions 16*ks + 8*h .. +8 (zero past the chunk).
  u32x4 qb[KS];
  {
    const bool valid = myrow < qlen;
    const uint16_t *qrow = q + ((size_t)(qs + (valid ? myrow : 0)) * Hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = valid ? load16(qrow + 16 * ks + 8 * h) : u32x4{0, 0, 0, 0};
  }
  __syncthreads();

  // Global -> register staging of one tile.  Thread tid moves key pieces
  // (token (tid/4) % 64, bytes 16*(tid%4).. of 64-byte pieces
  // tid/256 + KPR*i of the row, so a wave reads 16 tokens x 64 bytes
  // contiguously) and value chunks (dimension tid/8 + VDR*i, tokens
  // 8*(tid%8)..+8); a block id comes from the staged table.
  constexpr int KX = 32;              // elements per 64-byte key piece
  constexpr int KPR = kThreads / 256; // key pieces per chunk round
  constexpr int VDR = kThreads / 8;   // value dimensions per chunk round
  static_assert(KPT * KPR == D / KX, "whole key pieces per chunk round");
  const int ktok = (tid >> 2) & (kKT - 1), ksub = tid & 3, kpc = tid >> 8;
  auto load_tile = [&](int t, u32x4 (&kreg)[KPT], u32x4 (&vreg)[VPT]) {
    const int t0 = t * kKT;
    const bool full = t0 + kKT <= ctx;
    {
      const int pos = t0 + ktok;
      // Positions past the context read a harmless in-pool address; their
      // scores are masked.  An invalid block id (a broken caller contract)
      // reads block 0 instead of faulting.
      const int blk = (full || pos < ctx) ? max(sBT[pos / BS], 0) : 0;
      const uint16_t *kb = kpool + ((size_t)blk * Hkv + hkv) * D * BS + (pos % BS) * KX + 8 * ksub;
#pragma unroll
      for (int i = 0; i < KPT; ++i) kreg[i] = load16(kb + (size_t)(kpc + KPR * i) * BS * KX);
    }
    {
      const int pos = t0 + 8 * (tid % 8);
      const int blk = (full || pos < ctx) ? max(sBT[pos / BS], 0) : 0;
      const uint16_t *vblk = vpool + ((size_t)blk * Hkv + hkv) * D * BS + pos % BS;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const int e = tid / 8 + VDR * i;
        u32x4 x = load16(vblk + (size_t)e * BS);
        if (!full && pos + 8 > ctx) {
          // Slots past the context may hold anything: zero them.
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t keep = (pos + 2 * k < ctx ? 0x0000ffffu : 0u) |
                                  (pos + 2 * k + 1 < ctx ? 0xffff0000u : 0u);
            x[k] &= keep;
          }
        }
        vreg[i] = x;
      }
    }
  };
  // Staging of one tile into LDS buffer buf.  CONV: values re-encoded to fp16;
  // returns (through sOvf) whether any of them lay outside fp16's range.
  auto store_tile = [&](auto conv, int buf, const u32x4 (&kreg)[KPT], const u32x4 (&vreg)[VPT]) {
    constexpr bool CONV = decltype(conv)::value;
#pragma unroll
    for (int i = 0; i < KPT; ++i) *(u32x4 *)&sK[buf][ktok * KROW + KX * (kpc + KPR * i) + 8 * ksub] = kreg[i];
    u16x2 mag = {0, 0};
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      u32x4 x = vreg[i];
      if constexpr (CONV) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = bf16x2_to_f16x2(x[k], mag);
      }
      *(u32x4 *)&sV[buf][(tid / 8 + VDR * i) * VROW + 8 * (tid % 8)] = x;
    }
    if (CONV && bf16_beyond_f16(mag)) sOvf = 1;
  };

  float m, l;  // running max (scaled log2 units) and this lane's denominator share
  f32x16 acc[DT];
  const f32x16 zero16 = {};
  const int krow = perm_row(j32);  // key row (within a 32-token half) this lane feeds

  // The whole walk over the key/value tiles.  CONV (bf16 only): P.V on the
  // fp16 matrix cores; the walk reports whether every staged value fit fp16.
  auto attend = [&](auto conv) -> bool {
    constexpr bool CONV = decltype(conv)::value;
    using PV = typename std::conditional<CONV, Mfma32<F16>, Mfma32<E>>::type;
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
    // One tile's scores, softmax update and P.V: tile t, staged in LDS buffer cur.
    auto tile = [&](int t, int cur) {
      constexpr int HALVES = kKT / 32;
      f32x16 st[HALVES];  // raw scores q.k
      const uint16_t *krp = &sK[cur][krow * KROW + 8 * h];
#if PKV_PREFILL_EARLY_LDS
      // All key operands of the tile are read before the first product, so
      // the LDS latency is paid once rather than before every product; the
      // fence keeps the compiler from sinking the reads back.
      u32x4 kop[HALVES][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)
          kop[hf][ks] = *(const u32x4 *)(krp + 32 * hf * KROW + 16 * ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf) st[hf] = Mfma32<E>::mma(kop[hf][0], qb[0], zero16);
#pragma unroll
      for (int ks = 1; ks < KS; ++ks)
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)  // independent chains back to back
          st[hf] = Mfma32<E>::mma(kop[hf][ks], qb[ks], st[hf]);
      // The value operands of the whole tile, in flight during the softmax.
      u32x4 vop[2 * HALVES][DT];
#pragma unroll
      for (int c = 0; c < 2 * HALVES; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          vop[c][dt] = *(const u32x4 *)&sV[cur][(32 * dt + j32) * VROW + 16 * c + 8 * h];
      __builtin_amdgcn_sched_barrier(0);
#else
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf)
        st[hf] = Mfma32<E>::mma(*(const u32x4 *)(krp + 32 * hf * KROW), qb[0], zero16);
#pragma unroll
      for (int ks = 1; ks < KS; ++ks)
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)  // independent chains back to back
          st[hf] = Mfma32<E>::mma(*(const u32x4 *)(krp + 32 * hf * KROW + 16 * ks), qb[ks], st[hf]);
#endif
      // Item 4a+b of half hf is tile token 32*hf + perm(8a+4h+b).  Only a
      // tile that crosses this wave's diagonal needs the causal mask (the
      // hint keeps the compiler from turning the branch into selects that
      // every tile would pay for).
      if (__builtin_expect(t * kKT + kKT - 1 > wave_min_pos, 0)) {
#pragma unroll
        for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const int pos = t * kKT + 32 * hf + 16 * (a >> 1) + 8 * h + 4 * (a & 1) + b;
              if (pos > qpos) st[hf][4 * a + b] = -INFINITY;
            }
      }
      float mraw = -INFINITY;
#pragma unroll
      for (int hf = 0; hf < HALVES; ++hf)
#pragma unroll
        for (int i = 0; i < 16; ++i) mraw = fmaxf(mraw, st[hf][i]);
      mraw = fmaxf(mraw, __shfl_xor(mraw, 32));
      const float mb = mraw * scale_log2;  // scale > 0: the max commutes with scaling
      if (__any(mb > m + kRescaleLog2)) {
        const float mnew = fmaxf(m, mb);
        const float alpha = fast_exp2(m - mnew);  // 1 for rows that keep their reference
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      }
      float psum = 0.f;
#pragma unroll
      for (int c = 0; c < 2 * HALVES; ++c) {
        // This lane's 8 weights of k-step c (16 tokens) against the value
        // rows 32dt + j32, tokens 16c + 8h .. +8 of the staged tile.
        const int hf = c >> 1, c2 = c & 1;
        float p[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          p[k] = fast_exp2(fmaf(st[hf][8 * c2 + k], scale_log2, -m));
          psum += p[k];
        }
        u32x4 pb, pl;
        if constexpr (PV::kSplitP) {
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) split_bf16x2(p[2 * k], p[2 * k + 1], hi[k], lo[k]);
          pb = u32x4{hi[0], hi[1], hi[2], hi[3]};
          pl = u32x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
          pb = u32x4{PV::pack2(p[0], p[1]), PV::pack2(p[2], p[3]), PV::pack2(p[4], p[5]),
                     PV::pack2(p[6], p[7])};
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#if PKV_PREFILL_EARLY_LDS
          const u32x4 a = vop[c][dt];
#else
          const u32x4 a = *(const u32x4 *)&sV[cur][(32 * dt + j32) * VROW + 16 * c + 8 * h];
#endif
          acc[dt] = PV::mma(a, pb, acc[dt]);
          if constexpr (PV::kSplitP) acc[dt] = PV::mma(a, pl, acc[dt]);
        }
      }
      l += psum;
    };
    u32x4 kreg[KPT], vreg[VPT];
    load_tile(0, kreg, vreg);
    store_tile(conv, 0, kreg, vreg);
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int cur = t & 1;
      if (t + 1 < ntiles) load_tile(t + 1, kreg, vreg);  // in flight while this tile is computed
      if (t * kKT <= wave_max_pos) tile(t, cur);  // else entirely in this wave's future
      // The other buffer was last read in the previous iteration, before the
      // barrier that ended it; the barrier below publishes tile t+1.
      if (t + 1 < ntiles) store_tile(conv, cur ^ 1, kreg, vreg);
      __syncthreads();
    }
    return !CONV || uniform(sOvf) == 0;
  };

  // bf16: the fp16 route first; if any staged value lay outside fp16's range
  // (a flag every thread reads after the walk's last barrier), the whole walk
  // is redone on the exact bf16 route.  Nothing was written meanwhile.
  constexpr bool kConvV = std::is_same<E, BF16>::value && PKV_PREFILL_CONV_V;
  bool done = false;
  if constexpr (kConvV) done = attend(std::true_type{});
  if (!done) attend(std::false_type{});

  // Lanes l and l^32 hold the two row halves of the same query column.
  const float ltot = l + __shfl_xor(l, 32);
  if (myrow < qlen) {
    const float inv = 1.f / ltot;
    const size_t orow = ((size_t)(qs + myrow) * Hq + hq) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int dim = 32 * dt + 8 * a + 4 * h;
        const float o0 = acc[dt][4 * a] * inv, o1 = acc[dt][4 * a + 1] * inv;
        const float o2 = acc[dt][4 * a + 2] * inv, o3 = acc[dt][4 * a + 3] * inv;
        if (out_f32) {
          *(f32x4 *)((float *)out + orow + dim) = f32x4{o0, o1, o2, o3};
        } else {
          *(u32x2 *)((uint16_t *)out + orow + dim) =
              u32x2{Mfma32<E>::pack2(o0, o1), Mfma32<E>::pack2(o2, o3)};
        }
      }
  }
}

// Block-table entries staged per workgroup: the table's width, or fewer when
// max_context_len needs fewer.
int staged_entries(const PrefillArgs &a, int B) {
  return std::min(a.max_blocks_per_seq, (a.max_context_len + B - 1) / B);
}

template <typename E, int D, int BS>
size_t lds_bytes_t(const PrefillArgs &a) {
  // The kernel's static LDS is a property of its code: asked once.
  static const size_t static_bytes = [] {
    hipFuncAttributes fa{};
    return hipFuncGetAttributes(&fa, (const void *)prefill_kernel<E, D, BS>) == hipSuccess
               ? fa.sharedSizeBytes
               : SIZE_MAX;
  }();
  if (static_bytes == SIZE_MAX) return SIZE_MAX;
  return static_bytes + sizeof(int) * (size_t)staged_entries(a, BS);
}

template <typename E>
size_t lds_bytes_e(const CacheDesc &c, const PrefillArgs &a) {
  if (c.D == 64 && c.B == 8) return lds_bytes_t<E, 64, 8>(a);
  if (c.D == 128 && c.B == 8) return lds_bytes_t<E, 128, 8>(a);
  if (c.D == 64 && c.B == 16) return lds_bytes_t<E, 64, 16>(a);
  if (c.D == 64 && c.B == 32) return lds_bytes_t<E, 64, 32>(a);
  if (c.D == 128 && c.B == 16) return lds_bytes_t<E, 128, 16>(a);
  return lds_bytes_t<E, 128, 32>(a);
}

template <typename E, int D, int BS>
void launch_t(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  const int nqt = (a.max_query_len + kQT - 1) / kQT;
  const int64_t nwork = (int64_t)a.S * a.Hq * nqt;
  const int staged = staged_entries(a, BS);
  const size_t lds = sizeof(int) * (size_t)staged;   // staged block table
  hipLaunchKernelGGL((prefill_kernel<E, D, BS>), dim3((unsigned)nwork), dim3(kThreads), lds, stream,
                     a.out, (int)a.out_f32, (const uint16_t *)a.q, (const uint16_t *)c.k,
                     (const uint16_t *)c.v, a.query_start_loc, a.context_lens, a.block_tables,
                     c.num_blocks, c.H, a.Hq, a.max_blocks_per_seq, staged, nqt, a.scale * kLog2e);
}

template <typename E>
void launch_e(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  if (c.D == 64 && c.B == 8) launch_t<E, 64, 8>(c, a, stream);
  else if (c.D == 128 && c.B == 8) launch_t<E, 128, 8>(c, a, stream);
  else if (c.D == 64 && c.B == 16) launch_t<E, 64, 16>(c, a, stream);
  else if (c.D == 64 && c.B == 32) launch_t<E, 64, 32>(c, a, stream);
  else if (c.D == 128 && c.B == 16) launch_t<E, 128, 16>(c, a, stream);
  else launch_t<E, 128, 32>(c, a, stream);
}

}  // namespace

size_t prefill_lds_bytes(const CacheDesc &c, const PrefillArgs &a) {
  return c.dtype == 1 ? lds_bytes_e<F16>(c, a) : lds_bytes_e<BF16>(c, a);
}

hipError_t launch_prefill(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream) {
  if (a.max_query_len == 0 || a.S == 0) return hipSuccess;
  if (c.dtype == 1) launch_e<F16>(c, a, stream);
  else launch_e<BF16>(c, a, stream);
  return hipGetLastError();
}

}  // namespace pkv
