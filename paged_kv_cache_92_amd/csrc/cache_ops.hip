// Cache maintenance kernels: slot scatter, copy-on-write block copy, and the
// debug gather.  All are pure data movement (bit-exact, no conversion).
#include <type_traits>

#include "pkv_device.h"
#include "pkv_launch.h"

namespace pkv {
namespace {

// Slot scatter ("reshape_and_cache", [vLLM] PagedAttention, blog.secrett2633.cloud,
// section "PagedAttention 커널: 비연속 메모리 접근").  One workgroup moves kTok
// (16, or 64 for large batches: more loads in flight per thread) consecutive
// tokens of one head.  Key rows are copied 16 bytes at a time into
// the key tiles, whose rows are cut into 64-byte pieces ([D/X][B][X]).  Value rows are transposed through LDS so that
// lanes write consecutive tokens of one dimension: when the 16 slots are
// consecutive (a prompt chunk) each dimension row of a value tile receives
// contiguous runs.  Any slot mapping is handled (negative or out-of-range
// slots are skipped).  The 16-token instantiation (decode batches: one token
// per sequence, every value store a partial line) stores non-temporally:
// lines it left dirty in L2 were otherwise written back while the following
// decode streamed the pool (about 9 us more per 13B-shaped decode step).  The
// 64-token one (prompt chunks, whole lines) keeps plain stores, which measured
// faster there when the scatter follows a prefill kernel.
template <int EB, int D, int kTok>
__global__ __launch_bounds__(256) void scatter_kernel(const uint8_t *__restrict__ key,
                                                      const uint8_t *__restrict__ value,
                                                      const int64_t *__restrict__ slots,
                                                      uint8_t *__restrict__ kpool,
                                                      uint8_t *__restrict__ vpool, int64_t T, int H,
                                                      int B, int64_t nslots) {
  constexpr int VEC = 16 / EB;       // elements per 16-byte chunk
  constexpr int CH = D / VEC;        // chunks per (token, head) row
  constexpr int X = 64 / EB;         // elements per 64-byte key piece (4 chunks)
  constexpr int NC = D / X;          // key pieces per row
  using Elem = typename std::conditional<EB == 4, uint32_t, uint16_t>::type;
  __shared__ int64_t sslot[kTok];
  __shared__ Elem sv[D][kTok + 1];
  auto put = [](auto x, auto *p) {
    if constexpr (kTok == 16) __builtin_nontemporal_store(x, p);
    else *p = x;
  };

  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int tid = threadIdx.x;
  // The rows' loads do not depend on the slots: they are issued together with
  // the slot loads, and only the stores wait for the barrier.
  constexpr int NCH = kTok * CH;           // 16-byte chunks of the kTok rows
  constexpr int PER = (NCH + 255) / 256;   // per thread (256 threads)
  u32x4 kc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i;
    const int tt = c / CH, ch = c % CH;
    const int64_t t = t0 + tt;
    if (c >= NCH || t >= T) continue;
    const size_t src = ((size_t)t * H + h) * D + (size_t)ch * VEC;
    const u32x4 vc = load16(value + src * EB);
    kc[i] = load16(key + src * EB);
    // value chunk -> LDS, dimension-major
    if constexpr (EB == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) sv[ch * VEC + k][tt] = vc[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        sv[ch * VEC + 2 * k][tt] = (uint16_t)(vc[k] & 0xffffu);
        sv[ch * VEC + 2 * k + 1][tt] = (uint16_t)(vc[k] >> 16);
      }
    }
  }
  if (tid < kTok) {
    const int64_t t = t0 + tid;
    int64_t sl = t < T ? slots[t] : -1;
    if (sl >= nslots) sl = -1;
    sslot[tid] = sl;
  }
  __syncthreads();
  const int lgB = 31 - __builtin_clz(B);   // block_size is a power of two
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i;
    const int tt = c / CH, ch = c % CH;
    if (c >= NCH || t0 + tt >= T) continue;
    const int64_t sl = sslot[tt];
    if (sl < 0) continue;
    const int64_t blk = sl >> lgB;
    const int off = (int)(sl & (B - 1));
    put(kc[i], (u32x4 *)(kpool + ((((size_t)(blk * H + h) * NC + ch / 4) * B + off) * X + (ch % 4) * VEC) * EB));
  }
  Elem *vp = (Elem *)vpool;
  // 16-token groups: a wave writes 4 dimensions x 16 tokens.
  for (int c = tid; c < D * kTok; c += blockDim.x) {
    const int r = c % (D * 16);
    const int tt = c / (D * 16) * 16 + r % 16, e = r / 16;
    const int64_t sl = sslot[tt];
    if (sl < 0) continue;
    const int64_t blk = sl >> lgB;
    const int off = (int)(sl & (B - 1));
    put(sv[e][tt], &vp[((size_t)(blk * H + h) * D + e) * B + off]);
  }
}

// Slot scatter into an 8-bit cache: as scatter_kernel, but every element of
// the model-dtype key (value) row is stored as the E4M3 code of the fp32
// quotient x / k_scale (x / v_scale), one IEEE single division, rounded to
// nearest even and saturating (the cache-write call's kv_cache_dtype,
// k_scale and v_scale, [vLLM] PagedAttention, blog.secrett2633.cloud).  Key
// codes go out 8 at a time into the 64-byte pieces; value codes are
// transposed through LDS like the 16-bit values; stores are non-temporal, as
// there.
template <typename M, int D>
__global__ __launch_bounds__(256) void scatter_fp8_kernel(const uint16_t *__restrict__ key,
                                                          const uint16_t *__restrict__ value,
                                                          const int64_t *__restrict__ slots,
                                                          uint8_t *__restrict__ kpool,
                                                          uint8_t *__restrict__ vpool, int64_t T,
                                                          int H, int B, int64_t nslots,
                                                          float k_scale, float v_scale) {
  constexpr int kTok = 16;
  constexpr int CH = D / 8;          // 8-element groups per (token, head) row
  constexpr int NC = D / 64;         // 64-byte key pieces per row
  __shared__ int64_t sslot[kTok];
  __shared__ uint8_t sv[D][kTok + 4];

  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kTok;
  const int tid = threadIdx.x;
  auto quantise8 = [](const u32x4 &c, float scale) -> u32x2 {
    float f[8];
    unpack16<M>(c, f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i >> 2] |= f32_to_fp8_bits(__fdiv_rn(f[i], scale)) << (8 * (i & 3));
    return u32x2{w[0], w[1]};
  };
  // The rows' loads and their quantisation do not depend on the slots: only
  // the stores wait for the barrier.
  constexpr int NCH = kTok * CH;           // 8-element groups of the 16 rows
  constexpr int PER = (NCH + 255) / 256;   // per thread (256 threads)
  u32x2 kq[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i;
    const int tt = c / CH, g = c % CH;
    const int64_t t = t0 + tt;
    if (c >= NCH || t >= T) continue;
    const size_t src = ((size_t)t * H + h) * D + (size_t)g * 8;
    const u32x4 vraw = load16(value + src), kraw = load16(key + src);
    const u32x2 vq = quantise8(vraw, v_scale);
#pragma unroll
    for (int k = 0; k < 8; ++k) sv[g * 8 + k][tt] = (uint8_t)(vq[k >> 2] >> (8 * (k & 3)));
    kq[i] = quantise8(kraw, k_scale);
  }
  if (tid < kTok) {
    const int64_t t = t0 + tid;
    int64_t sl = t < T ? slots[t] : -1;
    if (sl >= nslots) sl = -1;
    sslot[tid] = sl;
  }
  __syncthreads();
  const int lgB = 31 - __builtin_clz(B);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + 256 * i;
    const int tt = c / CH, g = c % CH;
    if (c >= NCH || t0 + tt >= T) continue;
    const int64_t sl = sslot[tt];
    if (sl < 0) continue;
    const int64_t blk = sl >> lgB;
    const int off = (int)(sl & (B - 1));
    const int e0 = g * 8;
    __builtin_nontemporal_store(kq[i], (u32x2 *)(kpool + (((size_t)(blk * H + h) * NC + e0 / 64) * B + off) * 64 + e0 % 64));
  }
  for (int c = tid; c < D * kTok; c += blockDim.x) {
    const int tt = c % kTok, e = c / kTok;
    const int64_t sl = sslot[tt];
    if (sl < 0) continue;
    const int64_t blk = sl >> lgB;
    const int off = (int)(sl & (B - 1));
    __builtin_nontemporal_store(sv[e][tt], &vpool[((size_t)(blk * H + h) * D + e) * B + off]);
  }
}

// Copy-on-write block copy ("Sparse Computation and Memory Management...",
// pyy0715.github.io, section "Copy-on-Write"): both tiles of every head of
// block src go to block dst.  grid.y walks the pairs, grid.x strides over the
// 16-byte chunks of one block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t *__restrict__ kpool,
                                                          uint8_t *__restrict__ vpool,
                                                          const int32_t *__restrict__ pairs,
                                                          int64_t nblocks, int64_t chunks) {
  const int64_t p = blockIdx.y;
  const int32_t src = pairs[2 * p], dst = pairs[2 * p + 1];
  if (src < 0 || src >= nblocks || dst < 0 || dst >= nblocks) return;
  const size_t tile = (size_t)chunks * 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    const u32x4 a = load16(kpool + src * tile + i * 16);
    const u32x4 b = load16(vpool + src * tile + i * 16);
    *(u32x4 *)(kpool + dst * tile + i * 16) = a;
    *(u32x4 *)(vpool + dst * tile + i * 16) = b;
  }
}

// Debug gather with the attention kernels' address arithmetic: contiguous,
// token-major K and V of every sequence.  One thread per 16-byte output chunk.
template <int EB>
__global__ __launch_bounds__(256) void gather_kernel(const uint8_t *__restrict__ kpool,
                                                     const uint8_t *__restrict__ vpool,
                                                     uint8_t *__restrict__ kout,
                                                     uint8_t *__restrict__ vout,
                                                     const int32_t *__restrict__ bt, int mbps,
                                                     const int32_t *__restrict__ ctx,
                                                     const int32_t *__restrict__ cu, int64_t nblocks,
                                                     int H, int B, int D, int max_len) {
  constexpr int VEC = 16 / EB;
  constexpr int X = 64 / EB;
  const int chunks = D / VEC;
  const int NC = D / X;
  const int s = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)max_len * H * chunks) return;
  const int c = (int)(idx % chunks);
  const int h = (int)((idx / chunks) % H);
  const int j = (int)(idx / ((int64_t)chunks * H));
  const int L = min(ctx[s], mbps * B);
  if (j >= L) return;
  const int32_t blk = bt[(size_t)s * mbps + j / B];
  if (blk < 0 || blk >= nblocks) return;
  const int off = j % B;
  const size_t dst = (((size_t)cu[s] + j) * H + h) * D + (size_t)c * VEC;
  *(u32x4 *)(kout + dst * EB) = load16(
      kpool + ((((size_t)(blk * (int64_t)H + h) * NC + c / 4) * B + off) * X + (c % 4) * VEC) * EB);
  const size_t vrow = ((size_t)(blk * (int64_t)H + h) * D + (size_t)c * VEC) * B + off;
  u32x4 packed;
  if constexpr (EB == 1) {
    const uint8_t *vp = vpool;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) w |= (uint32_t)vp[vrow + (size_t)(4 * i + k) * B] << (8 * k);
      packed[i] = w;
    }
  } else if constexpr (EB == 4) {
    const uint32_t *vp = (const uint32_t *)vpool;
#pragma unroll
    for (int i = 0; i < 4; ++i) packed[i] = vp[vrow + (size_t)i * B];
  } else {
    const uint16_t *vp = (const uint16_t *)vpool;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      packed[i] = (uint32_t)vp[vrow + (size_t)(2 * i) * B] |
                  ((uint32_t)vp[vrow + (size_t)(2 * i + 1) * B] << 16);
  }
  *(u32x4 *)(vout + dst * EB) = packed;
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheDesc &c, const void *key, const void *value,
                                    const int64_t *slots, int64_t T, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 15) / 16), (unsigned)c.H);
  const int64_t nslots = c.num_blocks * c.B;
  // Large batches of 16-bit rows (prompt chunks) take 64 tokens per workgroup.
  const bool wide = T >= 2048 && c.elt_bytes() == 2;
  const dim3 grid64((unsigned)((T + 63) / 64), (unsigned)c.H);
  auto go = [&](auto kern16, auto kern64) {
    if (wide)
      hipLaunchKernelGGL(kern64, grid64, dim3(256), 0, stream, (const uint8_t *)key,
                         (const uint8_t *)value, slots, (uint8_t *)c.k, (uint8_t *)c.v, T, c.H, c.B,
                         nslots);
    else
      hipLaunchKernelGGL(kern16, grid, dim3(256), 0, stream, (const uint8_t *)key, (const uint8_t *)value,
                       slots, (uint8_t *)c.k, (uint8_t *)c.v, T, c.H, c.B, nslots);
  };
  auto go8 = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, (const uint16_t *)key, (const uint16_t *)value,
                       slots, (uint8_t *)c.k, (uint8_t *)c.v, T, c.H, c.B, nslots, c.k_scale, c.v_scale);
  };
  if (c.fp8()) {
    if (c.mdtype == 1) {
      if (c.D == 64) go8(scatter_fp8_kernel<F16, 64>);
      else go8(scatter_fp8_kernel<F16, 128>);
    } else {
      if (c.D == 64) go8(scatter_fp8_kernel<BF16, 64>);
      else go8(scatter_fp8_kernel<BF16, 128>);
    }
  } else if (c.elt_bytes() == 4) {
    // fp32 rows: 16 tokens already fill a thread's loads (prefill takes no fp32 cache).
    if (c.D == 64) go(scatter_kernel<4, 64, 16>, scatter_kernel<4, 64, 16>);
    else go(scatter_kernel<4, 128, 16>, scatter_kernel<4, 128, 16>);
  } else {
    if (c.D == 64) go(scatter_kernel<2, 64, 16>, scatter_kernel<2, 64, 64>);
    else go(scatter_kernel<2, 128, 16>, scatter_kernel<2, 128, 64>);
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CacheDesc &c, const int32_t *pairs, int64_t n,
                              hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t chunks = (int64_t)c.H * c.B * c.D * c.elt_bytes() / 16;
  const int64_t gx = (chunks + 255) / 256;
  const dim3 grid((unsigned)(gx < 64 ? gx : 64), (unsigned)n);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, (uint8_t *)c.k,
                     (uint8_t *)c.v, pairs, c.num_blocks, chunks);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const CacheDesc &c, void *k_out, void *v_out, const int32_t *bt,
                            int mbps, const int32_t *ctx, const int32_t *cu, int S,
                            int max_context_len, hipStream_t stream) {
  const int EB = c.elt_bytes();
  const int64_t work = (int64_t)max_context_len * c.H * (c.D * EB / 16);
  const dim3 grid((unsigned)((work + 255) / 256), (unsigned)S);
  if (EB == 1)
    hipLaunchKernelGGL(gather_kernel<1>, grid, dim3(256), 0, stream, (const uint8_t *)c.k,
                       (const uint8_t *)c.v, (uint8_t *)k_out, (uint8_t *)v_out, bt, mbps, ctx, cu,
                       c.num_blocks, c.H, c.B, c.D, max_context_len);
  else if (EB == 4)
    hipLaunchKernelGGL(gather_kernel<4>, grid, dim3(256), 0, stream, (const uint8_t *)c.k,
                       (const uint8_t *)c.v, (uint8_t *)k_out, (uint8_t *)v_out, bt, mbps, ctx, cu,
                       c.num_blocks, c.H, c.B, c.D, max_context_len);
  else
    hipLaunchKernelGGL(gather_kernel<2>, grid, dim3(256), 0, stream, (const uint8_t *)c.k,
                       (const uint8_t *)c.v, (uint8_t *)k_out, (uint8_t *)v_out, bt, mbps, ctx, cu,
                       c.num_blocks, c.H, c.B, c.D, max_context_len);
  return hipGetLastError();
}

}  // namespace pkv
