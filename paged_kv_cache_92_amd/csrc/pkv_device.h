// Device-side helpers shared by the pkv HIP kernels (gfx950, wave64).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Element tags: storage is float for fp32 and uint16_t bits for fp16/bf16.
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
};
struct F16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};
// 8-bit cache entries: OCP FP8 E4M3 codes (bias 7, 3 mantissa bits,
// S.1111.111 NaN, no infinities, largest magnitude 448).
struct FP8 {
  using storage = uint8_t;
  static constexpr int kBytes = 1;
};

// ---- scalar conversions ---------------------------------------------------
// Bit casts take their source by value: clang has been seen to read element 0
// when __builtin_bit_cast is applied directly to an ext-vector element.
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);  // round to nearest even
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}

template <typename E>
__device__ __forceinline__ float lo_to_f32(uint32_t w);
template <typename E>
__device__ __forceinline__ float hi_to_f32(uint32_t w);
template <>
__device__ __forceinline__ float lo_to_f32<F16>(uint32_t w) { return f16_bits_to_f32(w & 0xffffu); }
template <>
__device__ __forceinline__ float hi_to_f32<F16>(uint32_t w) { return f16_bits_to_f32(w >> 16); }
template <>
__device__ __forceinline__ float lo_to_f32<BF16>(uint32_t w) { return bf16_bits_to_f32(w & 0xffffu); }
template <>
__device__ __forceinline__ float hi_to_f32<BF16>(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Unpack a 16-byte chunk into VEC floats (VEC = 4 for fp32, 8 for 16-bit).
template <typename E>
__device__ __forceinline__ void unpack16(const u32x4 &c, float *out);
template <>
__device__ __forceinline__ void unpack16<F32>(const u32x4 &c, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = c[i];
    out[i] = as_f32(u);
  }
}
template <>
__device__ __forceinline__ void unpack16<F16>(const u32x4 &c, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = lo_to_f32<F16>(c[i]);
    out[2 * i + 1] = hi_to_f32<F16>(c[i]);
  }
}
template <>
__device__ __forceinline__ void unpack16<BF16>(const u32x4 &c, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = lo_to_f32<BF16>(c[i]);
    out[2 * i + 1] = hi_to_f32<BF16>(c[i]);
  }
}

template <>
__device__ __forceinline__ void unpack16<FP8>(const u32x4 &c, float *out) {
  // 16 codes; v_cvt_pk_f32_fp8 turns the low or high byte pair of a word into
  // two floats (exact: every E4M3 value is an fp32 value).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)c[i], true);
    out[4 * i] = lo[0];
    out[4 * i + 1] = lo[1];
    out[4 * i + 2] = hi[0];
    out[4 * i + 3] = hi[1];
  }
}

// fp32 -> E4M3 code: nearest, ties to the even code; magnitudes of 448 and
// beyond (infinities included) saturate to 448, NaN stays NaN.  Works on the
// fp32 bit fields: normal results keep the top 3 of the 23 mantissa bits
// with the dropped 20 rounded to nearest even (a carry out of the mantissa
// steps the exponent field, which the code's layout makes one add);
// results below 2^-6 sit on the subnormal grid of 2^-9.
__device__ __forceinline__ uint32_t f32_to_fp8_bits(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return sign | 0x7fu;        // NaN
  if (a >= 0x43e00000u) return sign | 0x7eu;       // >= 448 (and inf): saturate
  if (a < 0x3c800000u)                             // < 2^-6: multiples of 2^-9
    return sign | (uint32_t)__builtin_rintf(__builtin_bit_cast(float, a) * 512.f);
  const uint32_t e = (a >> 23) - 127 + 7;          // biased E4M3 exponent, 1..15
  const uint32_t top = (a >> 20) & 7u;             // kept mantissa bits
  const uint32_t rest = a & 0xfffffu;              // dropped mantissa bits
  const uint32_t up = rest > 0x80000u || (rest == 0x80000u && (top & 1u));
  return sign | (((e << 3) | top) + up);
}

// q.k over one 16-byte chunk, accumulated in fp32.  For 16-bit inputs each
// pair product is exact in fp32 (v_dot2_f32_f16 / v_dot2_f32_bf16); q is the
// matching chunk of the query in the same packed format.
template <typename E>
__device__ __forceinline__ float dot16(const u32x4 &k, const u32x4 &q);
template <>
__device__ __forceinline__ float dot16<F32>(const u32x4 &k, const u32x4 &q) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ku = k[i], qu = q[i];
    d = fmaf(as_f32(qu), as_f32(ku), d);
  }
  return d;
}
// q.k over four fp32 elements in fp64: the products are exact, one rounding
// per addition at 53 bits.
__device__ __forceinline__ double dot16_f64(const u32x4 &k, const u32x4 &q) {
  double d = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ku = k[i], qu = q[i];
    d = __builtin_fma((double)as_f32(qu), (double)as_f32(ku), d);
  }
  return d;
}
template <>
__device__ __forceinline__ float dot16<F16>(const u32x4 &k, const u32x4 &q) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ku = k[i], qu = q[i];
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qu), __builtin_bit_cast(f16x2, ku), d, false);
  }
  return d;
}
template <>
__device__ __forceinline__ float dot16<BF16>(const u32x4 &k, const u32x4 &q) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ku = k[i], qu = q[i];
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, qu), __builtin_bit_cast(bf16x2, ku),
                                        d, false);
  }
  return d;
}


// Two floats -> packed bf16 pair (round to nearest even), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));  // RNE
}

// Two bf16 values (one 32-bit word) re-encoded as two fp16 values.  Exact for
// |x| in [2^-17, 65504]; smaller magnitudes round on the fp16 subnormal grid
// (absolute error <= 2^-25).  A bf16 value of magnitude >= 65536 has no fp16
// encoding: `mag` keeps the running maximum of the magnitude bits (sign
// cleared, compared as integers, which orders non-negative floats) for
// bf16_beyond_f16 to check.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, u16x2 &mag) {
  mag = __builtin_elementwise_max(mag, __builtin_bit_cast(u16x2, w & 0x7fff7fffu));
  return pack_f16x2(as_f32(w << 16), as_f32(w & 0xffff0000u));
}
__device__ __forceinline__ bool bf16_beyond_f16(u16x2 mag) {
  return (mag[0] > mag[1] ? mag[0] : mag[1]) >= 0x4780u;  // 0x4780 = 65536 in bf16
}

// p = hi + lo with hi and lo in bf16: hi = RNE(p), lo = RNE(p - hi), so the
// pair carries 16 significant bits (|p - hi - lo| <= 2^-17 |p|).  Works on
// two values at once; hi and lo come back packed as the MFMA operands want.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t &hi, uint32_t &lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - as_f32(hi << 16), b - as_f32(hi & 0xffff0000u));
}

template <typename E>
__device__ __forceinline__ void store_elem(typename E::storage *p, float x);
template <>
__device__ __forceinline__ void store_elem<F32>(float *p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_elem<F16>(uint16_t *p, float x) { *p = f32_to_f16_bits(x); }
template <>
__device__ __forceinline__ void store_elem<BF16>(uint16_t *p, float x) { *p = f32_to_bf16_bits(x); }

// Attention outputs go out either in the cache dtype (rounded once, to
// nearest even, from fp32) or as the fp32 value itself.
template <typename E>
__device__ __forceinline__ void store_out(void *out, size_t idx, float x, bool out_f32) {
  if (out_f32)
    ((float *)out)[idx] = x;
  else
    store_elem<E>((typename E::storage *)out + idx, x);
}

// ---- wave reductions ---------------------------------------------------------
// DPP row controls (within rows of 16 lanes): quad_perm [1,0,3,2] and
// [2,3,0,1] swap neighbours at distance 1 and 2; half-row mirror pairs lane i
// with 7-i of its 8-lane half; row mirror pairs i with 15-i.  Applied in that
// order, each step adds a disjoint group, so after k steps every lane holds
// the sum over its aligned group of 2^k lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xf, 0xf, false));
}

// The same lane permutation applied to both halves of a double.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, (uint64_t)lo | ((uint64_t)hi << 32));
}

// Sum of a double over each aligned quad of lanes.
__device__ __forceinline__ double quad_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);
  return x + dpp_f64<0x4E>(x);
}

template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(WIDTH == 1 || WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16 ||
                    WIDTH == 32 || WIDTH == 64,
                "power-of-two group");
  if constexpr (WIDTH >= 2) x += dpp_f32<0xB1>(x);
  if constexpr (WIDTH >= 4) x += dpp_f32<0x4E>(x);
  if constexpr (WIDTH >= 8) x += dpp_f32<0x141>(x);
  if constexpr (WIDTH >= 16) x += dpp_f32<0x140>(x);
  if constexpr (WIDTH >= 32) x += __shfl_xor(x, 16);
  if constexpr (WIDTH >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Wave-wide max of a value that is already uniform within each quad: the
// half-row mirror then pairs whole quads, the row mirror whole half-rows.
__device__ __forceinline__ float quad_uniform_max(float x) {
  x = fmaxf(x, dpp_f32<0x141>(x));
  x = fmaxf(x, dpp_f32<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

// Max over lanes that differ only in bits [log2(FROM), log2(TO)) of the lane id.
template <int FROM, int TO>
__device__ __forceinline__ float xor_max(float x) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
template <int FROM, int TO>
__device__ __forceinline__ float xor_sum(float x) {
#pragma unroll
  for (int m = FROM; m < TO; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ u32x4 load16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x2 load8(const void *p) { return *(const u32x2 *)p; }
// Streaming loads for data read once per launch (the decode kernels' key and
// value tiles): the non-temporal hint keeps them from displacing reusable lines.
__device__ __forceinline__ u32x4 load16_stream(const void *p) {
  return __builtin_nontemporal_load((const u32x4 *)p);
}
__device__ __forceinline__ u32x2 load8_stream(const void *p) {
  return __builtin_nontemporal_load((const u32x2 *)p);
}
__device__ __forceinline__ uint32_t load4_stream(const void *p) {
  return __builtin_nontemporal_load((const uint32_t *)p);
}

// ---- the new token of an appending decode call ----------------------------
// The new token's key and value rows (model dtype Q, [seq][kv head][D]) and,
// for an 8-bit cache, the scales its codes are quantised with; read by the
// appending instantiations of the decode kernels.
template <typename Q>
struct Append {
  const typename Q::storage *k;
  const typename Q::storage *v;
  float k_scale, v_scale;
};

// 16 bytes of cache-format key data from the input row at src: the same bits
// for a 16/32-bit cache; for an 8-bit cache the E4M3 codes of 16 inputs
// (x / scale, one fp32 division each, as the scatter stores them).
template <typename E, typename Q>
__device__ __forceinline__ u32x4 cache_piece(const typename Q::storage *src, float scale) {
  if constexpr (E::kBytes == 1) {
    float f[16];
    unpack16<Q>(*(const u32x4 *)src, f);
    unpack16<Q>(*(const u32x4 *)(src + 8), f + 8);
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 2] |= f32_to_fp8_bits(__fdiv_rn(f[i], scale)) << (8 * (i & 3));
    return w;
  } else {
    return *(const u32x4 *)src;
  }
}

// One cache-format element (its bits, in the low E::kBytes bytes) of input x.
template <typename E, typename Q>
__device__ __forceinline__ uint32_t cache_elem(typename Q::storage x, float scale) {
  if constexpr (E::kBytes == 1) {
    float f;
    if constexpr (std::is_same<Q, F16>::value) f = f16_bits_to_f32(x);
    else f = bf16_bits_to_f32(x);
    return f32_to_fp8_bits(__fdiv_rn(f, scale));
  } else if constexpr (E::kBytes == 2) {
    return (uint32_t)x;
  } else {
    return __builtin_bit_cast(uint32_t, x);
  }
}

// The value of one cache element from its bits (low E::kBytes bytes), as
// unpack16 decodes it.
template <typename E>
__device__ __forceinline__ float elem_value(uint32_t bits) {
  float f[16];
  unpack16<E>(u32x4{bits, 0u, 0u, 0u}, f);
  return f[0];
}

// Stores the low EB bytes of bits at p, non-temporally (a cache element
// written for a later attention call, which reads it back from HBM).
template <int EB>
__device__ __forceinline__ void store_bits(void *p, uint32_t bits) {
  if constexpr (EB == 1) __builtin_nontemporal_store((uint8_t)bits, (uint8_t *)p);
  else if constexpr (EB == 2) __builtin_nontemporal_store((uint16_t)bits, (uint16_t *)p);
  else __builtin_nontemporal_store(bits, (uint32_t *)p);
}

// v with element e (of EB bytes each) replaced by the low EB bytes of bits.
template <int EB>
__device__ __forceinline__ u32x4 put_elem(u32x4 v, int e, uint32_t bits) {
  const int word = e * EB / 4, sh = (e * EB % 4) * 8;
  const uint32_t mask = (EB == 4 ? 0xffffffffu : ((1u << (8 * EB)) - 1u)) << sh;
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (w == word) v[w] = (v[w] & ~mask) | ((bits << sh) & mask);
  return v;
}

}  // namespace pkv
