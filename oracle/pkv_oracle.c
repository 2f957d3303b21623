/*
 * CPU oracle for the paged KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  The GPU library
 * never links, includes or calls it, and nothing here is shared with the
 * HIP kernels: this file decodes the raw fp16/bf16/fp32 bits itself, does
 * all arithmetic in fp64, and follows the definitions on the pages step by
 * step, with no blocking, fusion or reordering.
 *
 * Pages cited (titles as published):
 *   [T]  "'안녕하세요 반갑습니다'로 배우는 vLLM — KV Cache와 PagedAttention 완전 해부"
 *        (hrletsgo.me)
 *   [W]  "[vLLM] PagedAttention: OS 페이징 기법으로 KV 캐시를 관리하는 방법"
 *        (blog.secrett2633.cloud)
 *   [R]  "vLLM: LLM 서빙 메모리 최적화의 교과서" (velog.io/@doogunwo)
 *   [S]  "Sparse Computation and Memory Management for Efficient LLM Inference"
 *        (pyy0715.github.io)
 *
 * Pool layout (an interface contract of the library, restated here; the
 * pages fix only "fixed-size blocks of B token slots", [T] step 5):
 *   K pool  [num_blocks][H][d/X][B][X], X = 64 bytes / element size (64 E4M3,
 *           32 fp16/bf16, 16 fp32 values): a key row is cut into 64-byte
 *           pieces and the B pieces of one dimension range are adjacent;
 *           element (blk,h,off,e) at (((blk*H+h)*(d/X)+e/X)*B+off)*X+e%X
 *   V pool  [num_blocks][H][d][B]  element (blk,h,off,e) at ((blk*H+h)*d+e)*B+off
 *   slot s  = blk*B + off          (token slot off inside physical block blk)
 *
 * Every entry point returns 0 on success and a negative code on a contract
 * violation (out-of-range slot or block id, duplicate slot, bad sizes); on
 * error nothing is guaranteed about partially written outputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8 = 3 /* OCP FP8 E4M3, 8-bit cache only */ };

enum {
  ORC_OK = 0,
  ORC_ERR_ARG = -1,      /* bad sizes / dtype / null pointer */
  ORC_ERR_RANGE = -2,    /* slot, block id or position out of range */
  ORC_ERR_DUP = -3,      /* duplicate destination (no defined winner) */
  ORC_ERR_NOMEM = -4
};

static size_t elt_size(int dtype) {
  return dtype == ORC_F32 ? 4u : dtype == ORC_FP8 ? 1u : 2u;
}

/* IEEE-754 binary16 -> fp64, decoded from the bit fields. */
static double f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int mant = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)mant, -24); /* subnormal: mant * 2^-24 */
  } else if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + mant), expo - 25); /* (1.mant) * 2^(expo-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 is the top half of an IEEE binary32. */
static double bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/*
 * 8-bit float cache entries.  [W] section "PagedAttention 커널: 비연속 메모리
 * 접근": write_to_paged_cache passes kv_cache_dtype, k_scale and v_scale on
 * to reshape_and_cache.  Reading taken: for an 8-bit cache the stored code of
 * a key element x is the OCP FP8 E4M3 encoding of the fp32 quotient x /
 * k_scale (values with v_scale), and a read gives code * scale.
 *
 * E4M3: sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent field 0
 * holds subnormals m * 2^-9; the all-ones pattern S.1111.111 is NaN and there
 * are no infinities, so the largest magnitude is 1.110b * 2^8 = 448.
 */
static double fp8_to_double(uint8_t b) {
  int sign = b >> 7, expo = (b >> 3) & 15, mant = b & 7;
  double v;
  if (expo == 15 && mant == 7) v = NAN;
  else if (expo == 0) v = ldexp((double)mant, -9);
  else v = ldexp((double)(8 + mant), expo - 10); /* (1.mant) * 2^(expo-7) */
  return sign ? -v : v;
}

/* fp32 -> E4M3: round to nearest, ties to the even code; magnitudes of 448
 * and beyond (infinities included) saturate to +-448; NaN stays NaN. */
static uint8_t fp8_from_float(float x) {
  uint8_t sign = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return sign | 0x7F;
  double a = fabs((double)x);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) return sign | (uint8_t)rint(a * 512.0); /* subnormal grid 2^-9; 8 = 2^-6 */
  int e2;
  frexp(a, &e2);
  int E = e2 - 1;                      /* a in [2^E, 2^(E+1)) */
  int n = (int)rint(ldexp(a, 3 - E));  /* 8..16: significand in units of 2^(E-3) */
  if (n == 16) {
    E += 1;
    n = 8;
  }
  return sign | (uint8_t)(((E + 7) << 3) | (n - 8));
}

static double load_elt(const void *base, size_t idx, int dtype) {
  if (dtype == ORC_F32) return (double)((const float *)base)[idx];
  if (dtype == ORC_FP8) return fp8_to_double(((const uint8_t *)base)[idx]);
  uint16_t bits = ((const uint16_t *)base)[idx];
  return dtype == ORC_F16 ? f16_to_double(bits) : bf16_to_double(bits);
}

static void copy_elt(void *dst, size_t di, const void *src, size_t si, int dtype) {
  if (dtype == ORC_F32)
    ((uint32_t *)dst)[di] = ((const uint32_t *)src)[si];
  else if (dtype == ORC_FP8)
    ((uint8_t *)dst)[di] = ((const uint8_t *)src)[si];
  else
    ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
}

/* One element of a scatter: a bit copy, or for an 8-bit cache the code of
 * the fp32 quotient (the input value is exact in fp32; the division is one
 * IEEE single-precision division). */
static void store_elt(void *dst, size_t di, int kv_dtype, const void *src, size_t si, int in_dtype,
                      float scale) {
  if (kv_dtype != ORC_FP8) {
    copy_elt(dst, di, src, si, kv_dtype);
    return;
  }
  float x = (float)load_elt(src, si, in_dtype);
  ((uint8_t *)dst)[di] = fp8_from_float(x / scale);
}

static size_t k_index(int64_t blk, int h, int off, int e, int H, int B, int d, int dtype) {
  const int X = 64 / (int)elt_size(dtype);
  return (((size_t)(blk * H + h) * (size_t)(d / X) + (size_t)(e / X)) * B + off) * X + e % X;
}

static size_t v_index(int64_t blk, int h, int off, int e, int H, int B, int d) {
  return ((size_t)(blk * H + h) * d + e) * B + off;
}

static int check_geometry(int dtype, int64_t num_blocks, int H, int B, int d) {
  if (dtype != ORC_F32 && dtype != ORC_F16 && dtype != ORC_BF16 && dtype != ORC_FP8) return ORC_ERR_ARG;
  if (num_blocks <= 0 || H <= 0 || B <= 0 || d <= 0) return ORC_ERR_ARG;
  if (d % (64 / (int)elt_size(dtype)) != 0) return ORC_ERR_ARG; /* whole 64-byte key pieces */
  return ORC_OK;
}

/*
 * Slot scatter ("reshape_and_cache").  [W] section "PagedAttention 커널:
 * 비연속 메모리 접근": write_to_paged_cache hands each new token's key and
 * value, plus the slot that slot_mapping names for it, to reshape_and_cache,
 * which stores them in the paged cache.  [T] step 5 / step 6: a token lives in
 * slot `off` of physical block `blk` (the 6-token request fills slots 0..5 of
 * block 42 and decode writes the next token to slot 6), read here as
 * slot = blk*B + off.  A negative slot marks a padding token: nothing is
 * written.  key/value are [T][H][d], token-major.
 */
static int scatter(void *k_pool, void *v_pool, int kv_dtype, int in_dtype, float k_scale,
                   float v_scale, int64_t num_blocks, int H, int B, int d, const void *key,
                   const void *value, const int64_t *slots, int64_t T) {
  int rc = check_geometry(kv_dtype, num_blocks, H, B, d);
  if (rc) return rc;
  if (kv_dtype == ORC_FP8) {
    if (in_dtype != ORC_F16 && in_dtype != ORC_BF16) return ORC_ERR_ARG;
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || isinf(k_scale) || isinf(v_scale)) return ORC_ERR_ARG;
  } else if (in_dtype != kv_dtype) {
    return ORC_ERR_ARG;
  }
  if (T < 0 || (T > 0 && (!key || !value || !slots || !k_pool || !v_pool))) return ORC_ERR_ARG;
  int64_t nslots = num_blocks * B;
  /* Duplicate destinations have no defined winner: refuse them. */
  unsigned char *seen = calloc((size_t)nslots, 1);
  if (!seen) return ORC_ERR_NOMEM;
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0) continue;
    if (s >= nslots) { free(seen); return ORC_ERR_RANGE; }
    if (seen[s]) { free(seen); return ORC_ERR_DUP; }
    seen[s] = 1;
  }
  free(seen);
  for (int64_t t = 0; t < T; ++t) {
    int64_t s = slots[t];
    if (s < 0) continue;
    int64_t blk = s / B;
    int off = (int)(s % B);
    for (int h = 0; h < H; ++h) {
      for (int e = 0; e < d; ++e) {
        size_t src = ((size_t)t * H + h) * d + e;
        store_elt(k_pool, k_index(blk, h, off, e, H, B, d, kv_dtype), kv_dtype, key, src, in_dtype, k_scale);
        store_elt(v_pool, v_index(blk, h, off, e, H, B, d), kv_dtype, value, src, in_dtype, v_scale);
      }
    }
  }
  return ORC_OK;
}

int oracle_reshape_and_cache(void *k_pool, void *v_pool, int dtype, int64_t num_blocks,
                             int H, int B, int d, const void *key, const void *value,
                             const int64_t *slots, int64_t T) {
  return scatter(k_pool, v_pool, dtype, dtype, 1.f, 1.f, num_blocks, H, B, d, key, value, slots, T);
}

/* The same into an 8-bit cache: key/value rows in in_dtype (f16 or bf16). */
int oracle_reshape_and_cache_fp8(void *k_pool, void *v_pool, int in_dtype, float k_scale,
                                 float v_scale, int64_t num_blocks, int H, int B, int d,
                                 const void *key, const void *value, const int64_t *slots,
                                 int64_t T) {
  return scatter(k_pool, v_pool, ORC_FP8, in_dtype, k_scale, v_scale, num_blocks, H, B, d, key,
                 value, slots, T);
}

/*
 * Block copy for copy-on-write.  [S] section "Copy-on-Write": before a
 * sequence writes into a block whose reference count exceeds one, the block
 * is copied whole to a freshly allocated block (fused_block_copy(phys,
 * new_phys)) and the sequence's table entry is repointed.  [T] step 9 states
 * the same for shared prompt blocks.  src_dst is [n][2] = (src, dst); every
 * dst must be distinct and must not also appear as a src, so the copies are
 * independent of order.
 */
int oracle_copy_blocks(void *k_pool, void *v_pool, int dtype, int64_t num_blocks, int H, int B,
                       int d, const int32_t *src_dst, int64_t n) {
  int rc = check_geometry(dtype, num_blocks, H, B, d);
  if (rc) return rc;
  if (n < 0 || (n > 0 && !src_dst)) return ORC_ERR_ARG;
  unsigned char *role = calloc((size_t)num_blocks, 1); /* bit0: src, bit1: dst */
  if (!role) return ORC_ERR_NOMEM;
  for (int64_t i = 0; i < n; ++i) {
    int32_t s = src_dst[2 * i], t = src_dst[2 * i + 1];
    if (s < 0 || s >= num_blocks || t < 0 || t >= num_blocks) { free(role); return ORC_ERR_RANGE; }
    role[s] |= 1;
  }
  for (int64_t i = 0; i < n; ++i) {
    int32_t t = src_dst[2 * i + 1];
    if (role[t] & 3) { free(role); return ORC_ERR_DUP; }
    role[t] |= 2;
  }
  free(role);
  size_t tile = (size_t)H * B * d * elt_size(dtype);
  for (int64_t i = 0; i < n; ++i) {
    size_t s = (size_t)src_dst[2 * i], t = (size_t)src_dst[2 * i + 1];
    memcpy((char *)k_pool + t * tile, (const char *)k_pool + s * tile, tile);
    memcpy((char *)v_pool + t * tile, (const char *)v_pool + s * tile, tile);
  }
  return ORC_OK;
}

/* Logical position j of a sequence -> physical block through its table.
 * [T] step 5: the block table maps logical block i to a physical block;
 * [R] section "02. Idea: PagedAttention": logical blocks look contiguous to
 * the model while the physical blocks are scattered. */
static int lookup(const int32_t *bt_row, int j, int B, int64_t num_blocks, int64_t *blk, int *off) {
  int32_t b = bt_row[j / B];
  if (b < 0 || b >= num_blocks) return ORC_ERR_RANGE;
  *blk = b;
  *off = j % B;
  return ORC_OK;
}

/*
 * Reassembly of each sequence's contiguous K/V, bit for bit, in the cache
 * dtype: k_out/v_out are [sum_s ctx[s]][H][d], sequences back to back.
 */
int oracle_gather_kv(const void *k_pool, const void *v_pool, int dtype, int64_t num_blocks, int H,
                     int B, int d, const int32_t *block_tables, int max_blocks_per_seq,
                     const int32_t *context_lens, int S, void *k_out, void *v_out) {
  int rc = check_geometry(dtype, num_blocks, H, B, d);
  if (rc) return rc;
  size_t row = 0;
  for (int s = 0; s < S; ++s) {
    int L = context_lens[s];
    if (L < 0 || L > max_blocks_per_seq * B) return ORC_ERR_RANGE;
    const int32_t *bt = block_tables + (size_t)s * max_blocks_per_seq;
    for (int j = 0; j < L; ++j, ++row) {
      int64_t blk;
      int off;
      if ((rc = lookup(bt, j, B, num_blocks, &blk, &off))) return rc;
      for (int h = 0; h < H; ++h)
        for (int e = 0; e < d; ++e) {
          size_t dst = (row * H + h) * d + e;
          copy_elt(k_out, dst, k_pool, k_index(blk, h, off, e, H, B, d, dtype), dtype);
          copy_elt(v_out, dst, v_pool, v_index(blk, h, off, e, H, B, d), dtype);
        }
    }
  }
  return ORC_OK;
}

/* fp64 reassembly of positions [j0, n) of one sequence into Kc/Vc, which are
 * indexed by absolute position: [n][H][d] (rows before j0 untouched; the
 * table entries of their blocks are not read).  Entries of an 8-bit cache
 * read as code * scale (exact in fp64). */
static int reassemble(const void *k_pool, const void *v_pool, int dtype, double k_scale,
                      double v_scale, int64_t num_blocks, int H, int B, int d,
                      const int32_t *bt_row, int j0, int n, double *Kc, double *Vc) {
  const double ks = dtype == ORC_FP8 ? k_scale : 1.0, vs = dtype == ORC_FP8 ? v_scale : 1.0;
  for (int j = j0; j < n; ++j) {
    int64_t blk;
    int off;
    int rc = lookup(bt_row, j, B, num_blocks, &blk, &off);
    if (rc) return rc;
    for (int h = 0; h < H; ++h)
      for (int e = 0; e < d; ++e) {
        size_t dst = ((size_t)j * H + h) * d + e;
        Kc[dst] = ks * load_elt(k_pool, k_index(blk, h, off, e, H, B, d, dtype), dtype);
        Vc[dst] = vs * load_elt(v_pool, v_index(blk, h, off, e, H, B, d), dtype);
      }
  }
  return ORC_OK;
}

/*
 * Textbook causal attention for one query vector against contiguous K/V.
 * [R] section "01. Problem Definition": a_ij = softmax_j(q_i.k_j / sqrt(d))
 * over j <= i (the current position included) and o_i = sum_j a_ij v_j;
 * [T] "부록": softmax(Q K^T / sqrt(d)) V, the weights summing to one.  The
 * caller passes the scale (1/sqrt(d) as an fp32 value); keys 0..p are used.
 * The maximum is subtracted before exponentiation, which leaves the softmax
 * unchanged in exact arithmetic.  Grouped heads (GQA, [S] section "The
 * Hidden Waste of KV Cache": 32 query heads share 8 KV heads) read KV head
 * hkv = hq / (Hq / Hkv).  Keys lo..p are used: lo = 0, or the first position
 * of a sliding window.
 */
static void attend_one(const double *q, int lo, int p, const double *Kc, const double *Vc, int Hkv,
                       int hkv, int d, double scale, double *z, double *o) {
  double m = -INFINITY;
  for (int j = lo; j <= p; ++j) {
    const double *k = Kc + ((size_t)j * Hkv + hkv) * d;
    double dot = 0.0;
    for (int e = 0; e < d; ++e) dot += q[e] * k[e];
    z[j] = scale * dot;
    if (z[j] > m) m = z[j];
  }
  double Z = 0.0;
  for (int j = lo; j <= p; ++j) {
    z[j] = exp(z[j] - m);
    Z += z[j];
  }
  for (int e = 0; e < d; ++e) o[e] = 0.0;
  for (int j = lo; j <= p; ++j) {
    const double *v = Vc + ((size_t)j * Hkv + hkv) * d;
    double w = z[j] / Z;
    for (int e = 0; e < d; ++e) o[e] += w * v[e];
  }
}

/*
 * Attention for a list of query rows.  Row r belongs to sequence row_seq[r]
 * and sits at absolute position row_pos[r]; it attends to cached positions
 * 0..row_pos[r] of that sequence, or, with window > 0, to the window's
 * positions max(0, row_pos[r] - window + 1)..row_pos[r]: [W] section "블록
 * 할당: allocate_slots" releases the blocks that fall out of a sliding
 * window, read here as the W most recent positions, the row's own included.  q is [n][Hq][d] in q_dtype (the cache dtype, or f16/bf16 over an 8-bit cache), out
 * is [n][Hq][d] fp64.  The sequence's K/V are first reassembled into
 * contiguous fp64 arrays through its block table, then each head runs the
 * textbook formula above; consecutive rows of one sequence reuse one
 * reassembly.
 */
int oracle_paged_attention_rows(const void *k_pool, const void *v_pool, int dtype, int q_dtype,
                                double k_scale, double v_scale,
                                int64_t num_blocks, int Hkv, int B, int d, const void *q, int Hq,
                                const int32_t *block_tables, int max_blocks_per_seq,
                                const int32_t *context_lens, int S, const int32_t *row_seq,
                                const int32_t *row_pos, int64_t n, int window, float scale,
                                double *out) {
  int rc = check_geometry(dtype, num_blocks, Hkv, B, d);
  if (rc) return rc;
  if (Hq <= 0 || Hq % Hkv != 0 || n < 0 || S <= 0 || window < 0) return ORC_ERR_ARG;
  if (dtype == ORC_FP8 ? (q_dtype != ORC_F16 && q_dtype != ORC_BF16) : q_dtype != dtype) return ORC_ERR_ARG;
  int G = Hq / Hkv;
  int cap = max_blocks_per_seq * B;
  double *Kc = malloc(sizeof(double) * (size_t)cap * Hkv * d);
  double *Vc = malloc(sizeof(double) * (size_t)cap * Hkv * d);
  double *z = malloc(sizeof(double) * (size_t)cap);
  double *qv = malloc(sizeof(double) * (size_t)d);
  if (!Kc || !Vc || !z || !qv) { rc = ORC_ERR_NOMEM; goto done; }
  int cur_seq = -1, cur_lo = 0;
  for (int64_t r = 0; r < n; ++r) {
    int s = row_seq[r], p = row_pos[r];
    if (s < 0 || s >= S || p < 0 || p >= context_lens[s] || context_lens[s] > cap) {
      rc = ORC_ERR_RANGE;
      goto done;
    }
    int lo = window > 0 && p - window + 1 > 0 ? p - window + 1 : 0;
    if (s != cur_seq || lo < cur_lo) {
      const int32_t *bt = block_tables + (size_t)s * max_blocks_per_seq;
      if ((rc = reassemble(k_pool, v_pool, dtype, k_scale, v_scale, num_blocks, Hkv, B, d, bt, lo,
                           context_lens[s], Kc, Vc)))
        goto done;
      cur_seq = s;
      cur_lo = lo;
    }
    for (int hq = 0; hq < Hq; ++hq) {
      for (int e = 0; e < d; ++e) qv[e] = load_elt(q, ((size_t)r * Hq + hq) * d + e, q_dtype);
      attend_one(qv, lo, p, Kc, Vc, Hkv, hq / G, d, (double)scale, z,
                 out + ((size_t)r * Hq + hq) * d);
    }
  }
  rc = ORC_OK;
done:
  free(Kc);
  free(Vc);
  free(z);
  free(qv);
  return rc;
}

/*
 * Decode step: one new query per sequence at position ctx[s]-1, attending to
 * all ctx[s] cached tokens (the new token's K/V already scattered, so the
 * query sees itself as the equation's j <= i requires).  [T] step 6: decode
 * reads the whole cache every step; [R] eq. (4) is the block-wise form of
 * the same result.  With window > 0 only the last `window` positions are
 * attended (see oracle_paged_attention_rows).  q and out are [S][Hq][d].
 */
int oracle_paged_decode(const void *k_pool, const void *v_pool, int dtype, int q_dtype,
                        double k_scale, double v_scale, int64_t num_blocks,
                        int Hkv, int B, int d, const void *q, int Hq, const int32_t *block_tables,
                        int max_blocks_per_seq, const int32_t *context_lens, int S, int window,
                        float scale, double *out) {
  if (S <= 0) return ORC_ERR_ARG;
  int32_t *rs = malloc(sizeof(int32_t) * (size_t)S);
  int32_t *rp = malloc(sizeof(int32_t) * (size_t)S);
  if (!rs || !rp) { free(rs); free(rp); return ORC_ERR_NOMEM; }
  for (int s = 0; s < S; ++s) {
    rs[s] = s;
    rp[s] = context_lens[s] - 1;
  }
  int rc = oracle_paged_attention_rows(k_pool, v_pool, dtype, q_dtype, k_scale, v_scale, num_blocks,
                                       Hkv, B, d, q, Hq, block_tables, max_blocks_per_seq,
                                       context_lens, S, rs, rp, S, window, scale, out);
  free(rs);
  free(rp);
  return rc;
}

/*
 * Chunked prefill: sequence s contributes query rows
 * query_start_loc[s] .. query_start_loc[s+1]-1, the last chunk of its
 * ctx[s] tokens, so row i of the chunk sits at absolute position
 * ctx[s] - qlen_s + i and attends causally to positions 0..that position
 * (history plus the chunk's own earlier tokens).  [S] section
 * "Prefill-Decode Disaggregation": a long prompt is processed in chunks;
 * [T] step 6: prefill handles all prompt tokens at once.  q and out are
 * [total rows][Hq][d].
 */
int oracle_paged_prefill(const void *k_pool, const void *v_pool, int dtype, int q_dtype,
                         double k_scale, double v_scale, int64_t num_blocks,
                         int Hkv, int B, int d, const void *q, int Hq,
                         const int32_t *query_start_loc, const int32_t *context_lens,
                         const int32_t *block_tables, int max_blocks_per_seq, int S, float scale,
                         double *out) {
  if (S <= 0 || query_start_loc[0] != 0) return ORC_ERR_ARG;
  int64_t n = query_start_loc[S];
  for (int s = 0; s < S; ++s) {
    int ql = query_start_loc[s + 1] - query_start_loc[s];
    if (ql < 0 || ql > context_lens[s]) return ORC_ERR_RANGE;
  }
  int32_t *rs = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  int32_t *rp = malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  if (!rs || !rp) { free(rs); free(rp); return ORC_ERR_NOMEM; }
  for (int s = 0; s < S; ++s) {
    int ql = query_start_loc[s + 1] - query_start_loc[s];
    int hist = context_lens[s] - ql;
    for (int i = 0; i < ql; ++i) {
      rs[query_start_loc[s] + i] = s;
      rp[query_start_loc[s] + i] = hist + i;
    }
  }
  int rc = oracle_paged_attention_rows(k_pool, v_pool, dtype, q_dtype, k_scale, v_scale, num_blocks,
                                       Hkv, B, d, q, Hq, block_tables, max_blocks_per_seq,
                                       context_lens, S, rs, rp, n, 0, scale, out);
  free(rs);
  free(rp);
  return rc;
}

/* Bit decoders exported so that tests can pin them against known encodings. */
double oracle_f16_to_double(uint16_t h) { return f16_to_double(h); }
double oracle_bf16_to_double(uint16_t b) { return bf16_to_double(b); }
double oracle_fp8_to_double(uint8_t b) { return fp8_to_double(b); }
uint8_t oracle_fp8_from_float(float x) { return fp8_from_float(x); }
