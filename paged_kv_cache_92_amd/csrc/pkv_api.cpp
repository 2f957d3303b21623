// C ABI of libpkv.so: host-side argument validation and kernel dispatch.
// The contract of every entry point is documented in include/pkv.h.
#include "pkv.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <unordered_set>
#include <vector>

#include "pkv_launch.h"

namespace {

thread_local char g_err[512] = "";

pkv_status fail(pkv_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

pkv_status ok() {
  g_err[0] = '\0';
  return PKV_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

pkv_status check_cache(const pkv_cache *c, pkv::CacheDesc *d) {
  if (!c) return fail(PKV_ERR_INVALID, "cache descriptor is NULL");
  if (!c->k_pool || !c->v_pool) return fail(PKV_ERR_INVALID, "k_pool/v_pool is NULL");
  if (!aligned16(c->k_pool) || !aligned16(c->v_pool))
    return fail(PKV_ERR_INVALID, "k_pool/v_pool must be 16-byte aligned");
  if (c->num_blocks <= 0) return fail(PKV_ERR_INVALID, "num_blocks must be > 0");
  if (c->num_kv_heads <= 0) return fail(PKV_ERR_INVALID, "num_kv_heads must be > 0");
  if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d unsupported (8, 16 or 32)", c->block_size);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", c->head_dim);
  if (c->dtype != PKV_F32 && c->dtype != PKV_F16 && c->dtype != PKV_BF16 && c->dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_INVALID, "unknown dtype %d", c->dtype);
  if (c->dtype == PKV_FP8_E4M3) {
    if (c->model_dtype != PKV_F16 && c->model_dtype != PKV_BF16)
      return fail(PKV_ERR_INVALID, "an 8-bit cache needs model_dtype PKV_F16 or PKV_BF16");
    if (!(c->k_scale > 0.f) || !(c->k_scale < INFINITY) || !(c->v_scale > 0.f) || !(c->v_scale < INFINITY))
      return fail(PKV_ERR_INVALID, "k_scale and v_scale must be positive and finite");
  } else if (c->model_dtype != c->dtype) {
    return fail(PKV_ERR_INVALID, "model_dtype must equal dtype for a 16/32-bit cache");
  }
  d->k = c->k_pool;
  d->v = c->v_pool;
  d->num_blocks = c->num_blocks;
  d->H = c->num_kv_heads;
  d->B = c->block_size;
  d->D = c->head_dim;
  d->dtype = c->dtype;
  d->mdtype = c->model_dtype;
  d->k_scale = c->dtype == PKV_FP8_E4M3 ? c->k_scale : 1.f;
  d->v_scale = c->dtype == PKV_FP8_E4M3 ? c->v_scale : 1.f;
  return PKV_OK;
}

pkv_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

struct Partitioning {
  int tokens;
  int count;
};

Partitioning partitioning(int max_context_len, int partition_size, int B) {
  Partitioning p;
  if (partition_size <= 0 || partition_size >= max_context_len) {
    p.tokens = (max_context_len + B - 1) / B * B;
    p.count = 1;
  } else {
    p.tokens = partition_size;
    p.count = (max_context_len + partition_size - 1) / partition_size;
  }
  return p;
}

size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// How a decode call is scheduled and where its workspace pieces live.
struct DecodePlan {
  bool mfma = false;   // grouped heads on the matrix cores
  bool flat = false;   // balanced schedule
  int flat_grid = 0;
  Partitioning part{0, 1};
  size_t off_ml = 0, off_acc = 0, bytes = 0;
  bool reduce() const { return flat || part.count > 1; }
};

// Assumes a validated cache and sizes.
DecodePlan plan_decode(const pkv::CacheDesc &c, int S, int Hq, int max_context_len,
                       int partition_size) {
  DecodePlan d;
  const int G = Hq / c.H;
  d.mfma = G > 1 && c.dtype != PKV_F32;
  if (partition_size == PKV_PARTITION_AUTO && S <= pkv::kPlanMaxSeqs) {
    d.flat = true;
    d.flat_grid = d.mfma ? pkv::decode_mfma_flat_grid(c, G, S) : pkv::decode_valu_flat_grid(c, S);
    const size_t rows = (size_t)2 * d.flat_grid * (d.mfma ? G : 1);
    d.off_ml = round256(sizeof(int) * ((size_t)pkv::kFlatPrefixAt + S + 1));
    d.off_acc = d.off_ml + round256(rows * 2 * sizeof(float));
    d.bytes = d.off_acc + rows * c.D * sizeof(float);
    return d;
  }
  d.part = partitioning(max_context_len, partition_size == PKV_PARTITION_AUTO ? 0 : partition_size, c.B);
  if (d.part.count > 1) {
    const size_t rows = (size_t)S * Hq * d.part.count;
    d.off_ml = 0;
    d.off_acc = round256(rows * 2 * sizeof(float));
    d.bytes = d.off_acc + rows * c.D * sizeof(float);
  }
  return d;
}

// Validates a decode call and fills `a` and `plan`.
pkv_status prepare_decode(const pkv::CacheDesc &c, void *out, int32_t out_dtype, const void *q,
                          int32_t num_q_heads, const int32_t *block_tables,
                          int32_t max_blocks_per_seq, const int32_t *context_lens,
                          int32_t num_seqs, int32_t max_context_len, int32_t window, float scale,
                          int32_t partition_size, void *workspace, size_t ws_bytes,
                          pkv::DecodeArgs *a, DecodePlan *plan) {
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (!out || !q || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID, "out/q/block_tables/context_lens is NULL");
  if (!aligned16(out) || !aligned16(q)) return fail(PKV_ERR_INVALID, "q/out must be 16-byte aligned");
  if (out_dtype != c.mdtype && out_dtype != PKV_F32)
    return fail(PKV_ERR_INVALID, "out_dtype must be the model dtype or PKV_F32");
  if (num_q_heads <= 0 || num_q_heads % c.H != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c.H);
  if (num_q_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many query heads");
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (max_context_len <= 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * c.B)
    return fail(PKV_ERR_INVALID, "max_context_len %d outside [1, max_blocks_per_seq*block_size]",
                max_context_len);
  if (!(scale > 0.f) || !(scale < INFINITY)) return fail(PKV_ERR_INVALID, "scale must be positive and finite");
  if (window < 0) return fail(PKV_ERR_INVALID, "sliding_window %d < 0", window);
  if (partition_size != PKV_PARTITION_AUTO && (partition_size < 0 || partition_size % c.B != 0))
    return fail(PKV_ERR_INVALID,
                "partition_size %d must be PKV_PARTITION_AUTO, 0 or a positive multiple of block_size %d",
                partition_size, c.B);
  const int G = num_q_heads / c.H;
  if (G > 16 && c.dtype != PKV_F32) return fail(PKV_ERR_UNSUPPORTED, "group size %d > 16", G);
  *plan = plan_decode(c, num_seqs, num_q_heads, max_context_len, partition_size);
  const size_t need = plan->bytes;
  if (need > 0) {
    if (!workspace) return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes required", need);
    if (ws_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace has %zu bytes, %zu required", ws_bytes, need);
    if (!aligned16(workspace)) return fail(PKV_ERR_INVALID, "workspace must be 16-byte aligned");
  }
  a->out = out;
  a->out_f32 = out_dtype == PKV_F32;
  a->q = q;
  a->Hq = num_q_heads;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->S = num_seqs;
  a->max_context_len = max_context_len;
  {
    const int64_t reach = (int64_t)max_blocks_per_seq * c.B;
    const int64_t parts = plan->flat ? reach : (int64_t)plan->part.count * plan->part.tokens;
    a->cap_tokens = (int)std::min<int64_t>(std::min(reach, parts), INT32_MAX);
  }
  a->window = window;
  a->scale = scale;
  a->partition_tokens = plan->part.tokens;
  a->num_partitions = plan->part.count;
  a->flat = plan->flat;
  a->mfma = plan->mfma;
  a->flat_grid = plan->flat_grid;
  a->ws_ml = nullptr;
  a->ws_acc = nullptr;
  a->ws_hdr = nullptr;
  if (need > 0) {
    a->ws_hdr = plan->flat ? (int *)workspace : nullptr;
    a->ws_ml = (float *)((char *)workspace + plan->off_ml);
    a->ws_acc = (float *)((char *)workspace + plan->off_acc);
  }
  return PKV_OK;
}

pkv_status launch_decode(const pkv::CacheDesc &c, const pkv::DecodeArgs &a, const DecodePlan &plan,
                         hipStream_t stream) {
  hipError_t e = plan.mfma ? pkv::launch_decode_mfma(c, a, stream) : pkv::launch_decode_valu(c, a, stream);
  if (e != hipSuccess) return hip_status(e, "paged_decode launch");
  // An appending call's reduce kernel also stores the new tokens: it runs
  // even when there is nothing to reduce.
  if (plan.reduce() || a.new_k != nullptr) {
    e = pkv::launch_decode_reduce(c, a, stream);
    if (e != hipSuccess) return hip_status(e, "paged_decode reduce launch");
  }
  return PKV_OK;
}

// LDS one workgroup may allocate on the current device (0 if unknown),
// asked once per device.
int device_lds_bytes() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int bytes = 0;
  if (hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return 0;
  cache[dev] = bytes;
  return bytes;
}

// Validates a prefill call over num_seqs > 0 sequences and fills `a`.
pkv_status prepare_prefill(const pkv::CacheDesc &c, void *out, int32_t out_dtype, const void *q,
                           int32_t num_q_heads, const int32_t *query_start_loc,
                           const int32_t *context_lens, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_query_len,
                           int32_t max_context_len, float scale, pkv::PrefillArgs *a) {
  if (c.mdtype != PKV_F16 && c.mdtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "prefill supports f16, bf16 and 8-bit caches of f16/bf16 models");
  if (!out || !q || !query_start_loc || !context_lens || !block_tables)
    return fail(PKV_ERR_INVALID, "a required pointer is NULL");
  if (!aligned16(out) || !aligned16(q)) return fail(PKV_ERR_INVALID, "q/out must be 16-byte aligned");
  if (out_dtype != c.mdtype && out_dtype != PKV_F32)
    return fail(PKV_ERR_INVALID, "out_dtype must be the model dtype or PKV_F32");
  if (num_q_heads <= 0 || num_q_heads % c.H != 0)
    return fail(PKV_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                num_q_heads, c.H);
  if (max_blocks_per_seq <= 0) return fail(PKV_ERR_INVALID, "max_blocks_per_seq must be > 0");
  if (max_context_len <= 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * c.B)
    return fail(PKV_ERR_INVALID, "max_context_len %d outside [1, max_blocks_per_seq*block_size]",
                max_context_len);
  if (max_query_len > max_context_len) return fail(PKV_ERR_INVALID, "max_query_len > max_context_len");
  if (!(scale > 0.f) || !(scale < INFINITY)) return fail(PKV_ERR_INVALID, "scale must be positive and finite");
  const int64_t work = (int64_t)num_seqs * num_q_heads * ((max_query_len + 255) / 256);
  if (work >= (int64_t)1 << 31) return fail(PKV_ERR_UNSUPPORTED, "launch too large");
  a->out = out;
  a->out_f32 = out_dtype == PKV_F32;
  a->q = q;
  a->Hq = num_q_heads;
  a->query_start_loc = query_start_loc;
  a->context_lens = context_lens;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->S = num_seqs;
  a->max_query_len = max_query_len;
  a->max_context_len = max_context_len;
  a->scale = scale;
  const int lds_max = device_lds_bytes();
  if (lds_max <= 0) return fail(PKV_ERR_HIP, "cannot query the device's LDS size");
  const size_t lds = pkv::prefill_lds_bytes(c, *a);
  if (lds > (size_t)lds_max)
    return fail(PKV_ERR_UNSUPPORTED,
                "max_context_len %d needs %zu bytes of LDS per workgroup, the device has %d",
                max_context_len, lds, lds_max);
  return PKV_OK;
}

// A second stream, with the events that fork work onto it from a caller's
// stream and join it back.  Created on first use with the device current;
// default priority.  `mu` serialises the record/wait sequence of concurrent
// callers on one caller stream.
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  std::mutex mu;
};

// The side stream of (current device, caller stream): every caller stream gets
// its own, so mixed steps from different streams never queue behind each
// other, and a graph capture on one caller's stream forks only into that
// caller's side stream.  Created on first use, kept until the process ends.
pkv_status side_stream(hipStream_t caller, SideStream **out) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, SideStream *> streams;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, caller);
  auto it = streams.find(key);
  if (it != streams.end()) {
    *out = it->second;
    return PKV_OK;
  }
  SideStream *ss = new SideStream;
  e = hipStreamCreateWithFlags(&ss->stream, hipStreamNonBlocking);
  // Both ends of the fork and the join are queues of this device, and each
  // kernel's own end-of-dispatch release makes its writes visible device-wide;
  // the events skip the system-scope fence, which only serves the host.
  const unsigned ev_flags = hipEventDisableTiming | hipEventDisableSystemFence;
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ss->fork, ev_flags);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ss->join, ev_flags);
  if (e != hipSuccess) {
    if (ss->join) (void)hipEventDestroy(ss->join);
    if (ss->fork) (void)hipEventDestroy(ss->fork);
    if (ss->stream) (void)hipStreamDestroy(ss->stream);
    delete ss;
    return hip_status(e, "side stream setup");
  }
  streams[key] = ss;
  *out = ss;
  return PKV_OK;
}

}  // namespace

namespace pkv {

int report_error(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int resident_workgroups(const void *kernel, int threads, size_t lds_bytes) {
  static std::mutex mu;
  static std::map<std::tuple<const void *, size_t, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  const size_t lds_key = (lds_bytes + 1023) / 1024;
  const auto key = std::make_tuple(kernel, lds_key, dev);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds_key * 1024) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 1;
  const int n = per_cu * cus;
  cache[key] = n;
  return n;
}

}  // namespace pkv

extern "C" {

const char *pkv_last_error(void) { return g_err; }

const char *pkv_version(void) { return "pkv 0.1 gfx950"; }

pkv_status pkv_reshape_and_cache(const pkv_cache *cache, const void *key, const void *value,
                                 const int64_t *slot_mapping, int64_t num_tokens,
                                 hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_tokens < 0) return fail(PKV_ERR_INVALID, "num_tokens < 0");
  if (num_tokens == 0) return ok();
  if (!key || !value || !slot_mapping) return fail(PKV_ERR_INVALID, "key/value/slot_mapping is NULL");
  if (!aligned16(key) || !aligned16(value)) return fail(PKV_ERR_INVALID, "key/value must be 16-byte aligned");
  if ((num_tokens + 15) / 16 > 0x7fffffff) return fail(PKV_ERR_UNSUPPORTED, "too many tokens per call");
  if (c.H > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
  return hip_status(pkv::launch_reshape_and_cache(c, key, value, slot_mapping, num_tokens, stream),
                    "reshape_and_cache launch");
}

pkv_status pkv_copy_blocks(const pkv_cache *cache, const int32_t *src_dst, int64_t num_pairs,
                           hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_pairs < 0) return fail(PKV_ERR_INVALID, "num_pairs < 0");
  if (num_pairs == 0) return ok();
  if (!src_dst) return fail(PKV_ERR_INVALID, "src_dst is NULL");
  if (num_pairs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 pairs per call");
  return hip_status(pkv::launch_copy_blocks(c, src_dst, num_pairs, stream), "copy_blocks launch");
}

size_t pkv_decode_workspace_bytes(const pkv_cache *cache, int32_t num_seqs, int32_t num_q_heads,
                                  int32_t max_context_len, int32_t partition_size) {
  pkv::CacheDesc c;
  if (check_cache(cache, &c) != PKV_OK) return 0;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_q_heads % c.H != 0 || max_context_len <= 0)
    return 0;
  return plan_decode(c, num_seqs, num_q_heads, max_context_len, partition_size).bytes;
}

pkv_status pkv_paged_decode_window(const pkv_cache *cache, void *out, int32_t out_dtype,
                                   const void *q, int32_t num_q_heads,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *context_lens, int32_t num_seqs,
                                   int32_t max_context_len, int32_t sliding_window, float scale,
                                   int32_t partition_size, void *workspace, size_t ws_bytes,
                                   hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs < 0");
  if (num_seqs == 0) return ok();
  pkv::DecodeArgs a;
  DecodePlan plan;
  st = prepare_decode(c, out, out_dtype, q, num_q_heads, block_tables, max_blocks_per_seq,
                      context_lens, num_seqs, max_context_len, sliding_window, scale,
                      partition_size, workspace, ws_bytes, &a, &plan);
  if (st) return st;
  st = launch_decode(c, a, plan, stream);
  return st ? st : ok();
}

pkv_status pkv_paged_decode_append(const pkv_cache *cache, const void *key, const void *value,
                                   void *out, int32_t out_dtype, const void *q,
                                   int32_t num_q_heads, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *context_lens,
                                   int32_t num_seqs, int32_t max_context_len,
                                   int32_t sliding_window, float scale, int32_t partition_size,
                                   void *workspace, size_t ws_bytes, hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs < 0");
  if (num_seqs == 0) return ok();
  if (!key || !value) return fail(PKV_ERR_INVALID, "key/value is NULL");
  if (!aligned16(key) || !aligned16(value)) return fail(PKV_ERR_INVALID, "key/value must be 16-byte aligned");
  pkv::DecodeArgs a;
  DecodePlan plan;
  st = prepare_decode(c, out, out_dtype, q, num_q_heads, block_tables, max_blocks_per_seq,
                      context_lens, num_seqs, max_context_len, sliding_window, scale,
                      partition_size, workspace, ws_bytes, &a, &plan);
  if (st) return st;
  a.new_k = key;
  a.new_v = value;
  st = launch_decode(c, a, plan, stream);
  return st ? st : ok();
}

pkv_status pkv_paged_decode(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                            int32_t num_q_heads,
                            const int32_t *block_tables, int32_t max_blocks_per_seq,
                            const int32_t *context_lens, int32_t num_seqs,
                            int32_t max_context_len, float scale, int32_t partition_size,
                            void *workspace, size_t ws_bytes, hipStream_t stream) {
  return pkv_paged_decode_window(cache, out, out_dtype, q, num_q_heads, block_tables,
                                 max_blocks_per_seq, context_lens, num_seqs, max_context_len, 0,
                                 scale, partition_size, workspace, ws_bytes, stream);
}

pkv_status pkv_paged_prefill(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                             int32_t num_q_heads, const int32_t *query_start_loc,
                             const int32_t *context_lens, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, int32_t num_seqs, int32_t max_query_len,
                             int32_t max_context_len, float scale, hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (c.mdtype != PKV_F16 && c.mdtype != PKV_BF16)
    return fail(PKV_ERR_UNSUPPORTED, "prefill supports f16, bf16 and 8-bit caches of f16/bf16 models");
  if (num_seqs < 0 || max_query_len < 0) return fail(PKV_ERR_INVALID, "negative size");
  if (num_seqs == 0 || max_query_len == 0) return ok();
  pkv::PrefillArgs a;
  st = prepare_prefill(c, out, out_dtype, q, num_q_heads, query_start_loc, context_lens,
                       block_tables, max_blocks_per_seq, num_seqs, max_query_len, max_context_len,
                       scale, &a);
  if (st) return st;
  return hip_status(pkv::launch_prefill(c, a, stream), "paged_prefill launch");
}

pkv_status pkv_paged_mixed(const pkv_cache *cache, void *out, int32_t out_dtype, const void *q,
                           int32_t num_q_heads, const int32_t *query_start_loc,
                           const int32_t *context_lens, const int32_t *block_tables,
                           int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_decode_seqs,
                           int32_t max_query_len, int32_t max_context_len, float scale,
                           int32_t partition_size, void *workspace, size_t ws_bytes,
                           hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_seqs < 0 || num_decode_seqs < 0 || max_query_len < 0)
    return fail(PKV_ERR_INVALID, "negative size");
  if (num_decode_seqs > num_seqs) return fail(PKV_ERR_INVALID, "num_decode_seqs > num_seqs");
  const int32_t np = num_seqs - num_decode_seqs;
  const bool has_prefill = np > 0 && max_query_len > 0;
  const bool has_decode = num_decode_seqs > 0;
  if (!query_start_loc && np > 0) return fail(PKV_ERR_INVALID, "query_start_loc is NULL");
  pkv::DecodeArgs da;
  DecodePlan plan;
  if (has_decode) {
    st = prepare_decode(c, out, out_dtype, q, num_q_heads, block_tables, max_blocks_per_seq,
                        context_lens, num_decode_seqs, max_context_len, 0, scale, partition_size,
                        workspace, ws_bytes, &da, &plan);
    if (st) return st;
  }
  pkv::PrefillArgs pa;
  if (has_prefill) {
    // The chunk sequences' own rows of the integer inputs; query_start_loc
    // keeps absolute row numbers, so q and out stay the whole step's.
    st = prepare_prefill(c, out, out_dtype, q, num_q_heads, query_start_loc + num_decode_seqs,
                         context_lens + num_decode_seqs,
                         block_tables + (size_t)num_decode_seqs * max_blocks_per_seq,
                         max_blocks_per_seq, np, max_query_len, max_context_len, scale, &pa);
    if (st) return st;
  }
  if (!has_decode && !has_prefill) return ok();
  if (!has_decode) return hip_status(pkv::launch_prefill(c, pa, stream), "paged_mixed prefill launch");
  if (!has_prefill) {
    st = launch_decode(c, da, plan, stream);
    return st ? st : ok();
  }
  // Both kinds: the chunk rows go on the caller's stream first, the decode
  // rows on the side stream, so the matrix-core prefill and the HBM-bound
  // decode share the chip; the caller's stream then waits for the decode
  // kernel and reduces its split rows.
  SideStream *ss = nullptr;
  st = side_stream(stream, &ss);
  if (st) return st;
  std::lock_guard<std::mutex> lock(ss->mu);
  hipError_t e = hipEventRecord(ss->fork, stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(ss->stream, ss->fork, 0);
  if (e != hipSuccess) return hip_status(e, "paged_mixed fork");
  e = pkv::launch_prefill(c, pa, stream);
  if (e != hipSuccess) return hip_status(e, "paged_mixed prefill launch");
  // Only the decode kernel goes on the side stream; the reduce of its split
  // rows follows the join on the caller's stream, where the next call's work
  // then follows it without another cross-queue wait (a call 2-3 us shorter
  // than with the reduce on the side stream).  Join even after a failed
  // decode launch: the side stream must not run ahead of later work on the
  // caller's stream.
  const hipError_t ed = plan.mfma ? pkv::launch_decode_mfma(c, da, ss->stream)
                                  : pkv::launch_decode_valu(c, da, ss->stream);
  e = hipEventRecord(ss->join, ss->stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(stream, ss->join, 0);
  if (ed != hipSuccess) return hip_status(ed, "paged_mixed decode launch");
  if (e != hipSuccess) return hip_status(e, "paged_mixed join");
  if (plan.reduce()) {
    e = pkv::launch_decode_reduce(c, da, stream);
    if (e != hipSuccess) return hip_status(e, "paged_mixed reduce launch");
  }
  return ok();
}

pkv_status pkv_gather_kv(const pkv_cache *cache, void *k_out, void *v_out,
                         const int32_t *block_tables, int32_t max_blocks_per_seq,
                         const int32_t *context_lens, const int32_t *cu_context_lens,
                         int32_t num_seqs, int32_t max_context_len, hipStream_t stream) {
  pkv::CacheDesc c;
  pkv_status st = check_cache(cache, &c);
  if (st) return st;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID, "num_seqs < 0");
  if (num_seqs == 0) return ok();
  if (num_seqs > 65535) return fail(PKV_ERR_UNSUPPORTED, "at most 65535 sequences per call");
  if (!k_out || !v_out || !block_tables || !context_lens || !cu_context_lens)
    return fail(PKV_ERR_INVALID, "a required pointer is NULL");
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(PKV_ERR_INVALID, "outputs must be 16-byte aligned");
  if (max_blocks_per_seq <= 0 || max_context_len <= 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * c.B)
    return fail(PKV_ERR_INVALID, "bad max_blocks_per_seq / max_context_len");
  return hip_status(pkv::launch_gather_kv(c, k_out, v_out, block_tables, max_blocks_per_seq,
                                          context_lens, cu_context_lens, num_seqs, max_context_len,
                                          stream),
                    "gather_kv launch");
}

pkv_status pkv_validate_host(const int64_t *slot_mapping, int64_t num_tokens,
                             const int32_t *block_tables, int32_t max_blocks_per_seq,
                             const int32_t *context_lens, int32_t num_seqs, int64_t num_blocks,
                             int32_t block_size, int32_t max_context_len) {
  if (num_blocks <= 0 || block_size <= 0) return fail(PKV_ERR_INVALID, "bad pool geometry");
  if (slot_mapping && num_tokens > 0) {
    std::unordered_set<int64_t> seen;
    seen.reserve((size_t)num_tokens * 2);
    const int64_t nslots = num_blocks * block_size;
    for (int64_t t = 0; t < num_tokens; ++t) {
      const int64_t s = slot_mapping[t];
      if (s < 0) continue;
      if (s >= nslots)
        return fail(PKV_ERR_INVALID, "slot_mapping[%lld] = %lld >= %lld slots", (long long)t,
                    (long long)s, (long long)nslots);
      if (!seen.insert(s).second)
        return fail(PKV_ERR_INVALID, "slot %lld appears twice (token %lld)", (long long)s, (long long)t);
    }
  }
  if (context_lens && num_seqs > 0) {
    if (!block_tables || max_blocks_per_seq <= 0)
      return fail(PKV_ERR_INVALID, "block_tables needed with context_lens");
    for (int32_t s = 0; s < num_seqs; ++s) {
      const int32_t L = context_lens[s];
      if (L < 1 || (int64_t)L > (int64_t)max_blocks_per_seq * block_size)
        return fail(PKV_ERR_INVALID, "context_lens[%d] = %d outside [1, %lld]", s, L,
                    (long long)max_blocks_per_seq * block_size);
      if (max_context_len > 0 && L > max_context_len)
        return fail(PKV_ERR_INVALID, "context_lens[%d] = %d > max_context_len %d", s, L,
                    max_context_len);
      const int32_t nb = (L + block_size - 1) / block_size;
      for (int32_t i = 0; i < nb; ++i) {
        const int32_t b = block_tables[(size_t)s * max_blocks_per_seq + i];
        if (b < 0 || b >= num_blocks)
          return fail(PKV_ERR_INVALID, "block_tables[%d][%d] = %d outside [0, %lld)", s, i, b,
                      (long long)num_blocks);
      }
    }
  }
  return ok();
}

}  // extern "C"
