// Internal launch interface between the C-ABI layer (pkv_api.cpp) and the
// kernel translation units.  Host-only declarations; every launcher assumes
// its arguments were validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Sequences per launch that the decode kernels' in-LDS prefix supports;
// beyond it they run one workgroup per grid cell.
constexpr int kPlanMaxSeqs = 8192;

// Balanced-schedule workspace header (ints): [0] units per workgroup, [1]
// total units, then from kFlatPrefixAt the prefix sums of units per sequence.
constexpr int kFlatPrefixAt = 64;

struct CacheDesc {
  void *k;           // [num_blocks][H][D/X][B][X], X = 64 bytes / element
  void *v;           // [num_blocks][H][D][B]
  int64_t num_blocks;
  int H, B, D;
  int dtype;         // pools: 0 f32, 1 f16, 2 bf16, 3 fp8 e4m3
  int mdtype;        // key/value inputs, queries, outputs (== dtype unless fp8)
  float k_scale, v_scale;  // fp8 cache: stored = x / scale, read = code * scale
  int elt_bytes() const { return dtype == 0 ? 4 : dtype == 3 ? 1 : 2; }
  bool fp8() const { return dtype == 3; }
};

struct DecodeArgs {
  void *out;
  bool out_f32;           // out is fp32 instead of the cache dtype
  const void *q;
  int Hq;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *context_lens;
  int S;
  int max_context_len;
  // Every length is clamped to cap_tokens: the table's reach, and for the
  // partitioned schedules also num_partitions * partition_tokens, so that a
  // length beyond max_context_len (a broken contract) can never name a
  // partition the workspace has no row for.
  int cap_tokens;
  int window;             // sliding window in tokens (0: attend to the whole context)
  float scale;
  int partition_tokens;   // > 0, multiple of B
  int num_partitions;     // ceil(max_context_len / partition_tokens)
  bool flat;              // balanced schedule (partition fields unused)
  bool mfma = false;      // grouped heads on the matrix cores: one work unit per KV head
                          // (the decode and the reduce kernels must agree on it)
  int flat_grid;          // its workgroup count
  // Partial rows (running max and denominator in the log2 domain, weighted
  // sums): fixed partitions [S][Hq][num_partitions], balanced schedule
  // [2 * flat_grid][G].  ws_hdr: the balanced schedule's header.
  float *ws_ml;
  float *ws_acc;
  int *ws_hdr;
  // Appending call: the new token's key and value rows, [S][Hkv][D] in the
  // model dtype (nullptr: plain decode).
  const void *new_k = nullptr;
  const void *new_v = nullptr;
};

struct PrefillArgs {
  void *out;
  bool out_f32;
  const void *q;
  int Hq;
  const int32_t *query_start_loc;
  const int32_t *context_lens;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  int S;
  int max_query_len;
  int max_context_len;
  float scale;
};

// Sets this thread's last-error message (pkv_last_error) and returns
// `status`; for entry points defined outside pkv_api.cpp.
int report_error(int status, const char *fmt, ...);

// Workgroups of `kernel` (with `threads` threads and `lds_bytes` of dynamic
// LDS) that the current device keeps resident at once: the size of a
// persistent grid.  Cached per (kernel, LDS size, device).
int resident_workgroups(const void *kernel, int threads, size_t lds_bytes);

hipError_t launch_reshape_and_cache(const CacheDesc &c, const void *key, const void *value,
                                    const int64_t *slots, int64_t T, hipStream_t stream);
hipError_t launch_copy_blocks(const CacheDesc &c, const int32_t *pairs, int64_t n,
                              hipStream_t stream);
hipError_t launch_gather_kv(const CacheDesc &c, void *k_out, void *v_out, const int32_t *bt,
                            int mbps, const int32_t *ctx, const int32_t *cu, int S,
                            int max_context_len, hipStream_t stream);

// Wavefront dot-product decode (any dtype, one query head per workgroup).
hipError_t launch_decode_valu(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream);
// Matrix-core decode for grouped heads (f16/bf16, 2 <= G <= 16).
hipError_t launch_decode_mfma(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream);
// Workgroup count of the balanced schedule (the resident capacity of the
// device for that kernel): sizes its workspace.
int decode_valu_flat_grid(const CacheDesc &c, int S);
int decode_mfma_flat_grid(const CacheDesc &c, int G, int S);
// Combine split-KV partials into the output (only segments that were split).
hipError_t launch_decode_reduce(const CacheDesc &c, const DecodeArgs &a, hipStream_t stream);
// Matrix-core causal chunked prefill (f16/bf16).
hipError_t launch_prefill(const CacheDesc &c, const PrefillArgs &a, hipStream_t stream);
// LDS one prefill workgroup takes for these arguments (static tiles + the
// staged block table); SIZE_MAX if the kernel's attributes are unavailable.
size_t prefill_lds_bytes(const CacheDesc &c, const PrefillArgs &a);

}  // namespace pkv
