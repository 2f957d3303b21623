// Paged decode for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation.
// The split-KV partials that pkv_paged_decode keeps in a caller workspace
// live here in one file-scope device array instead, one copy per GPU.
#include <map>
#include <mutex>

#include "pkv.h"
#include "pkv_launch.h"

namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
}  // namespace

// Held on every GPU the library runs on until the process ends.  In host
// code this name is a host-side stand-in, not a device address: host code
// only ever uses the per-device address that scratch_address() asks for.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of the current GPU's copy of `scratch`, asked once per
// device with that device current and kept.
pkv_status scratch_address(void **ptr) {
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return (pkv_status)pkv::report_error(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it != addr.end()) {
    *ptr = it->second;
    return PKV_OK;
  }
  void *p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || p == nullptr)
    return (pkv_status)pkv::report_error(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s",
                                         dev, hipGetErrorString(e));
  addr[dev] = p;
  *ptr = p;
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_paged_decode_noalloc(const pkv_cache *cache, void *out,
                                               int32_t out_dtype, const void *q,
                                               int32_t num_q_heads, const int32_t *block_tables,
                                               int32_t max_blocks_per_seq,
                                               const int32_t *context_lens, int32_t num_seqs,
                                               int32_t max_context_len, float scale,
                                               int32_t partition_size, hipStream_t stream) {
  const size_t need = pkv_decode_workspace_bytes(cache, num_seqs, num_q_heads, max_context_len,
                                                 partition_size);
  if (need > kScratchBytes)
    return (pkv_status)pkv::report_error(
        PKV_ERR_WORKSPACE,
        "this decode needs %zu bytes of split-KV scratch; the static scratch holds %zu "
        "(use pkv_paged_decode with a workspace)",
        need, kScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const pkv_status st = scratch_address(&ws);
    if (st != PKV_OK) return st;
  }
  return pkv_paged_decode(cache, out, out_dtype, q, num_q_heads, block_tables, max_blocks_per_seq,
                          context_lens, num_seqs, max_context_len, scale, partition_size, ws,
                          need > 0 ? kScratchBytes : 0, stream);
}
