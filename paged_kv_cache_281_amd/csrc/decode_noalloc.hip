// Decode attention without a caller workspace and without any allocation: the split-
// context partials, task list and counters live in a fixed device array of this
// library, one copy per GPU, for callers that cannot allocate (code under HIP graph
// capture, serving loops that forbid allocation).  The kernels are those of
// pkv_paged_attention_decode; only the workspace differs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

static_assert(PKV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");

// The workspace of every pkv_paged_attention_decode_noalloc call on a device.  In host
// code this name is only a handle for hipGetSymbolAddress: kernels receive the device
// address that call returns, never the name.
__device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of this device's `scratch`, looked up once per device (with that
// device current).  Null on failure, with the error recorded.
void* scratch_address(int dev) {
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !addr) {
    char buf[256];
    std::snprintf(buf, sizeof(buf), "pkv_paged_attention_decode_noalloc: hipGetSymbolAddress failed on device %d: %s",
                  dev, hipGetErrorString(e));
    set_error(PKV_ERR_LAUNCH, buf);
    return nullptr;
  }
  g_scratch[dev].store(addr, std::memory_order_release);
  return addr;
}

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_paged_attention_decode_noalloc(const pkv_pool_desc* pool, const void* k_pool,
                                                      const void* v_pool, void* out, const void* q, int32_t num_seqs,
                                                      int32_t num_q_heads, const int32_t* block_tables,
                                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                                      float scale, void* stream) {
  const char* who = "pkv_paged_attention_decode_noalloc";
  const size_t need = pkv_paged_attention_workspace_bytes(num_seqs, num_q_heads, pool ? pool->head_dim : 0,
                                                          max_blocks_per_seq, pool ? pool->block_size : 0);
  if (need > PKV_NOALLOC_SCRATCH_BYTES) {
    char buf[256];
    std::snprintf(buf, sizeof(buf), "%s: these sizes need %zu bytes of workspace, more than the %zu-byte static "
                  "scratch; use pkv_paged_attention_decode with a caller workspace", who, need,
                  static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES));
    return pkv::set_error(PKV_ERR_WORKSPACE, buf);
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= pkv::kMaxDevices) {
    (void)hipGetLastError();
    return pkv::set_error(PKV_ERR_LAUNCH, "pkv_paged_attention_decode_noalloc: no current device");
  }
  void* ws = pkv::scratch_address(dev);
  if (!ws) return PKV_ERR_LAUNCH;
  return pkv_paged_attention_decode(pool, k_pool, v_pool, out, q, num_seqs, num_q_heads, block_tables,
                                    max_blocks_per_seq, context_lens, scale, ws, PKV_NOALLOC_SCRATCH_BYTES, stream);
}
