// noalloc.hip -- diffkv_decode_attn_noalloc: decode attention whose scratch
// is a fixed device array of the library instead of a caller workspace, for
// callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in the code object: every GPU the library runs on holds
// its own copy for the life of the process.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): the
// device address is looked up once per device with hipGetSymbolAddress,
// with that device current, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "diffkv.h"
#include "dkv_common.hpp"
#include "dkv_launch.hpp"

using namespace dkv;

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // DIFFKV_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == DIFFKV_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on the first call on
// that device), or null on a HIP error.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int diffkv_decode_attn_noalloc(const diffkv_config* cfg, const diffkv_pool* pool, int32_t batch,
                                          const uint16_t* q, const int32_t* page_table, const int32_t* tier_state,
                                          const int32_t* seq_len, float* out, int32_t update_scores,
                                          void* stream) {
  if (!cfg || !pool || batch < 0) return DIFFKV_E_INVALID;
  if (batch > 0 && (!q || !page_table || !tier_state || !seq_len || !out)) return DIFFKV_E_INVALID;
  if ((int64_t)batch * cfg->num_kv_heads > 65535) return DIFFKV_E_INVALID;
  // update_scores = 2 would leave logits for a later call in the shared array
  if (update_scores < 0 || update_scores > 1) return DIFFKV_E_INVALID;
  const size_t need = diffkv_workspace_bytes(cfg, update_scores ? DIFFKV_ATTN_SCORES : DIFFKV_ATTN, batch, 0);
  if (need == 0) return DIFFKV_E_INVALID;  // invalid config
  if (need > kScratchBytes) return DIFFKV_E_WORKSPACE;
  void* ws = scratch_address();
  if (!ws) return DIFFKV_E_HIP;
  return diffkv_decode_attn(cfg, pool, batch, q, page_table, tier_state, seq_len, out, update_scores, ws,
                            kScratchBytes, stream);
}
