// The whole layer (exmoe_moe_layer) for callers that cannot allocate device memory: its
// workspace is a fixed array in the library's device code object, one per GPU, instead of
// a caller buffer. Same kernels, same results.
#include <mutex>

#include "common.h"

namespace exmoe {

// Largest workspace the no-allocation layer call serves (every OLMoE-shaped decode size and
// prefill up to about 700 tokens). Device globals start zeroed, which the routing kernel's
// arrival counters at the front of a workspace require; every call leaves them zero.
constexpr size_t kScratchBytes = 64ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`, looked up once per device (with that
// device current): in host code the array's name is not a device address.
int scratch_for_current_device(void** out) {
  int dev = -1;
  EXMOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return set_error(EXMOE_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    EXMOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return set_error(EXMOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EXMOE_OK;
}
}  // namespace

}  // namespace exmoe

using namespace exmoe;

extern "C" int exmoe_moe_layer_noalloc(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias,
                                       const exmoe_expert_bank* bank, int T, int H, int I, int E, int k,
                                       int renormalize, int flags, exmoe_bf16* logits, int32_t* topk_ids,
                                       float* topk_weights, int32_t* expert_offsets, int32_t* sorted_flat,
                                       int32_t* flat_to_sorted, exmoe_bf16* y, hipStream_t stream) {
  if (flags & EXMOE_FLAG_DEBUG_COUNTERS)
    return set_error(EXMOE_ERR_UNSUPPORTED, "no workspace to read the exactness counters from: use exmoe_moe_layer");
  const size_t need = exmoe_moe_layer_workspace_bytes(T, H, I, E, k, flags);
  if (need == 0 && T != 0) {
    // the shape itself is invalid: let the layer call report it
    return exmoe_moe_layer(x, w_router, logit_bias, bank, T, H, I, E, k, renormalize, flags, logits, topk_ids,
                           topk_weights, expert_offsets, sorted_flat, flat_to_sorted, y, nullptr, 0, stream);
  }
  if (need > kScratchBytes)
    return set_error(EXMOE_ERR_UNSUPPORTED,
                     "this layer call needs a %zu-byte workspace; the no-allocation entry point holds %zu bytes "
                     "(use exmoe_moe_layer with a workspace)", need, kScratchBytes);
  void* ws = nullptr;
  int st = scratch_for_current_device(&ws);
  if (st) return st;
  return exmoe_moe_layer(x, w_router, logit_bias, bank, T, H, I, E, k, renormalize, flags, logits, topk_ids,
                         topk_weights, expert_offsets, sorted_flat, flat_to_sorted, y, ws, kScratchBytes, stream);
}
