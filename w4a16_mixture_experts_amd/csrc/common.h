// Internal definitions shared by the libexmoe sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstddef>
#include <cstdint>
#include <string>

#include "exmoe.h"

namespace exmoe {

constexpr int kGroup = 128;      // quantization group (inputs per scale)
constexpr int kTileRows = 16;    // output rows per packed tile
constexpr int kTileBytes = 1024; // 16 rows x 128 inputs x 4 bits
constexpr int kScaleBytes = 32;  // 16 bf16 scales per tile
constexpr int kMaxExperts = 256;
constexpr int kMaxDim = 16384;   // largest hidden / intermediate size (zero-row length)

__host__ __device__ inline size_t n_tiles(int H, int I) {
  return 2 * (size_t)(I / kTileRows) * (H / kGroup) + (size_t)(H / kTileRows) * (I / kGroup);
}
__host__ __device__ inline size_t packed_bytes(int H, int I) { return n_tiles(H, I) * (kTileBytes + kScaleBytes); }

// Thread-local error reporting.
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int hip_error(hipError_t e, const char* what);

#define EXMOE_HIP(call)                                   \
  do {                                                    \
    hipError_t _e = (call);                               \
    if (_e != hipSuccess) return ::exmoe::hip_error(_e, #call); \
  } while (0)

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Per-kernel timing for benchmarks (exmoe_profile_enable). While profiling is on and the
// stream is not being captured, the scope holds an event pair that EXMOE_LAUNCH hands to
// hipExtLaunchKernelGGL, which stamps the kernel's own start and end; otherwise
// EXMOE_LAUNCH is a plain launch.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t s);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;
  bool timing() const { return a_ != nullptr && b_ != nullptr; }
  hipEvent_t start() const { return a_; }
  hipEvent_t stop() const { return b_; }
  void used() { used_ = true; }

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t a_ = nullptr, b_ = nullptr;
  bool used_ = false;
};

#define EXMOE_LAUNCH(prof, kernel, grid, block, shmem, stream, ...)                                     \
  do {                                                                                                 \
    if ((prof).timing()) {                                                                             \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (prof).start(), (prof).stop(), 0,      \
                            __VA_ARGS__);                                                              \
      (prof).used();                                                                                   \
    } else {                                                                                           \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                             \
    }                                                                                                  \
  } while (0)

// ---- kernel launchers (defined in the .hip files); each returns a HIP error code
hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                               int E, uint16_t* logits, hipStream_t s);
hipError_t launch_topk(const uint16_t* logits, const int32_t* given_ids, int T, int E, int k,
                       int renormalize, int32_t* ids, float* w, hipStream_t s);
hipError_t launch_topk_group(const uint16_t* logits, int T, int E, int k, int renormalize, int32_t* ids,
                             float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                             hipStream_t s);
hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_flat,
                        int32_t* flat_to_sorted, hipStream_t s);

struct MoeArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* w;
  const int32_t* offsets;
  const int32_t* sorted_flat;
  const int32_t* flat_to_sorted;
  const uint8_t* base;
  size_t stride;
  const int32_t* e2s;
  int T, H, I, E, k;
  uint16_t* y;
  // workspace carve-up
  uint16_t* h;        // bf16 [T*k, I], sorted-row order
  float* y_perm;      // fp32 [T*k, H], sorted-row order, already multiplied by the routing weight
  float* gsum;        // fp32 [I/128][T*k + 128]: -136 * group sums of h per sorted row (down seeds)
  float* xsum;        // fp32 [H/128][T*k + 128]: -136 * group sums of x per sorted row (gate/up seeds)
  uint32_t* counters; // decode last-arriver counters
  uint32_t* debug;    // debug word(s)
};

size_t moe_workspace_layout(int T, int H, int I, int E, int k, int path, MoeArgs* a, void* ws);
// Routed rows up to which the decode kernels group the rows themselves from the top-k ids.
constexpr int kDecMaxRows = 1024;
// Decode path from offsets and permutation given by the caller.
hipError_t launch_moe_decode(const MoeArgs& a, hipStream_t s);
// Logits, top-k selection and routing weights of each token by one workgroup per token.
hipError_t launch_route_token(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                              int k, int renormalize, uint16_t* logits, int32_t* ids, float* w, hipStream_t s);
// Decode path from the top-k ids alone (T * k <= kDecMaxRows): the gate/up kernel groups
// the routed rows itself and publishes the grouping to offsets / sorted_flat /
// flat_to_sorted, which a.offsets and a.sorted_flat must alias.
hipError_t launch_moe_decode_from_ids(const MoeArgs& a, int32_t* offsets, int32_t* sorted_flat,
                                      int32_t* flat_to_sorted, hipStream_t s);
hipError_t launch_moe_prefill(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_expert_range(const MoeArgs& a, int expert, int rows, hipStream_t s);  // sequential path
hipError_t launch_combine(const MoeArgs& a, hipStream_t s);

}  // namespace exmoe
