// Internal definitions shared by the libexmoe sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "exmoe.h"

namespace exmoe {

constexpr int kGroup = 128;      // quantization group (inputs per scale)
constexpr int kTileRows = 16;    // output rows per packed tile
constexpr int kTileBytes = 1024; // 16 rows x 128 inputs x 4 bits
constexpr int kScaleBytes = 32;  // 16 bf16 scales per tile
constexpr int kMaxExperts = 256;
constexpr int kMaxK = 64;
constexpr int kSpanSub = 64;     // sub-slots of a launch span slot (by workgroup index)
constexpr int kMaxDim = 16384;   // largest hidden / intermediate size (zero-row length)

__host__ __device__ inline size_t n_tiles(int H, int I) {
  return 2 * (size_t)(I / kTileRows) * (H / kGroup) + (size_t)(H / kTileRows) * (I / kGroup);
}
__host__ __device__ inline size_t packed_bytes(int H, int I) { return n_tiles(H, I) * (kTileBytes + kScaleBytes); }
// dense bf16 expert of the comparator: gate, up and down, 2 bytes per weight
__host__ __device__ inline size_t bf16_expert_bytes(int H, int I) { return (size_t)6 * H * I; }

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
  // Next launch span slot while span stamps are enabled (also under stream capture), else
  // null. The slot is tagged with this scope's kernel name.
  unsigned long long* span();

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
hipError_t span_fill(unsigned long long* p, int n, hipStream_t s);
// dst[0..n) = host[0..n) (n <= kMaxExperts) by a one-workgroup kernel that takes the values
// as kernel arguments: ordered on s, and the host buffer may be reused when the call returns.
hipError_t table_upload(int32_t* dst, const int32_t* host, int n, hipStream_t s);
// After the waves of a cached forward: flags (bit 0 of *debug) every expert with a
// non-empty segment whose bit is clear in mask (the union of the waves' experts).
hipError_t check_wave_union(const int32_t* offsets, int E, const uint32_t mask[kMaxExperts / 32], uint32_t* debug,
                            hipStream_t s);
// xsum (optional, fp32 [H/128][T], H <= kLgtXsMaxH): also the grouped GEMM's correction
// seeds of x, the values launch_moe_prefill_xsum writes.
constexpr int kLgtXsMaxH = 4096;
hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                               int E, uint16_t* logits, hipStream_t s, float* xsum = nullptr);
hipError_t launch_topk(const uint16_t* logits, const int32_t* given_ids, int T, int E, int k,
                       int renormalize, int32_t* ids, float* w, hipStream_t s);
// group_ws: group_workspace_bytes(T * k, E) bytes (may be null when that is 0)
hipError_t launch_topk_group(const uint16_t* logits, int T, int E, int k, int renormalize, int32_t* ids,
                             float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                             int32_t* group_ws, hipStream_t s);
size_t group_workspace_bytes(int n, int E);
hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_flat,
                        int32_t* flat_to_sorted, int32_t* group_ws, hipStream_t s);

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
  float* part;        // fp32 [I/128][T*k, H]: fused decode, down output of each 128-wide slice of I
  int nparts;         // slices in part (0: the combine reads y_perm)
  float* y_perm;      // fp32 [T*k, H], sorted-row order, already multiplied by the routing weight
  float* gsum;        // fp32 [I/128][T*k + 128]: -136 * group sums of h per sorted row (down seeds)
  float* xsum;        // fp32 [H/128][T]: -136 * group sums of x per token (gate/up seeds)
  uint8_t* sel;       // u8 [E][16]: decode expert table, sel[e][t] = slot + 1 of token t (0: not routed)
  uint32_t* counters; // arrival counters of the routing kernel (zero between launches)
  uint32_t* debug;    // debug word(s)
  unsigned long long* span;   // launch span slot (benchmark timing) or null
  int skip_absent;    // experts without a slot are skipped silently (one wave of a cached forward)
  int32_t* wave_table;  // int32 [E] workspace: the expert->slot table of one wave
  int32_t* group_ws;    // chunk counts of the grouping of more than 4096 rows
  int32_t* rows_ctr;    // int32 [E] in the workspace header: rows executed per expert
                        // (EXMOE_FLAG_DEBUG_COUNTERS), or null
};

size_t moe_workspace_layout(int T, int H, int I, int E, int k, int path, MoeArgs* a, void* ws);
// Routed rows up to which the decode kernels group the rows themselves from the top-k ids.
constexpr int kDecMaxRows = 1024;
// Decode path from offsets and permutation given by the caller.
hipError_t launch_moe_decode(const MoeArgs& a, hipStream_t s);
// Whether the decode path runs gate/up and down in one kernel (down outputs per slice of
// 16 * the returned value rows of I, summed by the combine): 16 or 8 (that many waves per
// workgroup, one row block each) when that gives enough workgroups, 2 for the narrow
// kernel (32-row slices, 16 waves) when only a few rows are routed; 0: two kernels.
int decode_fused_waves(int T, int H, int I, int E, int k);
// Logits, top-k selection and routing weights of each token by one workgroup per token.
hipError_t launch_route_token(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                              int k, int renormalize, uint16_t* logits, int32_t* ids, float* w, hipStream_t s);
// Logits, top-k, weights and the decode expert table of T <= kRouteSelMaxTok tokens in one
// launch (arrival counters: ceil(T / 2) of them, zero before the launch and after it).
constexpr int kRouteSelMaxTok = 16;
constexpr int kSelRowBytes = 16;   // bytes per expert row of the routing table: one per token (T <= 16)
constexpr int kRouteSelCounters = 8, kRouteCounterStride = 64;   // counter i at word i * stride
hipError_t launch_route_sel(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E, int k,
                            int renormalize, uint16_t* logits, int32_t* ids, float* w, uint8_t* sel,
                            uint32_t* counters, hipStream_t s);
// Decode path that groups the routed rows inside its gate/up kernel (T * k <= kDecMaxRows),
// from ids (sel == nullptr) or from the expert table of launch_route_sel (when
// decode_table_routing_ok: every token row is then staged before the weight stream). The
// gate/up kernel publishes the grouping into offsets / sorted_flat / flat_to_sorted; a.ids,
// a.offsets and a.sorted_flat must alias those buffers.
bool decode_table_routing_ok(int T, int H, int E, int k);
hipError_t launch_moe_decode_routed(const MoeArgs& a, const uint8_t* sel, int32_t* offsets, int32_t* sorted_flat,
                                    int32_t* flat_to_sorted, hipStream_t s);
// Decode path that makes the top-k selection itself from the bf16 logits of
// launch_route_logits (when decode_logit_routing_ok: table routing with E <= 64 and the
// fused expert kernels): every workgroup ranks the experts of each token, and the
// publisher workgroup also writes ids and routing weights (a.ids / a.w alias them).
bool decode_logit_routing_ok(int T, int H, int I, int E, int k);
hipError_t launch_moe_decode_logit_routed(const MoeArgs& a, const uint16_t* logits, int renormalize, int32_t* ids,
                                          float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                                          hipStream_t s);
// The paths in parts (a forward in waves runs the expert kernels once per wave and the
// correction sums and the combine once): decode experts; prefill sums, experts.
hipError_t launch_moe_decode_experts(const MoeArgs& a, hipStream_t s);
// Experts per layer, slots per layer, dry-run flag and bytes per expert of a slot cache.
void slot_cache_shape(const exmoe_slot_cache* c, int* E, int* S, int* dry, size_t* expert_bytes);
int slot_cache_layers(const exmoe_slot_cache* c);
// exmoe_slot_cache_acquire whose copies wait only for `after` (an event recorded on the
// compute stream) unless one of them lands in a slot of protect_slots; after == NULL
// waits for everything enqueued on the compute stream so far (the public behaviour).
int slot_cache_acquire_ex(exmoe_slot_cache* c, int layer, const int32_t* active_ids_host, int n_active,
                          hipStream_t compute_stream, hipEvent_t after, const int32_t* protect_slots, int n_protect,
                          exmoe_expert_bank* bank_out);
// The cache-sized waves of a cached forward: A (any order, duplicates allowed) becomes the
// distinct ids in wave order (resident first, then the others, each ascending); returns
// the wave size.
int slot_cache_plan_waves(const exmoe_slot_cache* c, int layer, std::vector<int32_t>& A);
// Event i of the cache's pool (created on first use, destroyed with the cache).
hipError_t slot_cache_event(exmoe_slot_cache* c, int i, hipEvent_t* ev);
// Per-layer mark of the cached forward: recorded on the compute stream after the last
// kernels that read the layer's slots; null when unknown (none yet, or the layer was
// acquired through the public call since, whose readers the cache cannot see).
hipEvent_t slot_cache_layer_mark(exmoe_slot_cache* c, int layer);
hipError_t slot_cache_mark_layer(exmoe_slot_cache* c, int layer, hipStream_t s);
void slot_cache_forget_layer(exmoe_slot_cache* c, int layer);
hipError_t launch_moe_prefill_xsum(const MoeArgs& a, hipStream_t s);
// Dense bf16 experts (the comparator): decode and prefill expert kernels.
hipError_t launch_bf16_decode_experts(const MoeArgs& a, hipStream_t s);
hipError_t launch_bf16_prefill_experts(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_prefill_experts(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_expert_range(const MoeArgs& a, int expert, int rows, hipStream_t s);  // sequential path
hipError_t launch_combine(const MoeArgs& a, hipStream_t s);

}  // namespace exmoe
