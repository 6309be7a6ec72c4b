// libexmoe C ABI: argument validation, error reporting, the offline int4 packer, workspace
// layout and kernel dispatch. Every device entry point validates everything before it
// enqueues anything.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "common.h"
#include "moe_seq.h"
#include "exmoe.h"

namespace exmoe {

static thread_local char g_last_error[512] = "";

int set_error(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_error(hipError_t e, const char* what) {
  return set_error(e == hipErrorOutOfMemory ? EXMOE_ERR_OUT_OF_MEMORY : EXMOE_ERR_HIP, "%s: %s", what,
                   hipGetErrorString(e));
}

static int check_shape(int T, int H, int I, int E, int k) {
  if (T < 0) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %d)", T);
  if (H <= 0 || H % kGroup) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "H must be a positive multiple of 128 (got %d)", H);
  if (I <= 0 || I % kGroup) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "I must be a positive multiple of 128 (got %d)", I);
  if (E < 1 || E > kMaxExperts) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "E must be in [1, 256] (got %d)", E);
  if (k < 1 || k > E) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "k must be in [1, E] (got k=%d, E=%d)", k, E);
  if (k > 64) return set_error(EXMOE_ERR_UNSUPPORTED, "k > 64 is not supported (got %d)", k);
  if (H > kMaxDim || I > kMaxDim) return set_error(EXMOE_ERR_UNSUPPORTED, "H and I must be <= %d", kMaxDim);
  if ((long long)T * k > (1LL << 30)) return set_error(EXMOE_ERR_UNSUPPORTED, "T*k too large");
  return EXMOE_OK;
}

#define CHECK_PTR(p)                                                                           \
  do {                                                                                         \
    if (!(p)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "%s must not be NULL", #p);          \
    if (!aligned16(p)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "%s must be 16-byte aligned", #p); \
  } while (0)

#define CHECK_PTR4(p)                                                                          \
  do {                                                                                         \
    if (!(p)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "%s must not be NULL", #p);          \
    if (((uintptr_t)(p)) & 3u) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "%s must be 4-byte aligned", #p); \
  } while (0)

// ------------------------------------------------------------------------------------
// Offline quantize + pack (host)
// ------------------------------------------------------------------------------------
static inline uint16_t host_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static inline float host_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// One tile: rows 16b.., inputs 128g.. of a row-major [N, K] matrix.
static void pack_tile(const float* W, int K, int b, int g, uint8_t* tile_out, uint8_t* scale_out) {
  int8_t q[kTileRows][kGroup];
  for (int r = 0; r < kTileRows; r++) {
    const float* row = W + (size_t)(kTileRows * b + r) * K + (size_t)kGroup * g;
    float amax = 0.f;
    for (int c = 0; c < kGroup; c++) amax = std::max(amax, std::fabs(row[c]));
    const uint16_t sb = host_f32_to_bf16(amax / 7.0f);
    const double s = (double)host_bf16_to_f32(sb);
    for (int c = 0; c < kGroup; c++) {
      double v = s == 0.0 ? 0.0 : std::nearbyint((double)row[c] / s);   // ties to even
      v = std::min(7.0, std::max(-8.0, v));
      q[r][c] = (int8_t)v;
    }
    scale_out[2 * r] = (uint8_t)(sb & 0xFF);
    scale_out[2 * r + 1] = (uint8_t)(sb >> 8);
  }
  for (int l = 0; l < 64; l++) {
    const int r = l % 16, kq = 8 * (l / 16);
    for (int s = 0; s < 4; s++) {
      uint32_t w = 0;
      for (int j = 0; j < 8; j++) {
        const uint32_t u = (uint32_t)(q[r][32 * s + kq + j] + 8);
        const int sh = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);
        w |= u << sh;
      }
      uint8_t* p = tile_out + 16 * l + 4 * s;
      p[0] = (uint8_t)w;
      p[1] = (uint8_t)(w >> 8);
      p[2] = (uint8_t)(w >> 16);
      p[3] = (uint8_t)(w >> 24);
    }
  }
}

static bool all_finite(const float* p, size_t n) {
  for (size_t i = 0; i < n; i++)
    if (!std::isfinite(p[i])) return false;
  return true;
}

}  // namespace exmoe

using namespace exmoe;

extern "C" {

const char* exmoe_status_string(int status) {
  switch (status) {
    case EXMOE_OK: return "ok";
    case EXMOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case EXMOE_ERR_UNSUPPORTED: return "unsupported";
    case EXMOE_ERR_WORKSPACE: return "workspace too small";
    case EXMOE_ERR_HIP: return "HIP runtime error";
    case EXMOE_ERR_OUT_OF_MEMORY: return "out of memory";
    case EXMOE_ERR_CACHE: return "slot cache error";
    default: return "unknown status";
  }
}

const char* exmoe_last_error(void) { return g_last_error; }
int exmoe_abi_version(void) { return EXMOE_ABI_VERSION; }

size_t exmoe_packed_expert_bytes(int H, int I) {
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup) return 0;
  return packed_bytes(H, I);
}

int exmoe_quantize_pack(const float* w_gate, const float* w_up, const float* w_down, int H, int I,
                        int group_size, void* packed, size_t packed_bytes_given) {
  if (!w_gate || !w_up || !w_down || !packed)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "weights and packed buffer must not be NULL");
  if (group_size != kGroup) return set_error(EXMOE_ERR_UNSUPPORTED, "group_size must be 128 (got %d)", group_size);
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "H and I must be positive multiples of 128");
  const size_t need = packed_bytes(H, I);
  if (packed_bytes_given < need)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "packed buffer too small: %zu < %zu", packed_bytes_given, need);
  const size_t nw = (size_t)H * I;
  if (!all_finite(w_gate, nw) || !all_finite(w_up, nw) || !all_finite(w_down, nw))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "weights must be finite");
  const int G = H / kGroup, GD = I / kGroup;
  const size_t n_gu = 2 * (size_t)(I / kTileRows) * G;
  const size_t nt = n_tiles(H, I);
  uint8_t* out = static_cast<uint8_t*>(packed);
  uint8_t* scales = out + nt * kTileBytes;
  auto work = [&](size_t t0, size_t t1) {
    for (size_t t = t0; t < t1; t++) {
      if (t < n_gu) {
        const int b = (int)(t / (2 * G)), rem = (int)(t % (2 * G));
        const float* W = rem < G ? w_gate : w_up;
        pack_tile(W, H, b, rem % G, out + t * kTileBytes, scales + t * kScaleBytes);
      } else {
        const size_t u = t - n_gu;
        pack_tile(w_down, I, (int)(u / GD), (int)(u % GD), out + t * kTileBytes, scales + t * kScaleBytes);
      }
    }
  };
  unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (nt < 256) nth = 1;
  std::vector<std::thread> pool;
  const size_t chunk = (nt + nth - 1) / nth;
  for (unsigned i = 0; i < nth; i++) {
    const size_t a = i * chunk, b = std::min(nt, a + chunk);
    if (a < b) pool.emplace_back(work, a, b);
  }
  for (auto& th : pool) th.join();
  return EXMOE_OK;
}

int exmoe_unpack_expert(const void* packed, size_t packed_bytes_given, int H, int I, int8_t* q_gate,
                        int8_t* q_up, int8_t* q_down, exmoe_bf16* s_gate, exmoe_bf16* s_up,
                        exmoe_bf16* s_down) {
  if (!packed) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "packed must not be NULL");
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "H and I must be positive multiples of 128");
  if (packed_bytes_given < packed_bytes(H, I))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "packed buffer too small");
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  const int G = H / kGroup, GD = I / kGroup;
  const size_t n_gu = 2 * (size_t)(I / kTileRows) * G;
  const size_t nt = n_tiles(H, I);
  const uint8_t* scales = in + nt * kTileBytes;
  for (size_t t = 0; t < nt; t++) {
    int8_t* Q;
    exmoe_bf16* S;
    int K, b, g, SG;
    if (t < n_gu) {
      b = (int)(t / (2 * G));
      const int rem = (int)(t % (2 * G));
      g = rem % G;
      Q = rem < G ? q_gate : q_up;
      S = rem < G ? s_gate : s_up;
      K = H;
      SG = G;
    } else {
      const size_t u = t - n_gu;
      b = (int)(u / GD);
      g = (int)(u % GD);
      Q = q_down;
      S = s_down;
      K = I;
      SG = GD;
    }
    const uint8_t* tp = in + t * kTileBytes;
    for (int l = 0; l < 64; l++)
      for (int s = 0; s < 4; s++) {
        const uint8_t* p = tp + 16 * l + 4 * s;
        const uint32_t w = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
        for (int j = 0; j < 8; j++) {
          const int sh = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);
          const int qv = (int)((w >> sh) & 0xF) - 8;
          const int row = kTileRows * b + l % 16, col = kGroup * g + 32 * s + 8 * (l / 16) + j;
          if (Q) Q[(size_t)row * K + col] = (int8_t)qv;
        }
      }
    if (S)
      for (int r = 0; r < kTileRows; r++) {
        const uint8_t* p = scales + t * kScaleBytes + 2 * r;
        S[(size_t)(kTileRows * b + r) * SG + g] = (exmoe_bf16)(p[0] | (p[1] << 8));
      }
  }
  return EXMOE_OK;
}

size_t exmoe_bf16_expert_bytes(int H, int I) {
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup) return 0;
  return bf16_expert_bytes(H, I);
}

int exmoe_bf16_pack(const exmoe_bf16* w_gate, const exmoe_bf16* w_up, const exmoe_bf16* w_down, int H, int I,
                    void* out, size_t out_bytes) {
  if (!w_gate || !w_up || !w_down || !out)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "weights and output buffer must not be NULL");
  if (H <= 0 || I <= 0 || H % kGroup || I % kGroup)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "H and I must be positive multiples of 128");
  if (out_bytes < bf16_expert_bytes(H, I))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "output buffer too small: %zu < %zu", out_bytes, bf16_expert_bytes(H, I));
  uint16_t* o = static_cast<uint16_t*>(out);
  // one tile: rows 16b.., inputs 32c..; lane l's 8 values are row l % 16, inputs 8 (l / 16) + j
  auto tile = [&](const exmoe_bf16* W, int K, int b, int c, uint16_t* dst) {
    for (int l = 0; l < 64; l++)
      for (int j = 0; j < 8; j++)
        dst[8 * l + j] = W[(size_t)(16 * b + l % 16) * K + 32 * c + 8 * (l / 16) + j];
  };
  const int CH = H / 32, CI = I / 32;
  size_t t = 0;
  for (int b = 0; b < I / kTileRows; b++) {
    for (int c = 0; c < CH; c++) tile(w_gate, H, b, c, o + 512 * t++);
    for (int c = 0; c < CH; c++) tile(w_up, H, b, c, o + 512 * t++);
  }
  for (int b = 0; b < H / kTileRows; b++)
    for (int c = 0; c < CI; c++) tile(w_down, I, b, c, o + 512 * t++);
  return EXMOE_OK;
}

// ------------------------------------------------------------------------------------
// Routing and grouping
// ------------------------------------------------------------------------------------
int exmoe_route_topk(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias, int T, int H,
                     int E, int k, int renormalize, exmoe_bf16* logits, int32_t* topk_ids,
                     float* topk_weights, hipStream_t stream) {
  int st = check_shape(T, H, kGroup, E, k);
  if (st) return st;
  if (T == 0) return EXMOE_OK;
  CHECK_PTR(x);
  CHECK_PTR(w_router);
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  if (logit_bias && ((uintptr_t)logit_bias & 3u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logit_bias must be 4-byte aligned");
  if (logits && ((uintptr_t)logits & 1u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logits must be 2-byte aligned");
  // Logits go to the caller buffer or, when none is given, to the front of the weights
  // buffer is not possible (different sizes): require a logits buffer internally.
  uint16_t* lg = logits;
  void* tmp = nullptr;
  if (!lg) {
    EXMOE_HIP(hipMallocAsync(&tmp, (size_t)T * E * 2, stream));
    lg = static_cast<uint16_t*>(tmp);
  }
  EXMOE_HIP(launch_route_logits(x, w_router, logit_bias, T, H, E, lg, stream));
  EXMOE_HIP(launch_topk(lg, nullptr, T, E, k, renormalize, topk_ids, topk_weights, stream));
  if (tmp) EXMOE_HIP(hipFreeAsync(tmp, stream));
  return EXMOE_OK;
}

int exmoe_topk_from_logits(const exmoe_bf16* logits, int T, int E, int k, int renormalize, int32_t* topk_ids,
                           float* topk_weights, hipStream_t stream) {
  int st = check_shape(T, kGroup, kGroup, E, k);
  if (st) return st;
  if (T == 0) return EXMOE_OK;
  if (!logits || ((uintptr_t)logits & 1u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logits must be non-NULL and 2-byte aligned");
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  EXMOE_HIP(launch_topk(logits, nullptr, T, E, k, renormalize, topk_ids, topk_weights, stream));
  return EXMOE_OK;
}

int exmoe_route_weights(const exmoe_bf16* logits, const int32_t* topk_ids, int T, int E, int k, int renormalize,
                        float* topk_weights, hipStream_t stream) {
  int st = check_shape(T, kGroup, kGroup, E, k);
  if (st) return st;
  if (T == 0) return EXMOE_OK;
  if (!logits || ((uintptr_t)logits & 1u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logits must be non-NULL and 2-byte aligned");
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  EXMOE_HIP(launch_topk(logits, topk_ids, T, E, k, renormalize, nullptr, topk_weights, stream));
  return EXMOE_OK;
}

size_t exmoe_group_workspace_bytes(int T, int k, int E) {
  if (check_shape(T, kGroup, kGroup, E, k)) return 0;
  return group_workspace_bytes(T * k, E);
}

int exmoe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets, int32_t* sorted_flat,
                       int32_t* flat_to_sorted, void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(T, kGroup, kGroup, E, k);
  if (st) return st;
  CHECK_PTR4(expert_offsets);
  if (T > 0) {
    CHECK_PTR4(topk_ids);
    CHECK_PTR4(sorted_flat);
    CHECK_PTR4(flat_to_sorted);
  }
  const size_t need = group_workspace_bytes(T * k, E);
  if (need && (!workspace || ws_bytes < need))
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (need && ((uintptr_t)workspace & 3u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace must be 4-byte aligned");
  EXMOE_HIP(launch_group(topk_ids, T, k, E, expert_offsets, sorted_flat, flat_to_sorted,
                         static_cast<int32_t*>(need ? workspace : nullptr), stream));
  return EXMOE_OK;
}

int exmoe_active_experts(const int32_t* expert_offsets, int E, int32_t* ids_host, int* n_host, hipStream_t stream) {
  if (E < 1 || E > kMaxExperts) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "E must be in [1, 256]");
  CHECK_PTR4(expert_offsets);
  if (!ids_host || !n_host) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "ids_host and n_host must not be NULL");
  int32_t off[kMaxExperts + 1];
  EXMOE_HIP(hipMemcpyAsync(off, expert_offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost, stream));
  EXMOE_HIP(hipStreamSynchronize(stream));
  int n = 0;
  for (int e = 0; e < E; e++)
    if (off[e + 1] > off[e]) ids_host[n++] = e;
  *n_host = n;
  return EXMOE_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------------------
// Expert layer
// ------------------------------------------------------------------------------------
static int choose_path(int T, int H, int I, int E, int k, int flags) {
  const int p = flags & EXMOE_PATH_MASK;
  if (p != EXMOE_PATH_AUTO) return p;
  const long long rows = (long long)T * k;
  const long long act = std::min<long long>(E, rows);
  if (T <= 16) return EXMOE_PATH_DECODE;
  // Routed rows per possibly-active expert at which the grouped GEMM catches up, measured
  // on the OLMoE shape: about 10 against the pass-parallel fused decode kernel (64 tokens:
  // 62 vs 72 us; 96 tokens: 80 vs 76 us under Zipf skew, 88 vs 71 us uniform), about 16
  // for the two-kernel decode path and for the bf16 comparator's decode kernels (one
  // workgroup walks its expert's passes).
  const bool fused = !(flags & EXMOE_WEIGHTS_BF16) && decode_fused_waves(T, H, I, E, k) != 0;
  if (rows <= (fused ? 10 : 16) * act) return EXMOE_PATH_DECODE;
  return EXMOE_PATH_PREFILL;
}

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
// Workspace header: routing arrival counters (one per 256-byte line, so that their atomics
// do not serialize on one cache line), a debug word, and the per-expert row counters of
// EXMOE_FLAG_DEBUG_COUNTERS.
constexpr size_t kWsHeaderBytes = 4096, kWsCounterOffset = 0, kWsDebugOffset = 2048, kWsRowsOffset = 3072;
static_assert(kWsCounterOffset + (size_t)kRouteSelCounters * kRouteCounterStride * 4 <= kWsDebugOffset,
              "counters overlap the debug word");
static_assert(kWsRowsOffset + 4 * (size_t)kMaxExperts <= kWsHeaderBytes && kWsDebugOffset + 4 <= kWsRowsOffset,
              "row counters outside the header");

namespace exmoe {
size_t moe_workspace_layout(int T, int H, int I, int E, int k, int path, MoeArgs* a, void* ws) {
  const size_t rows = (size_t)T * k;
  // the first kWsHeaderBytes are the same in every layout: they hold the routing kernel's
  // arrival counters, which persist (as zeros) from one call to the next
  size_t off = kWsHeaderBytes;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_h = take(rows * I * 2);
  const size_t o_yp = take(rows * H * 4);
  // correction seeds of the prefill kernels: gate/up [group][token], down [group][sorted
  // row] with the rows padded by one tile
  const size_t o_gs = take((rows + 128) * (I / kGroup) * 4);
  const size_t o_xs = take((size_t)T * (H / kGroup) * 4);
  // fused decode: down-projection partial outputs per 128-wide slice of I
  const int fused_waves = path == EXMOE_PATH_DECODE ? decode_fused_waves(T, H, I, E, k) : 0;
  const int nparts = fused_waves ? I / (kTileRows * fused_waves) : 0;
  const size_t o_pt = take((size_t)nparts * rows * H * 4);
  const size_t o_sel = take((size_t)E * 16);
  const size_t o_wt = take((size_t)E * 4);
  const size_t o_gw = take(group_workspace_bytes((int)rows, E));
  if (a && ws) {
    uint8_t* b = static_cast<uint8_t*>(ws);
    a->sel = b + o_sel;
    a->wave_table = reinterpret_cast<int32_t*>(b + o_wt);
    a->group_ws = reinterpret_cast<int32_t*>(b + o_gw);
    a->h = reinterpret_cast<uint16_t*>(b + o_h);
    a->y_perm = reinterpret_cast<float*>(b + o_yp);
    a->gsum = reinterpret_cast<float*>(b + o_gs);
    a->xsum = reinterpret_cast<float*>(b + o_xs);
    a->part = nparts ? reinterpret_cast<float*>(b + o_pt) : nullptr;
    a->nparts = nparts;
    a->counters = reinterpret_cast<uint32_t*>(b + kWsCounterOffset);
    a->debug = reinterpret_cast<uint32_t*>(b + kWsDebugOffset);
    a->rows_ctr = nullptr;   // set by the entry point when EXMOE_FLAG_DEBUG_COUNTERS is given
  }
  return off;
}
}  // namespace exmoe

extern "C" size_t exmoe_moe_workspace_bytes(int T, int H, int I, int E, int k, int flags) {
  if (check_shape(T, H, I, E, k)) return 0;
  return moe_workspace_layout(T, H, I, E, k, choose_path(T, H, I, E, k, flags), nullptr, nullptr);
}

static int check_flags(int flags) {
  const int path = flags & EXMOE_PATH_MASK;
  if (path > EXMOE_PATH_SEQUENTIAL) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "unknown path %d", path);
  if (flags & ~(EXMOE_PATH_MASK | EXMOE_WEIGHTS_BF16 | EXMOE_FLAG_DEBUG_COUNTERS))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "unknown flag bits 0x%x", flags);
  if ((flags & EXMOE_WEIGHTS_BF16) && path == EXMOE_PATH_SEQUENTIAL)
    return set_error(EXMOE_ERR_UNSUPPORTED, "bf16 experts run on the decode and prefill paths only");
  return EXMOE_OK;
}

static int validate_bank(const exmoe_expert_bank* bank, int H, int I, int flags) {
  if (!bank) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bank must not be NULL");
  if (!bank->base || !aligned16(bank->base)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bank->base must be non-NULL and 16-byte aligned");
  if (bank->stride % 16) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bank->stride must be a multiple of 16");
  const size_t eb = (flags & EXMOE_WEIGHTS_BF16) ? bf16_expert_bytes(H, I) : packed_bytes(H, I);
  if (bank->stride < eb)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bank->stride %zu smaller than the expert size %zu", bank->stride, eb);
  if (bank->expert_to_slot && ((uintptr_t)bank->expert_to_slot & 3u))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bank->expert_to_slot must be 4-byte aligned");
  return EXMOE_OK;
}

static void set_row_counters(MoeArgs& a, void* workspace, int flags) {
  a.rows_ctr = (flags & EXMOE_FLAG_DEBUG_COUNTERS)
                   ? reinterpret_cast<int32_t*>(static_cast<uint8_t*>(workspace) + kWsRowsOffset)
                   : nullptr;
}

static int moe_forward_impl(const exmoe_bf16* x, const int32_t* topk_ids, const float* topk_weights,
                            const int32_t* expert_offsets, const int32_t* sorted_flat, const int32_t* flat_to_sorted,
                            const exmoe_expert_bank* bank, int T, int H, int I, int E, int k, int flags, exmoe_bf16* y,
                            void* workspace, size_t ws_bytes, hipStream_t stream, bool xsum_ready = false) {
  const int path = choose_path(T, H, I, E, k, flags);
  MoeArgs a{};
  a.x = x; a.ids = topk_ids; a.w = topk_weights; a.offsets = expert_offsets; a.sorted_flat = sorted_flat;
  a.flat_to_sorted = flat_to_sorted; a.base = static_cast<const uint8_t*>(bank->base); a.stride = bank->stride;
  a.e2s = bank->expert_to_slot; a.T = T; a.H = H; a.I = I; a.E = E; a.k = k; a.y = y;
  moe_workspace_layout(T, H, I, E, k, path, &a, workspace);
  set_row_counters(a, workspace, flags);
  if (flags & EXMOE_WEIGHTS_BF16) {
    a.part = nullptr;   // no sliced partial outputs: y_perm and the plain combine
    a.nparts = 0;
    if (path == EXMOE_PATH_DECODE) EXMOE_HIP(launch_bf16_decode_experts(a, stream));
    else EXMOE_HIP(launch_bf16_prefill_experts(a, stream));
    EXMOE_HIP(launch_combine(a, stream));
  } else if (path == EXMOE_PATH_DECODE) {
    EXMOE_HIP(launch_moe_decode(a, stream));
  } else if (path == EXMOE_PATH_PREFILL) {
    if (!xsum_ready) EXMOE_HIP(launch_moe_prefill_xsum(a, stream));
    EXMOE_HIP(launch_moe_prefill_experts(a, stream));
    EXMOE_HIP(launch_combine(a, stream));
  } else {
    // Sequential W4 reference: experts one after another in ascending id, each with its
    // own launches over its gathered rows; one host read of the offsets drives the loop.
    // Up to 16 rows, an expert runs on a launch pair built for a short latency chain;
    // more rows go through the decode kernel pair, which walks them in passes of 16 inside
    // one launch pair.
    int32_t off[kMaxExperts + 1];
    EXMOE_HIP(hipMemcpyAsync(off, expert_offsets, sizeof(int32_t) * (E + 1), hipMemcpyDeviceToHost, stream));
    EXMOE_HIP(hipStreamSynchronize(stream));
    for (int e = 0; e < E; e++) {
      const int cnt = off[e + 1] - off[e];
      if (cnt <= 0) continue;
      if (cnt <= kSeqMaxRows) EXMOE_HIP(launch_seq_expert(a, e, off[e], cnt, stream));
      else EXMOE_HIP(launch_moe_expert_range(a, e, cnt, stream));
    }
    EXMOE_HIP(launch_combine(a, stream));
  }
  return EXMOE_OK;
}

extern "C" {

int exmoe_moe_forward(const exmoe_bf16* x, const int32_t* topk_ids, const float* topk_weights,
                      const int32_t* expert_offsets, const int32_t* sorted_flat, const int32_t* flat_to_sorted,
                      const exmoe_expert_bank* bank, int T, int H, int I, int E, int k, int flags, exmoe_bf16* y,
                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(T, H, I, E, k);
  if (st) return st;
  if ((st = check_flags(flags))) return st;
  if ((st = validate_bank(bank, H, I, flags))) return st;
  if (T == 0) return EXMOE_OK;
  CHECK_PTR(x);
  CHECK_PTR(y);
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  CHECK_PTR4(expert_offsets);
  CHECK_PTR4(sorted_flat);
  CHECK_PTR4(flat_to_sorted);
  const size_t need = moe_workspace_layout(T, H, I, E, k, choose_path(T, H, I, E, k, flags), nullptr, nullptr);
  if (!workspace || ws_bytes < need)
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (((uintptr_t)workspace) & 255u) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  return moe_forward_impl(x, topk_ids, topk_weights, expert_offsets, sorted_flat, flat_to_sorted, bank, T, H, I, E,
                          k, flags, y, workspace, ws_bytes, stream);
}

int exmoe_moe_forward_cached(const exmoe_bf16* x, const int32_t* topk_ids, const float* topk_weights,
                             const int32_t* expert_offsets, const int32_t* sorted_flat, const int32_t* flat_to_sorted,
                             exmoe_slot_cache* cache, int layer, const int32_t* active_ids_host, int n_active, int T,
                             int H, int I, int E, int k, int flags, exmoe_bf16* y, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  int st = check_shape(T, H, I, E, k);
  if (st) return st;
  if ((st = check_flags(flags))) return st;
  if (!cache) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache must not be NULL");
  int cE = 0, cS = 0, dry = 0;
  size_t cB = 0;
  slot_cache_shape(cache, &cE, &cS, &dry, &cB);
  if (dry) return set_error(EXMOE_ERR_CACHE, "a dry-run cache holds no weights");
  if (cE != E) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache has %d experts per layer, the layer %d", cE, E);
  const size_t eb = (flags & EXMOE_WEIGHTS_BF16) ? bf16_expert_bytes(H, I) : packed_bytes(H, I);
  if (cB < eb) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache holds %zu bytes per expert, %zu needed", cB, eb);
  if (n_active < 0 || (n_active > 0 && !active_ids_host))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bad active list");
  std::vector<int32_t> A(active_ids_host, active_ids_host + n_active);
  for (int e : A)
    if (e < 0 || e >= E) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "expert id %d out of range", e);
  const int path = choose_path(T, H, I, E, k, flags);
  if (path == EXMOE_PATH_SEQUENTIAL) return set_error(EXMOE_ERR_UNSUPPORTED, "the sequential path does not run in waves");
  if (T == 0) return EXMOE_OK;
  CHECK_PTR(x);
  CHECK_PTR(y);
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  CHECK_PTR4(expert_offsets);
  CHECK_PTR4(sorted_flat);
  CHECK_PTR4(flat_to_sorted);
  const size_t need = moe_workspace_layout(T, H, I, E, k, path, nullptr, nullptr);
  if (!workspace || ws_bytes < need)
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (((uintptr_t)workspace) & 255u) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  MoeArgs a{};
  a.x = x; a.ids = topk_ids; a.w = topk_weights; a.offsets = expert_offsets; a.sorted_flat = sorted_flat;
  a.flat_to_sorted = flat_to_sorted; a.T = T; a.H = H; a.I = I; a.E = E; a.k = k; a.y = y;
  moe_workspace_layout(T, H, I, E, k, path, &a, workspace);
  set_row_counters(a, workspace, flags);
  const bool bf16w = (flags & EXMOE_WEIGHTS_BF16) != 0;
  if (bf16w) {
    a.part = nullptr;
    a.nparts = 0;
  }
  if (path == EXMOE_PATH_PREFILL && !bf16w) EXMOE_HIP(launch_moe_prefill_xsum(a, stream));
  // Waves: the active experts already resident first, then the others, each in ascending
  // id (a repeated active set larger than the cache then hits S times instead of
  // thrashing the LRU). An active set that fits is one wave; a larger one runs in waves of
  // S/2, so the misses of wave w+1 never evict an expert of wave w (the LRU victims are the
  // S - |wave w| - hits >= |misses| older residents) and its copies overlap wave w's
  // kernels: they wait only for wave w-1's. Per wave: acquire (misses copied), then the
  // expert kernels with a table that maps only this wave's experts; the rows of the other
  // experts are left alone (skipped silently) and written by their own wave.
  if (layer < 0 || layer >= slot_cache_layers(cache)) return set_error(EXMOE_ERR_CACHE, "layer %d out of range", layer);
  std::vector<int32_t> tbl(E), wave_tbl(E);
  const int W = slot_cache_plan_waves(cache, layer, A);
  const int n_waves = ((int)A.size() + W - 1) / W;
  // The layer's slots were last read by the kernels behind the layer's mark, when the cache
  // knows it: the copies of waves 0 and 1 then wait only for those and overlap the kernels
  // of other layers still in flight (without it, for all earlier work on the stream). The
  // mark is dropped while this call enqueues (a failure part-way leaves it unknown) and
  // recorded again after the last wave.
  hipEvent_t prior = slot_cache_layer_mark(cache, layer);
  slot_cache_forget_layer(cache, layer);
  std::vector<int32_t> prev_slots;
  hipEvent_t mark = nullptr, start = prior;
  if (n_waves > 1 && !prior) {
    EXMOE_HIP(slot_cache_event(cache, 0, &mark));
    EXMOE_HIP(hipEventRecord(mark, stream));   // everything before this call
    start = mark;
  }
  for (int w = 0; w < n_waves; w++) {
    const int w0 = w * W;
    const int n = std::min((int)A.size() - w0, W);
    exmoe_expert_bank bank{};
    hipEvent_t after = prior;     // wave 0: the layer's last readers (null: all earlier work)
    if (w == 1) after = start;
    if (w >= 2) EXMOE_HIP(slot_cache_event(cache, w - 1, &after));   // done through wave w-2
    if ((st = slot_cache_acquire_ex(cache, layer, A.data() + w0, n, stream, after, prev_slots.data(),
                                    (int)prev_slots.size(), &bank)))
      return st;
    a.base = static_cast<const uint8_t*>(bank.base);
    a.stride = bank.stride;
    if (n_waves == 1) {
      // every listed expert is resident now: the layer's own table serves, and a routed
      // expert without a slot is flagged in the debug word
      a.e2s = static_cast<const int32_t*>(bank.expert_to_slot);
      a.skip_absent = 0;
    } else {
      if ((st = exmoe_slot_cache_table(cache, layer, tbl.data()))) return st;
      std::fill(wave_tbl.begin(), wave_tbl.end(), -1);
      prev_slots.clear();
      for (int i = 0; i < n; i++) {
        wave_tbl[A[w0 + i]] = tbl[A[w0 + i]];
        prev_slots.push_back(tbl[A[w0 + i]]);
      }
      // by value in the kernel arguments (no staging, no wait on the host), ordered after
      // the previous wave's kernels on the same stream
      EXMOE_HIP(table_upload(a.wave_table, wave_tbl.data(), E, stream));
      a.e2s = a.wave_table;
      a.skip_absent = 1;
    }
    if (bf16w) {
      if (path == EXMOE_PATH_DECODE) EXMOE_HIP(launch_bf16_decode_experts(a, stream));
      else EXMOE_HIP(launch_bf16_prefill_experts(a, stream));
    } else if (path == EXMOE_PATH_DECODE) {
      EXMOE_HIP(launch_moe_decode_experts(a, stream));
    } else {
      EXMOE_HIP(launch_moe_prefill_experts(a, stream));
    }
    if (w + 2 < n_waves) {   // the mark that wave w+2's copies wait for
      EXMOE_HIP(slot_cache_event(cache, w + 1, &mark));
      EXMOE_HIP(hipEventRecord(mark, stream));
    }
  }
  EXMOE_HIP(slot_cache_mark_layer(cache, layer, stream));
  if (n_waves > 1) {
    // each wave skipped the experts outside it silently: an expert with rows that no wave
    // held (missing from the caller's list) is flagged here
    uint32_t mask[kMaxExperts / 32] = {};
    for (int e : A) mask[e >> 5] |= 1u << (e & 31);
    EXMOE_HIP(check_wave_union(expert_offsets, E, mask, a.debug, stream));
  }
  EXMOE_HIP(launch_combine(a, stream));
  return EXMOE_OK;
}

int exmoe_workspace_flags(void* workspace, size_t ws_bytes, int clear, uint32_t* flags_out, hipStream_t stream) {
  if (!workspace || !flags_out) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace and flags_out must not be NULL");
  if (ws_bytes < kWsHeaderBytes)
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes has no %zu-byte header", ws_bytes, kWsHeaderBytes);
  uint8_t* word = static_cast<uint8_t*>(workspace) + kWsDebugOffset;
  uint32_t v = 0;
  EXMOE_HIP(hipMemcpyAsync(&v, word, sizeof(v), hipMemcpyDeviceToHost, stream));
  EXMOE_HIP(hipStreamSynchronize(stream));
  *flags_out = v;
  if (clear && v) {
    const uint32_t zero = 0;
    EXMOE_HIP(hipMemcpyAsync(word, &zero, sizeof(zero), hipMemcpyHostToDevice, stream));
    EXMOE_HIP(hipStreamSynchronize(stream));
  }
  return EXMOE_OK;
}

int exmoe_workspace_rows(void* workspace, size_t ws_bytes, int E, int clear, int32_t* rows_out, hipStream_t stream) {
  if (!workspace || !rows_out) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace and rows_out must not be NULL");
  if (E < 1 || E > kMaxExperts) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "E must be in [1, 256]");
  if (ws_bytes < kWsHeaderBytes)
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes has no %zu-byte header", ws_bytes, kWsHeaderBytes);
  uint8_t* rows = static_cast<uint8_t*>(workspace) + kWsRowsOffset;
  EXMOE_HIP(hipMemcpyAsync(rows_out, rows, sizeof(int32_t) * E, hipMemcpyDeviceToHost, stream));
  EXMOE_HIP(hipStreamSynchronize(stream));
  if (clear) {
    static const int32_t zeros[kMaxExperts] = {};
    EXMOE_HIP(hipMemcpyAsync(rows, zeros, sizeof(int32_t) * E, hipMemcpyHostToDevice, stream));
    EXMOE_HIP(hipStreamSynchronize(stream));
  }
  return EXMOE_OK;
}

size_t exmoe_moe_layer_workspace_bytes(int T, int H, int I, int E, int k, int flags) {
  return exmoe_moe_workspace_bytes(T, H, I, E, k, flags);
}

int exmoe_moe_layer(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias,
                    const exmoe_expert_bank* bank, int T, int H, int I, int E, int k, int renormalize, int flags,
                    exmoe_bf16* logits, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                    int32_t* sorted_flat, int32_t* flat_to_sorted, exmoe_bf16* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream) {
  int st = check_shape(T, H, I, E, k);
  if (st) return st;
  if ((st = check_flags(flags))) return st;
  if ((st = validate_bank(bank, H, I, flags))) return st;
  CHECK_PTR4(expert_offsets);
  if (T == 0) return exmoe_group_tokens(topk_ids, 0, k, E, expert_offsets, sorted_flat, flat_to_sorted, nullptr, 0, stream);
  CHECK_PTR(x);
  CHECK_PTR(w_router);
  CHECK_PTR(y);
  if (!logits || ((uintptr_t)logits & 1u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logits must be non-NULL and 2-byte aligned");
  CHECK_PTR4(topk_ids);
  CHECK_PTR4(topk_weights);
  CHECK_PTR4(sorted_flat);
  CHECK_PTR4(flat_to_sorted);
  if (logit_bias && ((uintptr_t)logit_bias & 3u)) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "logit_bias must be 4-byte aligned");
  const size_t need = moe_workspace_layout(T, H, I, E, k, choose_path(T, H, I, E, k, flags), nullptr, nullptr);
  if (!workspace || ws_bytes < need)
    return set_error(EXMOE_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : 0);
  if (((uintptr_t)workspace) & 255u) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (!(flags & EXMOE_WEIGHTS_BF16) && choose_path(T, H, I, E, k, flags) == EXMOE_PATH_DECODE &&
      (long long)T * k <= kDecMaxRows) {
    // Decode sizes: the expert kernel groups the rows itself and publishes the grouping;
    // for a few tokens and E <= 64 it also makes the top-k selection from the logits (for
    // larger E the routing kernel makes it and writes a per-expert token table), otherwise
    // one workgroup per token routes it first.
    MoeArgs a{};
    a.x = x; a.ids = topk_ids; a.w = topk_weights; a.offsets = expert_offsets; a.sorted_flat = sorted_flat;
    a.flat_to_sorted = flat_to_sorted; a.base = static_cast<const uint8_t*>(bank->base); a.stride = bank->stride;
    a.e2s = bank->expert_to_slot; a.T = T; a.H = H; a.I = I; a.E = E; a.k = k; a.y = y;
    moe_workspace_layout(T, H, I, E, k, EXMOE_PATH_DECODE, &a, workspace);
    set_row_counters(a, workspace, flags);
    if (decode_logit_routing_ok(T, H, I, E, k)) {
      // the logits only; every expert workgroup makes the top-k selection from them
      EXMOE_HIP(launch_route_logits(x, w_router, logit_bias, T, H, E, logits, stream));
      EXMOE_HIP(launch_moe_decode_logit_routed(a, logits, renormalize, topk_ids, topk_weights, expert_offsets,
                                               sorted_flat, flat_to_sorted, stream));
    } else if (decode_table_routing_ok(T, H, E, k)) {
      EXMOE_HIP(launch_route_sel(x, w_router, logit_bias, T, H, E, k, renormalize, logits, topk_ids, topk_weights,
                                 a.sel, a.counters, stream));
      EXMOE_HIP(launch_moe_decode_routed(a, a.sel, expert_offsets, sorted_flat, flat_to_sorted, stream));
    } else {
      EXMOE_HIP(launch_route_token(x, w_router, logit_bias, T, H, E, k, renormalize, logits, topk_ids,
                                   topk_weights, stream));
      EXMOE_HIP(launch_moe_decode_routed(a, nullptr, expert_offsets, sorted_flat, flat_to_sorted, stream));
    }
    return EXMOE_OK;
  }
  MoeArgs ag{};
  const int path = choose_path(T, H, I, E, k, flags);
  moe_workspace_layout(T, H, I, E, k, path, &ag, workspace);
  // the grouped GEMM's correction seeds come with the logits (the routing kernel loads x)
  const bool xs = path == EXMOE_PATH_PREFILL && !(flags & EXMOE_WEIGHTS_BF16) && H <= kLgtXsMaxH;
  EXMOE_HIP(launch_route_logits(x, w_router, logit_bias, T, H, E, logits, stream, xs ? ag.xsum : nullptr));
  EXMOE_HIP(launch_topk_group(logits, T, E, k, renormalize, topk_ids, topk_weights, expert_offsets, sorted_flat,
                              flat_to_sorted, ag.group_ws, stream));
  return moe_forward_impl(x, topk_ids, topk_weights, expert_offsets, sorted_flat, flat_to_sorted, bank, T, H, I, E,
                          k, flags, y, workspace, ws_bytes, stream, xs);
}

}  // extern "C"
