// Decode-sized expert layer (a few tokens per expert), gfx950.
//
// Every selected expert runs (ExactMoE abstract; Fig. 1). With a handful of tokens per
// expert the layer is bound by streaming the packed int4 weights from HBM, so these
// kernels are laid out for bandwidth and short dependency chains:
//  * a workgroup owns one active expert and a slice of output rows; each wave streams
//    whole 1 KiB tiles (one wave-wide 128-bit load each) in chunks of two 128-input
//    groups, double-buffered in registers, with the activation fragments of the same
//    groups issued alongside, so loads stay in flight while the previous chunk computes;
//  * the tokens of the expert (padded to 16) ride in the N dimension of
//    v_mfma_f32_16x16x32_bf16; more than 16 tokens loop over 16-token tiles;
//  * when few workgroups would exist (batch-1 decode), the four waves split the
//    reduction dimension instead of the rows and add their partial sums through LDS.
// Dequantization is exact: a packed word becomes bf16 operands 128 + u (u = q + 8) with
// two bitwise ops per pair; an MFMA chain of the constant -136 against the same
// activation fragments seeds each group's accumulator with -136 * sum(x), so each group
// chain ends at sum(x * q); the bf16 row scale is applied once per group in fp32.
//
// Kernel 1 (gate/up): h = bf16(silu(W_gate x) * (W_up x)). In the whole-layer call it
//   also redoes the top-k selection and grouping of the (few) tokens from the bf16 logits
//   in every workgroup -- a microsecond of ALU instead of another launch -- and
//   workgroup (0, 0) publishes that routing for the following kernels.
// Kernel 2 (down): o = W_down h, times the routing weight, into y_perm (fp32).
// Kernel 3 (combine): y[t] = bf16(sum over slots j in order of y_perm[row(t, j)]).
// Workgroups never wait on each other: a device-scope release costs a serialized L2
// write-back on this chip, far more than a kernel boundary inside a graph.
#include "common.h"
#include "device.h"
#include "group_block.h"
#include "topk.h"

namespace exmoe {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / 64;
// Below this many (expert, 16-row block) items the four waves of a workgroup share one
// item and split its reduction dimension (more waves in flight for batch-1 decode).
constexpr int kDecSplitBelow = 1024;

struct Frag4 {
  bf16x8 s[4];
};

// -136 * (sum of the group's activations) in the C layout (lane l: token l % 16).
__device__ __forceinline__ f32x4 corr_chain(const Frag4& act) {
  const bf16x8 n136 = neg136_operand();
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; s++) c = mfma16(n136, act.s[s], c);
  return c;
}

// sum_k x_k q_k over one tile for rows 4(l/16)+i, token l%16.
__device__ __forceinline__ f32x4 tile_chain(uint4 words, const Frag4& act, f32x4 corr) {
  f32x4 c = corr;
  c = mfma16(dequant_word(words.x), act.s[0], c);
  c = mfma16(dequant_word(words.y), act.s[1], c);
  c = mfma16(dequant_word(words.z), act.s[2], c);
  c = mfma16(dequant_word(words.w), act.s[3], c);
  return c;
}

// Routing state shared by a workgroup.
constexpr int kDecMaxRows = 1024;   // T*k routed rows handled by the in-kernel routing
struct DecShared {
  int32_t offsets[kMaxExperts + 1];
  int32_t act[kMaxExperts];
  int32_t n_act;
};
struct DecFusedShared {          // only in the variant that redoes the routing
  int32_t ids[kDecMaxRows];
  float w[kDecMaxRows];
  int32_t sorted[kDecMaxRows];
  int32_t f2s[kDecMaxRows];
  GroupSharedT<kDecThreads> gs;
};

template <bool F>
struct FusedSlot {
  DecFusedShared v;
  __device__ DecFusedShared* ptr() { return &v; }
};
template <>
struct FusedSlot<false> {
  int unused;
  __device__ DecFusedShared* ptr() { return nullptr; }
};

struct DecRoute {
  const uint16_t* logits;   // non-NULL: recompute top-k + grouping in every workgroup
  int renormalize;
  int32_t* ids_out;         // published by workgroup (0, 0)
  float* w_out;
  int32_t* offsets_out;
  int32_t* sorted_out;
  int32_t* f2s_out;
};

// Fills sh.offsets / sh.act / sh.n_act (and, in fused mode, the routing arrays). Returns
// the sorted_flat pointer to use (LDS copy in fused mode, caller's array otherwise).
__device__ const int32_t* dec_routing(const MoeArgs& a, const DecRoute& rt, int fixed_expert, DecShared& sh,
                                     DecFusedShared* fs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* sorted = a.sorted_flat;
  if (fs) {
    DecFusedShared& f = *fs;
    for (int t = wave; t < a.T; t += kDecWaves) {
      int id;
      float wt;
      topk_token(rt.logits + (size_t)t * a.E, nullptr, a.E, a.k, rt.renormalize, id, wt);
      if (lane < a.k) {
        f.ids[t * a.k + lane] = id;
        f.w[t * a.k + lane] = wt;
      }
    }
    __syncthreads();
    group_block<kDecThreads>(f.ids, a.T * a.k, a.E, sh.offsets, f.sorted, f.f2s, f.gs);
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0) {
      const int n = a.T * a.k;
      for (int i = tid; i < n; i += kDecThreads) {
        rt.ids_out[i] = f.ids[i];
        rt.w_out[i] = f.w[i];
        rt.sorted_out[i] = f.sorted[i];
        rt.f2s_out[i] = f.f2s[i];
      }
      for (int i = tid; i <= a.E; i += kDecThreads) rt.offsets_out[i] = sh.offsets[i];
    }
    sorted = f.sorted;
  } else {
    for (int i = tid; i <= a.E; i += kDecThreads) sh.offsets[i] = a.offsets[i];
    __syncthreads();
  }
  if (wave == 0) {
    if (fixed_expert >= 0) {
      if (lane == 0) {
        sh.act[0] = fixed_expert;
        sh.n_act = 1;
      }
    } else {
      int base = 0;
      for (int c0 = 0; c0 < a.E; c0 += 64) {
        const int e = c0 + lane;
        const bool on = e < a.E && sh.offsets[e + 1] > sh.offsets[e];
        const uint64_t m = __ballot(on);
        if (on) sh.act[base + __popcll(m & ((1ull << lane) - 1ull))] = e;
        base += __popcll(m);
      }
      if (lane == 0) sh.n_act = base;
    }
  }
  __syncthreads();
  return sorted;
}

struct ExpertRef {
  int e, seg0, cnt;
  const uint4* tiles;
  const uint16_t* scales;
};

__device__ __forceinline__ bool dec_expert(const MoeArgs& a, const DecShared& sh, int idx, ExpertRef& r) {
  if (idx >= sh.n_act) return false;
  r.e = sh.act[idx];
  r.seg0 = sh.offsets[r.e];
  r.cnt = sh.offsets[r.e + 1] - r.seg0;
  if (r.cnt <= 0) return false;
  const int slot = a.e2s ? a.e2s[r.e] : r.e;
  if (slot < 0) {
    if (threadIdx.x == 0) atomicOr(a.debug, 1u);   // routed expert without a slot
    return false;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  r.tiles = reinterpret_cast<const uint4*>(blob);
  r.scales = reinterpret_cast<const uint16_t*>(blob + n_tiles(a.H, a.I) * kTileBytes);
  return true;
}

// ------------------------------------------------------------------------------------
// Streaming core. One wave owns one (expert, 16-row block) item and walks its 128-input
// groups g = g0, g0 + gstep, ...: NM packed tiles per group (2 = gate and up, 1 = down)
// with their scales from HBM, kept kWRing groups ahead in registers, and the activation
// fragments of the same groups from L2 (the expert's token rows; padding lanes read the
// zero row), kept kXRing groups ahead. Loads are unconditional (indices past the end
// repeat the last group), so the compiler can count them and keep them in flight.
// ------------------------------------------------------------------------------------
constexpr int kWRing = 4;
constexpr int kXRing = 2;
template <int NM>
struct WSlot {
  uint4 w[NM];
  uint2 s[NM];
};

// Padding token slots read this all-zero row (device globals start zeroed; never written).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row[kMaxDim];

__device__ __forceinline__ Frag4 load_act(const uint16_t* row_ptr, int col0) {
  Frag4 f;
  const int lane = (int)lane_id();
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const uint4 u = *reinterpret_cast<const uint4*>(row_ptr + col0 + 32 * s + 8 * (lane >> 4));
    i32x4 v = {(int)u.x, (int)u.y, (int)u.z, (int)u.w};
    f.s[s] = __builtin_bit_cast(bf16x8, v);
  }
  return f;
}

template <int NM, typename F>
__device__ __forceinline__ void stream_groups(const uint4* tiles, const uint16_t* scales, const size_t* tbase,
                                              int g0, int gstep, int ngroups, const uint16_t* xrow, F&& consume) {
  const int lane = (int)lane_id();
  auto gidx = [&](int i) { return g0 + (i < ngroups ? i : ngroups - 1) * gstep; };
  auto issue_w = [&](int i, WSlot<NM>& w) {
    const int g = gidx(i);
#pragma unroll
    for (int m = 0; m < NM; m++) {
      const size_t t = tbase[m] + g;
      w.w[m] = tiles[t * 64 + lane];
      w.s[m] = *reinterpret_cast<const uint2*>(scales + t * 16 + 4 * (lane >> 4));
    }
  };
  WSlot<NM> W[kWRing];
  Frag4 X[kXRing];
#pragma unroll
  for (int j = 0; j < kWRing; j++) issue_w(j, W[j]);
#pragma unroll
  for (int j = 0; j < kXRing; j++) X[j] = load_act(xrow, gidx(j) * kGroup);
  for (int i0 = 0; i0 < ngroups; i0 += kWRing) {
#pragma unroll
    for (int j = 0; j < kWRing; j++) {
      if (i0 + j < ngroups) consume(W[j], X[j % kXRing]);
      issue_w(i0 + j + kWRing, W[j]);
      X[j % kXRing] = load_act(xrow, gidx(i0 + j + kXRing) * kGroup);
    }
  }
}

// ------------------------------------------------------------------------------------
// gate/up + SiLU*up.  KSPLIT = 1: each wave owns its own item (expert, row block).
//                     KSPLIT = 4: the 4 waves of a workgroup share one item and split its
//                     groups (g = wave mod 4), adding partial sums through LDS.
// ------------------------------------------------------------------------------------
template <int KSPLIT, bool FUSED>
__global__ __launch_bounds__(kDecThreads) void decode_gateup_kernel(MoeArgs a, DecRoute rt, int fixed_expert) {
  __shared__ DecShared sh;
  __shared__ FusedSlot<FUSED> fsh;
  __shared__ f32x4 red[KSPLIT > 1 ? kDecWaves : 1][2][64];
  const int lane = (int)lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t* sorted = dec_routing(a, rt, fixed_expert, sh, fsh.ptr());
  const int nrb = a.I / kTileRows;
  const int item = KSPLIT == 1 ? (int)blockIdx.x * kDecWaves + wave : (int)blockIdx.x;
  ExpertRef ex;
  if (!dec_expert(a, sh, item / nrb, ex)) return;       // uniform per wave (KSPLIT 1) or workgroup
  const int rb = item % nrb;
  const int G = a.H / kGroup;
  const int g0 = KSPLIT == 1 ? 0 : wave;
  const int ngroups = (G - g0 + KSPLIT - 1) / KSPLIT;
  const size_t tbase[2] = {(size_t)(rb * 2) * G, (size_t)(rb * 2 + 1) * G};
  const int n = lane & 15;
  const int ntt = (ex.cnt + 15) / 16;

  for (int tt = 0; tt < ntt; tt++) {
    const int r = tt * 16 + n;
    const bool valid = r < ex.cnt;
    const uint16_t* xrow = valid ? a.x + (size_t)(sorted[ex.seg0 + r] / a.k) * a.H : g_zero_row;
    f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
    if (ngroups > 0)
      stream_groups<2>(ex.tiles, ex.scales, tbase, g0, KSPLIT, ngroups, xrow,
                       [&](const WSlot<2>& w, const Frag4& act) {
                         const f32x4 corr = corr_chain(act);
                         scale_accum(accg, tile_chain(w.w[0], act, corr), w.s[0]);
                         scale_accum(accu, tile_chain(w.w[1], act, corr), w.s[1]);
                       });
    if (KSPLIT > 1) {
      red[wave][0][lane] = accg;
      red[wave][1][lane] = accu;
      __syncthreads();
      if (wave == 0)
        for (int w = 1; w < kDecWaves; w++) {
          accg += red[w][0][lane];
          accu += red[w][1][lane];
        }
    }
    if ((KSPLIT == 1 || wave == 0) && valid) {
      uint16_t hb[4];
#pragma unroll
      for (int i = 0; i < 4; i++) hb[i] = f32_to_bf16(accg[i] / (1.0f + expf(-accg[i])) * accu[i]);
      uint2 pk;
      pk.x = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
      pk.y = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
      *reinterpret_cast<uint2*>(a.h + (size_t)(ex.seg0 + r) * a.I + rb * 16 + 4 * (lane >> 4)) = pk;
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// down (+ routing weight) into y_perm, in flat (token, slot) order so that the combine
// reads it without an index. Same two layouts as gate/up, rows of H.
// ------------------------------------------------------------------------------------
template <int KSPLIT>
__global__ __launch_bounds__(kDecThreads) void decode_down_kernel(MoeArgs a, int fixed_expert) {
  __shared__ DecShared sh;
  __shared__ f32x4 red[KSPLIT > 1 ? kDecWaves : 1][64];
  const int lane = (int)lane_id(), wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  DecRoute none{};
  const int32_t* sorted = dec_routing(a, none, fixed_expert, sh, nullptr);
  const int nrb = a.H / kTileRows;
  const int item = KSPLIT == 1 ? (int)blockIdx.x * kDecWaves + wave : (int)blockIdx.x;
  ExpertRef ex;
  if (!dec_expert(a, sh, item / nrb, ex)) return;
  const int rb = item % nrb;
  const int G = a.I / kGroup;
  const int g0 = KSPLIT == 1 ? 0 : wave;
  const int ngroups = (G - g0 + KSPLIT - 1) / KSPLIT;
  const size_t tbase[1] = {2 * (size_t)(a.I / kTileRows) * (a.H / kGroup) + (size_t)rb * G};
  const int n = lane & 15;
  const int ntt = (ex.cnt + 15) / 16;

  for (int tt = 0; tt < ntt; tt++) {
    const int r = tt * 16 + n;
    const bool valid = r < ex.cnt;
    const uint16_t* hrow = valid ? a.h + (size_t)(ex.seg0 + r) * a.I : g_zero_row;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (ngroups > 0)
      stream_groups<1>(ex.tiles, ex.scales, tbase, g0, KSPLIT, ngroups, hrow,
                       [&](const WSlot<1>& w, const Frag4& act) {
                         scale_accum(acc, tile_chain(w.w[0], act, corr_chain(act)), w.s[0]);
                       });
    if (KSPLIT > 1) {
      red[wave][lane] = acc;
      __syncthreads();
      if (wave == 0)
        for (int w = 1; w < kDecWaves; w++) acc += red[w][lane];
    }
    if ((KSPLIT == 1 || wave == 0) && valid) {
      const int f = sorted[ex.seg0 + r];
      const float wt = a.w[f];
      *reinterpret_cast<float4*>(a.y_perm + (size_t)f * a.H + rb * 16 + 4 * (lane >> 4)) =
          make_float4(acc[0] * wt, acc[1] * wt, acc[2] * wt, acc[3] * wt);
    }
    if (KSPLIT > 1) __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// combine: y[t, rows] = bf16(sum_j y_perm[t k + j, rows]) in slot order
// ------------------------------------------------------------------------------------
constexpr int kCombineTok = 16;
__global__ __launch_bounds__(256) void combine_kernel(MoeArgs a) {
  const int t0 = blockIdx.y * kCombineTok;
  const int t1 = t0 + kCombineTok < a.T ? t0 + kCombineTok : a.T;
  const int row0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < (t1 - t0) * 16; i += blockDim.x) {
    const int t = t0 + i / 16, c = row0 + (i % 16) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; j++) {
      const float4 v = *reinterpret_cast<const float4*>(a.y_perm + ((size_t)t * a.k + j) * a.H + c);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
    *reinterpret_cast<uint2*>(a.y + (size_t)t * a.H + c) = pk;
  }
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
static hipError_t launch_decode_experts(const MoeArgs& a, const DecRoute& rt, int fixed_expert, int ny,
                                        hipStream_t s) {
  // ny = upper bound of active experts; items = (active expert, 16-row block)
  const int items_gu = ny * (a.I / kTileRows);
  {
    ProfScope prof("decode_gateup", s);
    const dim3 g1((items_gu + kDecWaves - 1) / kDecWaves), g4(items_gu);
    const bool split = items_gu < kDecSplitBelow;
    if (rt.logits) {
      if (!split)
        EXMOE_LAUNCH(prof, (decode_gateup_kernel<1, true>), g1, dim3(kDecThreads), 0, s, a, rt, fixed_expert);
      else
        EXMOE_LAUNCH(prof, (decode_gateup_kernel<4, true>), g4, dim3(kDecThreads), 0, s, a, rt, fixed_expert);
    } else {
      if (!split)
        EXMOE_LAUNCH(prof, (decode_gateup_kernel<1, false>), g1, dim3(kDecThreads), 0, s, a, rt, fixed_expert);
      else
        EXMOE_LAUNCH(prof, (decode_gateup_kernel<4, false>), g4, dim3(kDecThreads), 0, s, a, rt, fixed_expert);
    }
  }
  const int items_d = ny * (a.H / kTileRows);
  {
    ProfScope prof("decode_down", s);
    if (items_d >= kDecSplitBelow)
      EXMOE_LAUNCH(prof, decode_down_kernel<1>, dim3((items_d + kDecWaves - 1) / kDecWaves), dim3(kDecThreads), 0,
                         s, a, fixed_expert);
    else
      EXMOE_LAUNCH(prof, decode_down_kernel<4>, dim3(items_d), dim3(kDecThreads), 0, s, a, fixed_expert);
  }
  return hipGetLastError();
}

hipError_t launch_moe_decode(const MoeArgs& a, hipStream_t s) {
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  DecRoute none{};
  hipError_t e = launch_decode_experts(a, none, -1, ny, s);
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

// Redoing the routing in every gate/up workgroup beats a separate top-k launch only when
// there are very few tokens (measured: batch 1 and 2).
bool decode_fused_routing_ok(int T, int k) { return T <= 2 && T * k <= kDecMaxRows; }

hipError_t launch_moe_decode_fused(const MoeArgs& a, const uint16_t* logits, int renormalize, int32_t* ids,
                                   float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                                   hipStream_t s) {
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  DecRoute rt{logits, renormalize, ids, w, offsets, sorted_flat, flat_to_sorted};
  hipError_t e = launch_decode_experts(a, rt, -1, ny, s);
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

hipError_t launch_moe_expert_range(const MoeArgs& a, int expert, int rows, hipStream_t s) {
  (void)rows;
  DecRoute none{};
  return launch_decode_experts(a, none, expert, 1, s);
}

hipError_t launch_combine(const MoeArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  ProfScope prof("combine", s);
  EXMOE_LAUNCH(prof, combine_kernel, dim3(a.H / 64, (a.T + kCombineTok - 1) / kCombineTok), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace exmoe
