// Decode-sized expert layer (few tokens per expert), gfx950.
//
// Every selected expert runs (ExactMoE abstract; Fig. 1). With a handful of tokens per
// expert the layer is bound by streaming the packed int4 weights from HBM, so these
// kernels are laid out for bandwidth: each workgroup owns one active expert and a slice
// of output rows, its four waves split the reduction dimension, every lane issues all of
// its 128-bit weight loads up front (whole 1 KiB tiles per wave instruction), and the
// tokens of the expert (padded to 16) ride in the N dimension of v_mfma_f32_16x16x32_bf16.
//
// Dequantization is exact: a packed word becomes bf16 values 128 + u (u = q + 8) with two
// bitwise ops per pair, and an MFMA chain of the constant -136 against the same activation
// fragments seeds each group's accumulator with -136 * sum(x), so the group's chain ends
// at sum(x * q) exactly up to fp32 accumulation; the bf16 group scale is applied once per
// group in fp32.
//
// Kernel 1 (gate/up): h = bf16(silu(W_gate x) * (W_up x)) for 16 rows per row block.
// Kernel 2 (down): o = W_down h, times the routing weight, into y_perm (fp32); the last
// workgroup to finish a row slice (an agent-scope counter) sums the k slots of every
// token in slot order into y (bf16), so no extra combine launch is needed.
#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kDecodeWaves = 4;
constexpr int kGuRB = 1;      // gate/up: 16-row blocks per workgroup
constexpr int kDownRB = 2;    // down: 16-row blocks per workgroup
constexpr int kNG = 4;        // groups per wave held in registers at once

struct Frag4 {
  bf16x8 s[4];
};

// Activation fragments of one 128-input group for one 16-token tile: lane l supplies
// token (l % 16) and inputs 32 s + 8 (l / 16) + 0..7. Invalid tokens supply zeros.
__device__ __forceinline__ Frag4 load_act(const uint16_t* row_ptr, bool valid, int col0) {
  Frag4 f;
  const int lane = (int)lane_id();
#pragma unroll
  for (int s = 0; s < 4; s++) {
    i32x4 v = {0, 0, 0, 0};
    if (valid) {
      uint4 u = *reinterpret_cast<const uint4*>(row_ptr + col0 + 32 * s + 8 * (lane >> 4));
      v[0] = (int)u.x; v[1] = (int)u.y; v[2] = (int)u.z; v[3] = (int)u.w;
    }
    f.s[s] = __builtin_bit_cast(bf16x8, v);
  }
  return f;
}

// -136 * sum over the group of the activations, in the C layout (all 4 values of a lane
// belong to token l % 16).
__device__ __forceinline__ f32x4 corr_chain(const Frag4& act) {
  const bf16x8 n136 = neg136_operand();
  f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; s++) c = mfma16(n136, act.s[s], c);
  return c;
}

// sum_k x_k q_k over one tile-group for rows 4(l/16)+i, token l%16.
__device__ __forceinline__ f32x4 tile_chain(uint4 words, const Frag4& act, f32x4 corr) {
  f32x4 c = corr;
  c = mfma16(dequant_word(words.x), act.s[0], c);
  c = mfma16(dequant_word(words.y), act.s[1], c);
  c = mfma16(dequant_word(words.z), act.s[2], c);
  c = mfma16(dequant_word(words.w), act.s[3], c);
  return c;
}

struct ExpertCtx {
  int e, n_act, seg0, cnt;
  const uint4* tiles;
  const uint16_t* scales;
};

__device__ __forceinline__ bool resolve_expert(const MoeArgs& a, int fixed_expert, ExpertCtx& cx) {
  if (fixed_expert >= 0) {
    if (blockIdx.y != 0) return false;
    cx.e = fixed_expert;
    cx.n_act = 1;
  } else {
    cx.e = nth_active_expert(a.offsets, a.E, (int)blockIdx.y, &cx.n_act);
    if (cx.e < 0) return false;
  }
  cx.seg0 = a.offsets[cx.e];
  cx.cnt = a.offsets[cx.e + 1] - cx.seg0;
  if (cx.cnt <= 0) return false;
  const int slot = a.e2s ? a.e2s[cx.e] : cx.e;
  if (slot < 0) {
    if (threadIdx.x == 0) atomicOr(a.debug, 1u);   // routed expert without a slot
    return false;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  cx.tiles = reinterpret_cast<const uint4*>(blob);
  cx.scales = reinterpret_cast<const uint16_t*>(blob + n_tiles(a.H, a.I) * kTileBytes);
  return true;
}

// ------------------------------------------------------------------------------------
// gate/up + SiLU*up
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void decode_gateup_kernel(MoeArgs a, int fixed_expert) {
  __shared__ f32x4 red[kDecodeWaves][kGuRB][2][64];
  const int lane = (int)lane_id(), wave = threadIdx.x >> 6;
  if (fixed_expert < 0 && blockIdx.x == 0 && blockIdx.y == 0) {
    const int nc = a.H / (kTileRows * kDownRB);
    for (int i = threadIdx.x; i < nc; i += blockDim.x) a.counters[i] = 0;
  }
  ExpertCtx cx;
  if (!resolve_expert(a, fixed_expert, cx)) return;
  const int G = a.H / kGroup;
  const int rb0 = blockIdx.x * kGuRB;
  const int ntt = (cx.cnt + 15) / 16;
  const int n = lane & 15;

  for (int tt = 0; tt < ntt; tt++) {
    const int r = tt * 16 + n;
    const bool valid = r < cx.cnt;
    const uint16_t* xrow = a.x;
    if (valid) xrow = a.x + (size_t)(a.sorted_flat[cx.seg0 + r] / a.k) * a.H;
    f32x4 acc[kGuRB][2];
#pragma unroll
    for (int rb = 0; rb < kGuRB; rb++)
      for (int m = 0; m < 2; m++) acc[rb][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g0 = wave * kNG; g0 < G; g0 += kDecodeWaves * kNG) {
      uint4 wv[kNG][kGuRB][2];
      uint2 sc[kNG][kGuRB][2];
#pragma unroll
      for (int q = 0; q < kNG; q++) {
        const int g = g0 + q;
        if (g < G) {
#pragma unroll
          for (int rb = 0; rb < kGuRB; rb++)
#pragma unroll
            for (int m = 0; m < 2; m++) {
              const size_t t = (size_t)((rb0 + rb) * 2 + m) * G + g;
              wv[q][rb][m] = cx.tiles[t * 64 + lane];
              sc[q][rb][m] = *reinterpret_cast<const uint2*>(cx.scales + t * 16 + 4 * (lane >> 4));
            }
        }
      }
#pragma unroll
      for (int q = 0; q < kNG; q++) {
        const int g = g0 + q;
        if (g < G) {
          Frag4 act = load_act(xrow, valid, g * kGroup);
          f32x4 corr = corr_chain(act);
#pragma unroll
          for (int rb = 0; rb < kGuRB; rb++)
#pragma unroll
            for (int m = 0; m < 2; m++)
              scale_accum(acc[rb][m], tile_chain(wv[q][rb][m], act, corr), sc[q][rb][m]);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < kGuRB; rb++)
      for (int m = 0; m < 2; m++) red[wave][rb][m][lane] = acc[rb][m];
    __syncthreads();
    if (wave == 0 && valid) {
#pragma unroll
      for (int rb = 0; rb < kGuRB; rb++) {
        f32x4 gs = red[0][rb][0][lane], us = red[0][rb][1][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; w++) {
          gs += red[w][rb][0][lane];
          us += red[w][rb][1][lane];
        }
        uint16_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const float gv = gs[i];
          hb[i] = f32_to_bf16(gv / (1.0f + expf(-gv)) * us[i]);
        }
        uint2 pk;
        pk.x = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
        pk.y = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
        *reinterpret_cast<uint2*>(a.h + (size_t)(cx.seg0 + r) * a.I + (rb0 + rb) * 16 +
                                  4 * (lane >> 4)) = pk;
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------
// down (+ routing weight), then last-arriver combine of the row slice
// ------------------------------------------------------------------------------------
__device__ void combine_rows(const MoeArgs& a, int row0, int nrows, int t0, int t1) {
  // y[t, row0 .. row0+nrows) = bf16(sum_j y_perm[flat_to_sorted[t k + j], .]) in slot order
  const int per_tok = nrows / 4;                       // float4 chunks per token
  for (int i = threadIdx.x; i < (t1 - t0) * per_tok; i += blockDim.x) {
    const int t = t0 + i / per_tok, c = (i % per_tok) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; j++) {
      const int r = a.flat_to_sorted[t * a.k + j];
      const float4 v = *reinterpret_cast<const float4*>(a.y_perm + (size_t)r * a.H + row0 + c);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(s.x) | ((uint32_t)f32_to_bf16(s.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(s.z) | ((uint32_t)f32_to_bf16(s.w) << 16);
    *reinterpret_cast<uint2*>(a.y + (size_t)t * a.H + row0 + c) = pk;
  }
}

__global__ __launch_bounds__(256) void decode_down_kernel(MoeArgs a, int fixed_expert) {
  __shared__ f32x4 red[kDecodeWaves][kDownRB][64];
  __shared__ int s_last;
  const int lane = (int)lane_id(), wave = threadIdx.x >> 6;
  ExpertCtx cx;
  if (!resolve_expert(a, fixed_expert, cx)) return;
  const int G = a.I / kGroup;
  const int rb0 = blockIdx.x * kDownRB;
  const size_t tile0 = 2 * (size_t)(a.I / kTileRows) * (a.H / kGroup);
  const int ntt = (cx.cnt + 15) / 16;
  const int n = lane & 15;

  for (int tt = 0; tt < ntt; tt++) {
    const int r = tt * 16 + n;
    const bool valid = r < cx.cnt;
    const uint16_t* hrow = a.h + (size_t)(cx.seg0 + (valid ? r : 0)) * a.I;
    f32x4 acc[kDownRB];
#pragma unroll
    for (int rb = 0; rb < kDownRB; rb++) acc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int g0 = wave * kNG; g0 < G; g0 += kDecodeWaves * kNG) {
      uint4 wv[kNG][kDownRB];
      uint2 sc[kNG][kDownRB];
#pragma unroll
      for (int q = 0; q < kNG; q++) {
        const int g = g0 + q;
        if (g < G) {
#pragma unroll
          for (int rb = 0; rb < kDownRB; rb++) {
            const size_t t = tile0 + (size_t)(rb0 + rb) * G + g;
            wv[q][rb] = cx.tiles[t * 64 + lane];
            sc[q][rb] = *reinterpret_cast<const uint2*>(cx.scales + t * 16 + 4 * (lane >> 4));
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kNG; q++) {
        const int g = g0 + q;
        if (g < G) {
          Frag4 act = load_act(hrow, valid, g * kGroup);
          f32x4 corr = corr_chain(act);
#pragma unroll
          for (int rb = 0; rb < kDownRB; rb++)
            scale_accum(acc[rb], tile_chain(wv[q][rb], act, corr), sc[q][rb]);
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < kDownRB; rb++) red[wave][rb][lane] = acc[rb];
    __syncthreads();
    if (wave == 0 && valid) {
      const float wt = a.w[a.sorted_flat[cx.seg0 + r]];
#pragma unroll
      for (int rb = 0; rb < kDownRB; rb++) {
        f32x4 o = red[0][rb][lane];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; w++) o += red[w][rb][lane];
        float4 v = make_float4(o[0] * wt, o[1] * wt, o[2] * wt, o[3] * wt);
        *reinterpret_cast<float4*>(a.y_perm + (size_t)(cx.seg0 + r) * a.H + (rb0 + rb) * 16 +
                                   4 * (lane >> 4)) = v;
      }
    }
    __syncthreads();
  }
  if (fixed_expert >= 0) return;    // sequential mode combines in a separate launch
  // Last-arriver combine: release our y_perm rows, count, and let the last one sum.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (uint32_t)(cx.n_act - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  combine_rows(a, rb0 * kTileRows, kDownRB * kTileRows, 0, a.T);
  if (threadIdx.x == 0)
    __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kCombineTok = 16;
__global__ __launch_bounds__(256) void combine_kernel(MoeArgs a) {
  const int t0 = blockIdx.y * kCombineTok;
  const int t1 = t0 + kCombineTok < a.T ? t0 + kCombineTok : a.T;
  const int nrows = a.H - (int)blockIdx.x * 64 < 64 ? a.H - (int)blockIdx.x * 64 : 64;
  combine_rows(a, blockIdx.x * 64, nrows, t0, t1);
}

hipError_t launch_moe_decode(const MoeArgs& a, hipStream_t s) {
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  {
    ProfScope prof("decode_gateup", s);
    hipLaunchKernelGGL(decode_gateup_kernel, dim3(a.I / (kTileRows * kGuRB), ny), dim3(256), 0, s, a, -1);
  }
  {
    ProfScope prof("decode_down", s);
    hipLaunchKernelGGL(decode_down_kernel, dim3(a.H / (kTileRows * kDownRB), ny), dim3(256), 0, s, a, -1);
  }
  return hipGetLastError();
}

hipError_t launch_moe_expert_range(const MoeArgs& a, int expert, int rows, hipStream_t s) {
  (void)rows;
  hipLaunchKernelGGL(decode_gateup_kernel, dim3(a.I / (kTileRows * kGuRB), 1), dim3(256), 0, s, a, expert);
  hipLaunchKernelGGL(decode_down_kernel, dim3(a.H / (kTileRows * kDownRB), 1), dim3(256), 0, s, a, expert);
  return hipGetLastError();
}

hipError_t launch_combine(const MoeArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  ProfScope prof("combine", s);
  hipLaunchKernelGGL(combine_kernel, dim3((a.H + 63) / 64, (a.T + kCombineTok - 1) / kCombineTok), dim3(256),
                     0, s, a);
  return hipGetLastError();
}

}  // namespace exmoe
