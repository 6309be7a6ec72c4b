// BF16 router logits, top-k selection and routing weights (gfx950).
//
// ExactMoE keeps the router in BF16 and its top-k procedure unchanged (abstract; Fig. 1
// caption). Logits: exact bf16 x bf16 products (exact in fp32) accumulated in fp64 and
// rounded once to bf16, so that the selection made on them does not depend on the
// summation order. Selection: (logit descending, expert id ascending) on the bf16 logits.
#include "common.h"
#include "device.h"

namespace exmoe {

// ---------------------------------------------------------------------------------
// Logits. A workgroup of 256 threads owns 4 tokens x 4 experts; 16 lanes split each
// (token, expert) dot product over H in interleaved 8-element chunks (each 16-lane
// group reads 256 contiguous bytes), then reduce in fp64 with lane shuffles.
// ---------------------------------------------------------------------------------
constexpr int kRouteTB = 4, kRouteEB = 4, kRouteSplit = 16;

__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wr,
                                                           const float* __restrict__ bias, int T,
                                                           int H, int E,
                                                           uint16_t* __restrict__ logits) {
  const int tid = threadIdx.x;
  const int sp = tid % kRouteSplit;
  const int p = tid / kRouteSplit;          // 0..15
  const int t = blockIdx.x * kRouteTB + p / kRouteEB;
  const int e = blockIdx.y * kRouteEB + p % kRouteEB;
  const bool valid = t < T && e < E;
  double acc = 0.0;
  if (valid) {
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
    const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)e * H);
    const int chunks = H / 8;
    for (int c = sp; c < chunks; c += kRouteSplit) {
      uint4 xv = xr[c], wv = wrow[c];
      const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float x0 = __uint_as_float(xa[q] << 16), x1 = __uint_as_float(xa[q] & 0xFFFF0000u);
        float w0 = __uint_as_float(wa[q] << 16), w1 = __uint_as_float(wa[q] & 0xFFFF0000u);
        acc += (double)(x0 * w0);   // bf16 x bf16 is exact in fp32
        acc += (double)(x1 * w1);
      }
    }
  }
#pragma unroll
  for (int off = kRouteSplit / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (valid && sp == 0) {
    if (bias) acc += (double)bias[e];
    logits[(size_t)t * E + e] = f64_to_bf16(acc);
  }
}

// ---------------------------------------------------------------------------------
// Top-k + weights: one wave per token. Each lane holds up to 4 experts (E <= 256) as
// 32-bit keys (order-preserving logit bits << 16 | (0xFFFF - id)); k rounds of a wave
// max pick the winners in slot order. -0 is canonicalized to +0 so the two tie.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(uint16_t b, int e) {
  if (b == 0x8000) b = 0;
  uint32_t o = (b & 0x8000) ? (uint32_t)(~b & 0xFFFF) : (uint32_t)(b | 0x8000);
  return (o << 16) | (uint32_t)(0xFFFF - e);
}

__global__ __launch_bounds__(256) void topk_kernel(const uint16_t* __restrict__ logits,
                                                   const int32_t* __restrict__ given_ids, int T,
                                                   int E, int k, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = (int)lane_id();
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  const uint16_t* lrow = logits + (size_t)t * E;
  uint32_t key[4];
  float lv[4];
  float m_all = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    int e = lane + 64 * q;
    if (e < E) {
      uint16_t b = lrow[e];
      key[q] = order_key(b, e);
      lv[q] = bf16_to_f32(b);
      m_all = fmaxf(m_all, lv[q]);
    } else {
      key[q] = 0;
      lv[q] = -INFINITY;
    }
  }
  m_all = wave_max(m_all);
  // Slot j (k <= 64) lands in lane j.
  float my_sel = -INFINITY;
  int my_id = -1;
  if (given_ids) {
    if (lane < k) {
      my_id = given_ids[(size_t)t * k + lane];
      my_sel = (my_id >= 0 && my_id < E) ? bf16_to_f32(lrow[my_id]) : -INFINITY;
    }
  } else {
    for (int j = 0; j < k; j++) {
      uint32_t best = key[0];
#pragma unroll
      for (int q = 1; q < 4; q++) best = key[q] > best ? key[q] : best;
      best = wave_max(best);
      const int id = 0xFFFF - (int)(best & 0xFFFF);
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (lane + 64 * q == id) key[q] = 0;     // the owner removes the winner
      if (lane == j) {
        my_id = id;
        my_sel = bf16_to_f32(lrow[id]);
      }
    }
  }
  float m, denom;
  if (renormalize) {
    m = wave_max(my_sel);
    denom = wave_sum(lane < k ? expf(my_sel - m) : 0.f);
  } else {
    m = m_all;
    float z = 0.f;
#pragma unroll
    for (int q = 0; q < 4; q++)
      if (lane + 64 * q < E) z += expf(lv[q] - m);
    denom = wave_sum(z);
  }
  if (lane < k) {
    if (ids) ids[(size_t)t * k + lane] = my_id;
    w[(size_t)t * k + lane] = expf(my_sel - m) / denom;
  }
}

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                               int E, uint16_t* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((T + kRouteTB - 1) / kRouteTB, (E + kRouteEB - 1) / kRouteEB);
  ProfScope prof("route_logits", s);
  hipLaunchKernelGGL(route_logits_kernel, grid, dim3(256), 0, s, x, wr, bias, T, H, E, logits);
  return hipGetLastError();
}

hipError_t launch_topk(const uint16_t* logits, const int32_t* given_ids, int T, int E, int k,
                       int renormalize, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  ProfScope prof("topk", s);
  hipLaunchKernelGGL(topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, given_ids, T, E, k,
                     renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace exmoe
