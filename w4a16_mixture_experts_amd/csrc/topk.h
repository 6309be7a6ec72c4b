// Top-k selection and routing weights of one token by one wave (shared by the routing
// kernels: the prefill top-k, the per-token decode routing and the last arriver of the
// few-token routing kernel).
#pragma once

#include "common.h"
#include "device.h"

namespace exmoe {

// ---------------------------------------------------------------------------------
// Top-k + weights for one token, by one wave. Each lane holds up to 4 experts (E <= 256)
// as 32-bit keys (order-preserving logit bits << 16 | (0xFFFF - id)); k rounds of a DPP
// wave max pick the winners in slot order (the owner lane clears its key). -0 is
// canonicalized to +0 so the two tie. Slot j (k <= 64) ends in lane j.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(uint16_t b, int e) {
  if (b == 0x8000) b = 0;
  const uint32_t o = (b & 0x8000) ? (uint32_t)(~b & 0xFFFF) : (uint32_t)(b | 0x8000);
  return (o << 16) | (uint32_t)(0xFFFF - e);
}

// Routing weights of the selected slots (slot j in lane j, logit my_sel), shared by both
// selection methods so that their weights agree bit for bit. renormalize: softmax over
// the k selected logits; otherwise the full softmax probability (lv: this lane's logits).
__device__ __forceinline__ float topk_weight(float my_sel, const float* lv, int nq, int E, int k, int renormalize) {
  const int lane = (int)lane_id();
  float m, denom;
  if (renormalize) {
    m = wave_max_f32(my_sel);
    denom = wave_sum_f32(lane < k ? expf(my_sel - m) : 0.f);
  } else {
    float m_all = -INFINITY;
    for (int q = 0; q < nq; q++) m_all = fmaxf(m_all, lv[q]);
    m = wave_max_f32(m_all);
    float z = 0.f;
    for (int q = 0; q < nq; q++)
      if (lane + 64 * q < E) z += expf(lv[q] - m);
    denom = wave_sum_f32(z);
  }
  return lane < k ? expf(my_sel - m) / denom : 0.f;
}

__device__ __forceinline__ void topk_token(const uint16_t* __restrict__ lrow,
                                           const int32_t* __restrict__ given, int E, int k,
                                           int renormalize, int& my_id, float& my_w) {
  const int lane = (int)lane_id();
  uint32_t key[4];
  float lv[4];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const int e = lane + 64 * q;
    if (e < E) {
      const uint16_t b = lrow[e];
      key[q] = order_key(b, e);
      lv[q] = bf16_to_f32(b);
    } else {
      key[q] = 0;
      lv[q] = -INFINITY;
    }
  }
  float my_sel = -INFINITY;
  my_id = -1;
  if (given) {
    if (lane < k) {
      my_id = given[lane];
      my_sel = (my_id >= 0 && my_id < E) ? bf16_to_f32(lrow[my_id]) : -INFINITY;
    }
  } else {
    for (int j = 0; j < k; j++) {
      uint32_t best = key[0];
#pragma unroll
      for (int q = 1; q < 4; q++) best = key[q] > best ? key[q] : best;
      best = wave_max_u32(best);
      const int id = 0xFFFF - (int)(best & 0xFFFF);
#pragma unroll
      for (int q = 0; q < 4; q++)
        if (lane + 64 * q == id) key[q] = 0;
      if (lane == j) {
        my_id = id;
        const uint32_t o = best >> 16;
        my_sel = bf16_to_f32((o & 0x8000) ? (uint16_t)(o & 0x7FFF) : (uint16_t)(~o & 0xFFFF));
      }
    }
  }
  my_w = topk_weight(my_sel, lv, 4, E, k, renormalize);
}

// ---------------------------------------------------------------------------------
// The same selection and weights for E <= 64 by ranks: lane e holds expert e's key; its
// rank is the number of keys above it (64 independent compares against readlane
// broadcasts instead of k dependent wave reductions). Keys are distinct, so ranks
// 0 .. k-1 are the selected experts in slot order; one ballot per slot moves slot j to
// lane j, and the weights come from topk_weight as in topk_token.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ void topk_rank_token(const uint16_t* __restrict__ lrow, int E, int k, int renormalize,
                                                int& my_id, float& my_w) {
  const int lane = (int)lane_id();
  const bool in = lane < E;
  const uint16_t b = in ? lrow[lane] : (uint16_t)0;
  const uint32_t key = in ? order_key(b, lane) : 0u;
  float lv[1] = {in ? bf16_to_f32(b) : -INFINITY};
  int r = 0;
#pragma unroll
  for (int j = 0; j < 64; j++) {
    const uint32_t kj = (uint32_t)__builtin_amdgcn_readlane((int)key, j);
    r += kj > key ? 1 : 0;
  }
  const int rank = in ? r : 64;
  my_id = -1;
  float my_sel = -INFINITY;
  for (int j = 0; j < k; j++) {
    const int src = (int)__builtin_ctzll(__ballot(rank == j));
    if (lane == j) my_id = src;
  }
  if (lane < k) my_sel = bf16_to_f32(lrow[my_id]);
  my_w = topk_weight(my_sel, lv, 1, E, k, renormalize);
}

}  // namespace exmoe
