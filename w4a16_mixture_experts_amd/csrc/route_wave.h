// Router logits of a lane group and the selection part of a table-routed launch,
// shared by the routing kernels and the decode kernel that routes its own tokens.
//
// ExactMoE keeps the router in BF16 and its top-k procedure unchanged (abstract; Fig. 1
// caption). Logits: exact bf16 x bf16 products (exact in fp32) accumulated in fp64 and
// rounded once to bf16, so that the selection made on them does not depend on the
// summation order. Selection: (logit descending, expert id ascending) on the bf16 logits.
#pragma once
#include "common.h"
#include "device.h"
#include "topk.h"

namespace exmoe {

// ---------------------------------------------------------------------------------
// Logits. A lane group owns a block of TB tokens x EB experts and splits H among its
// LANES lanes in interleaved 16-byte chunks (contiguous bytes across the group); each
// chunk is converted to fp64 once and feeds TB*EB fp64 FMAs (bf16 products are exact in
// fp64). Partial sums are added with DPP row rotations (and across rows with readlane
// when LANES = 64); one lane rounds once to bf16. Used with LANES = 64 and small blocks
// (many waves) for a few tokens; many tokens go to the fp64 matrix-core kernel.
// ---------------------------------------------------------------------------------
// WT: write-through (agent-scope atomic) stores of the logits, read back by another
// workgroup in the same launch. ONE: the caller guarantees H <= 8 LANES MC (one pass of
// loads, all issued before any arithmetic). XS (LANES = 64): the lane groups also write
// the grouped GEMM's correction seeds of their tokens from the activation chunks they
// load, xsum[g][t] = -136 * (sum of group g of token t) in the order of chunk8_sum and
// row16_tree_sum (a 16-lane row holds the 16 chunks of one group).
template <int TB, int EB, int LANES, int MC, bool WT, bool ONE = false, bool XS = false>
__device__ __forceinline__ void route_logits_wave(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                                                  const float* __restrict__ bias, int T, int H, int E,
                                                  uint16_t* __restrict__ logits, int blk,
                                                  float* __restrict__ xsum = nullptr) {
  static_assert(!XS || LANES == 64, "seed rows need 16-lane rows of consecutive chunks");
  const int lane = (int)lane_id();
  const int li = lane % LANES;
  const int nEB = (E + EB - 1) / EB;
  const int tb = blk / nEB, eb = blk % nEB;   // (token block, expert block)
  const int t0 = tb * TB, e0 = eb * EB;
  double acc[TB][EB];
#pragma unroll
  for (int i = 0; i < TB; i++)
#pragma unroll
    for (int j = 0; j < EB; j++) acc[i][j] = 0.0;
  if (t0 < T) {
    const int chunks = H / 8;
    // MC chunks per lane are loaded before any arithmetic: one memory latency per piece
    for (int c0 = 0; ONE ? c0 == 0 : c0 < chunks; c0 += LANES * MC) {
      uint4 xu[TB][MC], wu[EB][MC];
#pragma unroll
      for (int m = 0; m < MC; m++) {
        int c = c0 + li + LANES * m;
        c = c < chunks ? c : chunks - 1;
#pragma unroll
        for (int i = 0; i < TB; i++) {
          const int t = t0 + i < T ? t0 + i : T - 1;
          xu[i][m] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[c];
        }
#pragma unroll
        for (int j = 0; j < EB; j++) {
          const int e = e0 + j < E ? e0 + j : E - 1;
          wu[j][m] = reinterpret_cast<const uint4*>(wr + (size_t)e * H)[c];
        }
      }
      if (ONE) {
        // chunks past H become zeros (a product 0 * 0 added to a sum that starts at +0.0
        // leaves its bits unchanged), so that no load sits under a per-lane branch
#pragma unroll
        for (int m = 0; m < MC; m++) {
          const bool on = c0 + li + LANES * m < chunks;
#pragma unroll
          for (int i = 0; i < TB; i++) xu[i][m] = on ? xu[i][m] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
          for (int j = 0; j < EB; j++) wu[j][m] = on ? wu[j][m] : make_uint4(0u, 0u, 0u, 0u);
        }
      }
      if (XS) {
        // row r of the wave holds chunks c0 + 64 m + 16 r + (0..15), i.e. group
        // (c0 + 64 m) / 16 + r; group g is summed by the lane groups of expert block
        // g mod the block count
#pragma unroll
        for (int m = 0; m < MC; m++) {
          const int c = c0 + li + LANES * m, g0 = (c0 + LANES * m) / 16;
          if ((eb - g0 % nEB + nEB) % nEB >= 4) continue;   // none of the wave's four groups (wave-uniform)
          const bool mine = (c / 16) % nEB == eb && (li & 15) == 0 && c < chunks;
#pragma unroll
          for (int i = 0; i < TB; i++) {
            const float v = row16_tree_sum(chunk8_sum(xu[i][m]));
            if (mine && t0 + i < T) xsum[(size_t)(c / 16) * T + t0 + i] = -136.0f * v;
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MC; m++) {
        if (ONE || c0 + li + LANES * m < chunks) {
          double xv[TB][8], wv[EB][8];
#pragma unroll
          for (int i = 0; i < TB; i++) {
            const uint32_t q4[4] = {xu[i][m].x, xu[i][m].y, xu[i][m].z, xu[i][m].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
              xv[i][2 * q] = (double)__uint_as_float(q4[q] << 16);
              xv[i][2 * q + 1] = (double)__uint_as_float(q4[q] & 0xFFFF0000u);
            }
          }
#pragma unroll
          for (int j = 0; j < EB; j++) {
            const uint32_t q4[4] = {wu[j][m].x, wu[j][m].y, wu[j][m].z, wu[j][m].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
              wv[j][2 * q] = (double)__uint_as_float(q4[q] << 16);
              wv[j][2 * q + 1] = (double)__uint_as_float(q4[q] & 0xFFFF0000u);
            }
          }
#pragma unroll
          for (int i = 0; i < TB; i++)
#pragma unroll
            for (int j = 0; j < EB; j++)
#pragma unroll
              for (int q = 0; q < 8; q++) acc[i][j] = fma(xv[i][q], wv[j][q], acc[i][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TB; i++)
#pragma unroll
    for (int j = 0; j < EB; j++) {
      double s = row16_sum_f64(acc[i][j]);
      if (LANES == 64) {
        // rows 0..3 of the wave, added in a fixed order
        const long long b = __double_as_longlong(s);
        const int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
        double r[4];
#pragma unroll
        for (int q = 0; q < 4; q++)
          r[q] = __longlong_as_double(((long long)(unsigned)__builtin_amdgcn_readlane(lo, 16 * q)) |
                                      ((long long)__builtin_amdgcn_readlane(hi, 16 * q) << 32));
        s = ((r[0] + r[1]) + r[2]) + r[3];
      }
      const int t = t0 + i, e = e0 + j;
      if (li == 0 && t < T && e < E) {
        const double v = bias ? s + (double)bias[e] : s;
        if (WT) __hip_atomic_store(logits + (size_t)t * E + e, f64_to_bf16(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else logits[(size_t)t * E + e] = f64_to_bf16(v);
      }
    }
}

// ---------------------------------------------------------------------------------
// Selection part of a table-routed launch (T <= kRouteSelMaxTok, H <= kRouteSelMaxH: the
// logits of a wave take one pass of loads). Workgroup `blk` of NW
// waves takes one block of 4 tokens (wave w: token w % 4) and NW / 4 blocks of 2 experts
// (wave w: block w / 4 of the workgroup's), and computes those logits. The last workgroup
// of the token block to arrive (one arrival counter per token block) then selects each
// token's experts from the bf16 logits of all workgroups, one wave per token, writes ids
// and weights, and fills word tb of every expert's 16-byte table row: byte t % 4 of it is
// slot + 1 when token t selected the expert, else 0. It clears the counter, so the
// counters are zero between launches (and must be zero before the first one). Returns
// true in that last arriver. The ids, weights and table are read by later launches.
// Ordering: the logits are stored with agent-scope atomic stores, the workgroup barrier
// puts every wave's stores before thread 0's count, and the count is an agent-scope
// acquire-release read-modify-write: the releases of all workgroups of the token block
// happen before the last arriver's acquire, which the barrier after it extends to all of
// its waves; they then read the logits with agent-scope atomic loads.
// ---------------------------------------------------------------------------------
constexpr int kRouteSelTB = 4, kRouteSelEB = 2;
constexpr int kRouteSelMaxH = 8 * 64 * 4;   // 16-byte chunks x lanes x chunks per lane
static_assert(kRouteSelMaxTok <= kRouteSelTB * kRouteSelCounters, "one counter per token block");

struct RouteSelShared {
  uint16_t lg[kRouteSelTB][kMaxExperts];   // the token block's logits
  uint8_t tab[kRouteSelTB][kMaxExperts];   // slot + 1 per (token, expert)
  int last;
};

// workgroups of NW waves per token block
__host__ __device__ inline int route_sel_groups(int E, int NW) {
  const int nEB = (E + kRouteSelEB - 1) / kRouteSelEB, pairs = NW / kRouteSelTB;
  return (nEB + pairs - 1) / pairs;
}

template <int NW>
__device__ bool route_sel_part(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                               const float* __restrict__ bias, int T, int H, int E, int k, int renormalize,
                               uint16_t* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w,
                               uint8_t* __restrict__ sel, uint32_t* __restrict__ counters, int blk,
                               RouteSelShared& sh) {
  static_assert(NW % kRouteSelTB == 0, "whole token blocks");
  constexpr int PAIRS = NW / kRouteSelTB;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nEB = (E + kRouteSelEB - 1) / kRouteSelEB;
  const int nWB = route_sel_groups(E, NW);
  const int tb = blk / nWB, wb = blk % nWB;
  const int t = tb * kRouteSelTB + (wave % kRouteSelTB);   // this wave's token
  const int eb = wb * PAIRS + wave / kRouteSelTB;          // this wave's expert block
  if (t < T && eb < nEB)
    route_logits_wave<1, kRouteSelEB, 64, 4, true, true>(x, wr, bias, T, H, E, logits, t * nEB + eb);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);   // this wave's logits stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(counters + tb * kRouteCounterStride, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = old == (uint32_t)(nWB - 1);
  }
  __syncthreads();
  if (!sh.last) return false;
  if (wave < kRouteSelTB) {
    const int tt = tb * kRouteSelTB + wave;
    for (int e = lane; e < E; e += 64) sh.tab[wave][e] = 0;
    if (tt < T) {
      for (int e = lane; e < E; e += 64)
        sh.lg[wave][e] = __hip_atomic_load(logits + (size_t)tt * E + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      int id;
      float wt;
      if (E <= 64) topk_rank_token(sh.lg[wave], E, k, renormalize, id, wt);
      else topk_token(sh.lg[wave], nullptr, E, k, renormalize, id, wt);
      if (lane < k) {
        __hip_atomic_store(ids + (size_t)tt * k + lane, id, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        w[(size_t)tt * k + lane] = wt;
        sh.tab[wave][id] = (uint8_t)(lane + 1);   // the k ids are distinct
      }
    }
  }
  __syncthreads();
  // word tb of every expert's table row: the token block's four slots
  for (int e = (int)threadIdx.x; e < E; e += 64 * NW) {
    const uint32_t v = (uint32_t)sh.tab[0][e] | ((uint32_t)sh.tab[1][e] << 8) | ((uint32_t)sh.tab[2][e] << 16) |
                       ((uint32_t)sh.tab[3][e] << 24);
    __hip_atomic_store(reinterpret_cast<uint32_t*>(sel) + (size_t)e * (kSelRowBytes / 4) + tb, v, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every workgroup of the token block has counted, so the counter can be cleared at once:
  // it is read again only by the next launch, which starts after every store of this one
  // has completed (no wait here for the ids and table words).
  if (threadIdx.x == 0)
    __hip_atomic_store(counters + tb * kRouteCounterStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

}  // namespace exmoe
