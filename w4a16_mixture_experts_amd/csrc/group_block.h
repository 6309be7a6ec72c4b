// Stable grouping of routed (token, slot) pairs by expert, as a device function of one
// 1024-thread workgroup (shared by the grouping kernel and the fused top-k + grouping
// kernel). The flat ids are walked in chunks of 1024: lanes holding the same expert
// find each other with one ballot per id bit, rank with a masked popcount, and add the
// counts of earlier waves (LDS) and earlier chunks (running bases).
#pragma once

#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;
constexpr int kTopkGroupMaxRows = 4096;
constexpr int kGroupSingleMaxRows = 4096;   // more rows: the chunked three-launch grouping

template <int THREADS>
struct GroupSharedT {
  int count[kMaxExperts];
  int base[kMaxExperts];
  int wave[THREADS / 64][kMaxExperts];
};
using GroupShared = GroupSharedT<kGroupThreads>;

// Called by every thread of a THREADS-thread workgroup; outputs may live in LDS or global
// memory.
template <int THREADS = kGroupThreads>
__device__ __forceinline__ void group_block(const int32_t* ids, int n, int E, int32_t* offsets,
                                            int32_t* sorted_flat, int32_t* flat_to_sorted,
                                            GroupSharedT<THREADS>& gs) {
  constexpr int kThreads = THREADS;
  constexpr int kWaves = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ebits = 32 - __clz(E - 1 > 0 ? E - 1 : 1);

  for (int e = tid; e < E; e += kThreads) gs.count[e] = 0;
  __syncthreads();
  // 1. histogram (integer LDS atomics: order-independent)
  for (int f = tid; f < n; f += kThreads) {
    const int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&gs.count[e], 1);
  }
  __syncthreads();
  // 2. exclusive scan by wave 0 (E <= 256 -> 4 values per lane)
  if (wave == 0) {
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = lane * 4 + q;
      v[q] = e < E ? gs.count[e] : 0;
      run += v[q];
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = lane * 4 + q;
      if (e < E) {
        gs.base[e] = excl;
        offsets[e] = excl;
      }
      excl += v[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  // 3. stable scatter, chunk by chunk
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    for (int i = tid; i < kWaves * E; i += kThreads) gs.wave[i / E][i % E] = 0;
    __syncthreads();
    const int f = c0 + tid;
    const int e = f < n ? ids[f] : -1;
    const bool ok = e >= 0 && e < E;
    const uint64_t okm = __ballot(ok);
    uint64_t peers = ok ? okm : 0ull;
    for (int b = 0; b < ebits; b++) {
      const uint64_t m = __ballot(ok && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t below = peers & ((1ull << lane) - 1ull);
    const int rank = __popcll(below);
    if (ok && below == 0) gs.wave[wave][e] = __popcll(peers);   // wave leader of this expert
    __syncthreads();
    if (ok) {
      int pos = gs.base[e] + rank;
      for (int w = 0; w < wave; w++) pos += gs.wave[w][e];
      sorted_flat[pos] = f;
      flat_to_sorted[f] = pos;
    } else if (f < n) {
      flat_to_sorted[f] = -1;   // id outside [0, E): in no segment
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kThreads) {
      int add = 0;
      for (int w = 0; w < kWaves; w++) add += gs.wave[w][e2];
      gs.base[e2] += add;
    }
    __syncthreads();
  }
}

}  // namespace exmoe
