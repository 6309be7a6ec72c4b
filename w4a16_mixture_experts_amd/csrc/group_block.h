// Stable grouping of routed (token, slot) pairs by expert, as a device function of one
// workgroup (shared by the grouping kernel, the fused top-k + grouping kernel and the
// publisher of the table-routed decode). The flat ids are walked in chunks of one id per
// thread: lanes holding the same expert find each other with one ballot per id bit, rank
// with a masked popcount, and add the counts of earlier waves (LDS prefixes) and earlier
// chunks (running bases).
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

// Called by every thread of a THREADS-thread workgroup with n <= kGroupSingleMaxRows;
// outputs may live in LDS or global memory. Every id the thread handles is loaded first,
// all at once (chunk c: flat index c * THREADS + tid), so that one memory latency covers
// the ids of all chunks.
template <int THREADS = kGroupThreads>
__device__ __forceinline__ void group_block(const int32_t* ids, int n, int E, int32_t* offsets,
                                            int32_t* sorted_flat, int32_t* flat_to_sorted,
                                            GroupSharedT<THREADS>& gs) {
  constexpr int kThreads = THREADS;
  constexpr int kWaves = THREADS / 64;
  constexpr int kChunks = kGroupSingleMaxRows / THREADS;   // ids per thread
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ebits = 32 - __clz(E - 1 > 0 ? E - 1 : 1);

  int idr[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; c++) idr[c] = -1;
  if (n > 0) {
#pragma unroll
    for (int c = 0; c < kChunks; c++) {
      const int f = c * kThreads + tid;
      const int v = ids[f < n ? f : n - 1];   // clamped: no load under a per-thread branch
      idr[c] = f < n ? v : -1;
    }
  }
  // 1. ranks inside each wave (lanes holding the same expert find each other with one
  // ballot per id bit) and the histogram: one LDS atomic per (wave, chunk, expert), by
  // the expert's first lane in the wave
  int rank[kChunks], nlead[kChunks];
  for (int e = tid; e < E; e += kThreads) gs.count[e] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kChunks; c++) {
    rank[c] = 0;
    nlead[c] = 0;
    if (c * kThreads >= n) break;   // uniform
    const int e = idr[c];
    const bool ok = e >= 0 && e < E;
    const uint64_t okm = __ballot(ok);
    uint64_t peers = ok ? okm : 0ull;
    for (int b = 0; b < ebits; b++) {
      const uint64_t m = __ballot(ok && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t below = peers & ((1ull << lane) - 1ull);
    rank[c] = __popcll(below);
    nlead[c] = ok && below == 0 ? __popcll(peers) : 0;   // the wave leader of this expert
    if (nlead[c]) atomicAdd(&gs.count[e], nlead[c]);
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
  // 3. stable scatter, chunk by chunk: the per-wave counts of the chunk become, per
  // expert, exclusive prefixes over the waves (a 16-lane row per expert with 16 waves, else
  // one thread per expert), which place each wave's rows after those of the earlier waves
  // and chunks
#pragma unroll
  for (int c = 0; c < kChunks; c++) {
    if (c * kThreads >= n) break;   // uniform
    for (int i = tid; i < kWaves * E; i += kThreads) gs.wave[i / E][i % E] = 0;
    __syncthreads();
    const int e = idr[c];
    if (nlead[c]) gs.wave[wave][e] = nlead[c];
    __syncthreads();
    if constexpr (kWaves == 16) {
      // 16 lanes per expert (lane w of the row: wave w), an inclusive scan along the row by
      // DPP row shifts (lanes without a source add 0), then base + exclusive prefix; the
      // row's last lane moves the base on (its lanes read the base before, in program order)
      for (int e0 = 0; e0 < E; e0 += kThreads / 16) {
        const int e2 = e0 + (tid >> 4), w = tid & 15;
        const int v = e2 < E ? gs.wave[w][e2] : 0;
        int incl = v;
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);   // row_shr:1
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);   // row_shr:2
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);   // row_shr:4
        incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);   // row_shr:8
        if (e2 < E) {
          const int b = gs.base[e2];
          gs.wave[w][e2] = b + incl - v;
          if (w == 15) gs.base[e2] = b + incl;
        }
      }
    } else {
      for (int e2 = tid; e2 < E; e2 += kThreads) {
        int run = gs.base[e2];
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
          const int v = gs.wave[w][e2];
          gs.wave[w][e2] = run;
          run += v;
        }
        gs.base[e2] = run;
      }
    }
    __syncthreads();
    const int f = c * kThreads + tid;
    if (e >= 0 && e < E) {
      const int pos = gs.wave[wave][e] + rank[c];
      sorted_flat[pos] = f;
      flat_to_sorted[f] = pos;
    } else if (f < n) {
      flat_to_sorted[f] = -1;   // id outside [0, E): in no segment
    }
    __syncthreads();   // the wave counts are cleared for the next chunk
  }
}

}  // namespace exmoe
