// Group routed (token, slot) pairs by expert: counts, exclusive scan and a stable
// scatter (gfx950). Fig. 1 of ExactMoE groups tokens by selected expert; the grouping is
// the unique stable one (ascending flat index f = t*k + j inside each expert), so the
// result is bit-identical to a stable argsort whatever the scheduling.
//
// One workgroup of 1024 threads (16 waves) walks the flat ids in chunks of 1024. Inside
// a wave, the lanes holding the same expert find each other with one ballot per id bit
// (a match-any built from ballots) and take their rank with a masked popcount; ranks
// across waves come from per-wave counts in LDS, across chunks from running bases.
#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kGroupThreads = 1024;
constexpr int kGroupWaves = kGroupThreads / 64;

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int n,
                                                              int E, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_flat,
                                                              int32_t* __restrict__ flat_to_sorted) {
  __shared__ int s_count[kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_wave[kGroupWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ebits = 32 - __clz(E - 1 > 0 ? E - 1 : 1);

  for (int e = tid; e < E; e += kGroupThreads) s_count[e] = 0;
  __syncthreads();
  // 1. histogram (integer LDS atomics: order-independent)
  for (int f = tid; f < n; f += kGroupThreads) {
    int e = ids[f];
    if (e >= 0 && e < E) atomicAdd(&s_count[e], 1);
  }
  __syncthreads();
  // 2. exclusive scan by wave 0 (E <= 256 -> 4 values per lane)
  if (wave == 0) {
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int e = lane * 4 + q;
      v[q] = e < E ? s_count[e] : 0;
      run += v[q];
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int excl = incl - run;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int e = lane * 4 + q;
      if (e < E) {
        s_base[e] = excl;
        offsets[e] = excl;
      }
      excl += v[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  // 3. stable scatter, chunk by chunk
  for (int c0 = 0; c0 < n; c0 += kGroupThreads) {
    for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) s_wave[i / E][i % E] = 0;
    __syncthreads();
    const int f = c0 + tid;
    int e = f < n ? ids[f] : -1;
    const bool ok = e >= 0 && e < E;
    uint64_t peers = __ballot(ok);
    if (!ok) peers = 0;
    for (int b = 0; b < ebits; b++) {
      uint64_t m = __ballot(ok && ((e >> b) & 1));
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t below = peers & ((1ull << lane) - 1ull);
    const int rank = __popcll(below);
    if (ok && below == 0) s_wave[wave][e] = __popcll(peers);   // wave leader of this expert
    __syncthreads();
    if (ok) {
      int pos = s_base[e] + rank;
      for (int w = 0; w < wave; w++) pos += s_wave[w][e];
      sorted_flat[pos] = f;
      flat_to_sorted[f] = pos;
    }
    __syncthreads();
    for (int e2 = tid; e2 < E; e2 += kGroupThreads) {
      int add = 0;
      for (int w = 0; w < kGroupWaves; w++) add += s_wave[w][e2];
      s_base[e2] += add;
    }
    __syncthreads();
  }
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_flat,
                        int32_t* flat_to_sorted, hipStream_t s) {
  ProfScope prof("group", s);
  hipLaunchKernelGGL(group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, T * k, E, offsets,
                     sorted_flat, flat_to_sorted);
  return hipGetLastError();
}

}  // namespace exmoe
