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
#include "group_block.h"

namespace exmoe {

__global__ __launch_bounds__(kGroupThreads) void group_kernel(const int32_t* __restrict__ ids, int n,
                                                              int E, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_flat,
                                                              int32_t* __restrict__ flat_to_sorted) {
  __shared__ GroupShared gs;
  group_block(ids, n, E, offsets, sorted_flat, flat_to_sorted, gs);
}

// ---------------------------------------------------------------------------------
// More rows than one workgroup walks quickly (n > kGroupSingleMaxRows): launches over
// chunks of kGroupThreads rows. Counts: one workgroup per chunk adds its rows into an LDS
// histogram and writes cnt[c][e]. Scan: one workgroup turns the counts into the offsets
// and, in place, into each chunk's base per expert, base[c][e] = offsets[e] + (rows of
// expert e in the chunks before c). Scatter: one workgroup per chunk ranks its rows as the
// single-workgroup grouping does inside a chunk and writes them at base + rank. Up to
// kGroupScanInScatterChunks chunks each scatter workgroup makes its own bases from the
// counts, and the scan launch does not run. The result is the same unique stable
// grouping.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(kGroupThreads) void group_count_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                    int32_t* __restrict__ cnt) {
  __shared__ int hist[kMaxExperts];
  const int tid = threadIdx.x, c = blockIdx.x;
  for (int e = tid; e < E; e += kGroupThreads) hist[e] = 0;
  __syncthreads();
  const int f = c * kGroupThreads + tid;
  const int e = f < n ? ids[f] : -1;
  if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  __syncthreads();
  for (int i = tid; i < E; i += kGroupThreads) cnt[(size_t)c * E + i] = hist[i];
}

__global__ __launch_bounds__(256) void group_scan_kernel(int32_t* __restrict__ cnt, int nchunks, int E,
                                                         int32_t* __restrict__ offsets) {
  __shared__ int total[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < E) {
    int s = 0;
    for (int c = 0; c < nchunks; c++) s += cnt[(size_t)c * E + tid];
    total[tid] = s;
  }
  __syncthreads();
  __shared__ int excl_s[kMaxExperts];
  if (tid < 64) {   // exclusive scan over E <= 256 experts: 4 per lane
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = lane * 4 + q;
      v[q] = e < E ? total[e] : 0;
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
        excl_s[e] = excl;
        offsets[e] = excl;
      }
      excl += v[q];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  if (tid < E) {
    int run = excl_s[tid];
    for (int c = 0; c < nchunks; c++) {
      const int v = cnt[(size_t)c * E + tid];
      cnt[(size_t)c * E + tid] = run;   // becomes the chunk's base for this expert
      run += v;
    }
  }
}

__global__ __launch_bounds__(kGroupThreads) void group_scatter_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                                      const int32_t* __restrict__ base,
                                                                      int32_t* __restrict__ sorted_flat,
                                                                      int32_t* __restrict__ flat_to_sorted) {
  __shared__ int wavecnt[kGroupWaves][kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x;
  const int ebits = 32 - __clz(E - 1 > 0 ? E - 1 : 1);
  for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) wavecnt[i / E][i % E] = 0;
  __syncthreads();
  const int f = c * kGroupThreads + tid;
  const int e = f < n ? ids[f] : -1;
  const bool ok = e >= 0 && e < E;
  const uint64_t okm = __ballot(ok);
  uint64_t peers = ok ? okm : 0ull;
  for (int b = 0; b < ebits; b++) {
    const uint64_t m = __ballot(ok && ((e >> b) & 1));
    peers &= ((e >> b) & 1) ? m : ~m;
  }
  const uint64_t below = peers & ((1ull << lane) - 1ull);
  if (ok && below == 0) wavecnt[wave][e] = __popcll(peers);   // wave leader of this expert
  __syncthreads();
  if (ok) {
    int pos = base[(size_t)c * E + e] + __popcll(below);
    for (int w = 0; w < wave; w++) pos += wavecnt[w][e];
    sorted_flat[pos] = f;
    flat_to_sorted[f] = pos;
  } else if (f < n) {
    flat_to_sorted[f] = -1;   // id outside [0, E): in no segment
  }
}

// Up to kGroupScanInScatterChunks chunks the scan runs inside the scatter: every scatter
// workgroup reads the counts of all chunks (nchunks x E ints, loaded with its ids), adds
// the totals and the counts of the chunks before its own, scans the totals over the
// experts, and writes its rows at offsets[e] + (rows of e in earlier chunks) + rank;
// workgroup 0 also writes the offsets. One launch less than count, scan, scatter.
constexpr int kGroupScanInScatterChunks = 64;
__global__ __launch_bounds__(kGroupThreads) void group_scan_scatter_kernel(const int32_t* __restrict__ ids, int n,
                                                                           int E, const int32_t* __restrict__ cnt,
                                                                           int32_t* __restrict__ offsets,
                                                                           int32_t* __restrict__ sorted_flat,
                                                                           int32_t* __restrict__ flat_to_sorted) {
  __shared__ int wavecnt[kGroupWaves][kMaxExperts];
  __shared__ int s_tot[kMaxExperts], s_base[kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = blockIdx.x, nchunks = gridDim.x;
  const int ebits = 32 - __clz(E - 1 > 0 ? E - 1 : 1);
  const int f = c * kGroupThreads + tid;
  const int e = f < n ? ids[f] : -1;
  int pre = 0;
  if (tid < E) {
    int tot = 0;
#pragma unroll 8
    for (int c2 = 0; c2 < nchunks; c2++) {
      const int v = cnt[(size_t)c2 * E + tid];
      tot += v;
      pre += c2 < c ? v : 0;
    }
    s_tot[tid] = tot;
  }
  for (int i = tid; i < kGroupWaves * E; i += kGroupThreads) wavecnt[i / E][i % E] = 0;
  __syncthreads();
  if (tid < 64) {   // exclusive scan of the totals over E <= 256 experts: 4 per lane
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int ee = lane * 4 + q;
      v[q] = ee < E ? s_tot[ee] : 0;
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
      const int ee = lane * 4 + q;
      if (ee < E) {
        s_base[ee] = excl;
        if (c == 0) offsets[ee] = excl;
      }
      excl += v[q];
    }
    if (c == 0 && lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  if (tid < E) s_base[tid] += pre;   // this chunk's first position per expert
  const bool ok = e >= 0 && e < E;
  const uint64_t okm = __ballot(ok);
  uint64_t peers = ok ? okm : 0ull;
  for (int b = 0; b < ebits; b++) {
    const uint64_t m = __ballot(ok && ((e >> b) & 1));
    peers &= ((e >> b) & 1) ? m : ~m;
  }
  const uint64_t below = peers & ((1ull << lane) - 1ull);
  if (ok && below == 0) wavecnt[wave][e] = __popcll(peers);   // wave leader of this expert
  __syncthreads();
  if (ok) {
    int pos = s_base[e] + __popcll(below);
    for (int w = 0; w < wave; w++) pos += wavecnt[w][e];
    sorted_flat[pos] = f;
    flat_to_sorted[f] = pos;
  } else if (f < n) {
    flat_to_sorted[f] = -1;   // id outside [0, E): in no segment
  }
}

size_t group_workspace_bytes(int n, int E) {
  if (n <= kGroupSingleMaxRows) return 0;
  return (size_t)((n + kGroupThreads - 1) / kGroupThreads) * E * sizeof(int32_t);
}

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_flat,
                        int32_t* flat_to_sorted, int32_t* ws, hipStream_t s) {
  const int n = T * k;
  ProfScope prof("group", s);
  if (n <= kGroupSingleMaxRows) {
    EXMOE_LAUNCH(prof, group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, n, E, offsets, sorted_flat,
                 flat_to_sorted);
    return hipGetLastError();
  }
  if (!ws) return hipErrorInvalidValue;
  const int nchunks = (n + kGroupThreads - 1) / kGroupThreads;
  EXMOE_LAUNCH(prof, group_count_kernel, dim3(nchunks), dim3(kGroupThreads), 0, s, ids, n, E, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nchunks <= kGroupScanInScatterChunks) {
    ProfScope p3("group_scatter", s);
    EXMOE_LAUNCH(p3, group_scan_scatter_kernel, dim3(nchunks), dim3(kGroupThreads), 0, s, ids, n, E, ws, offsets,
                 sorted_flat, flat_to_sorted);
    return hipGetLastError();
  }
  {
    ProfScope p2("group_scan", s);
    EXMOE_LAUNCH(p2, group_scan_kernel, dim3(1), dim3(256), 0, s, ws, nchunks, E, offsets);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope p3("group_scatter", s);
    EXMOE_LAUNCH(p3, group_scatter_kernel, dim3(nchunks), dim3(kGroupThreads), 0, s, ids, n, E, ws, sorted_flat,
                 flat_to_sorted);
  }
  return hipGetLastError();
}

}  // namespace exmoe
