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

hipError_t launch_group(const int32_t* ids, int T, int k, int E, int32_t* offsets, int32_t* sorted_flat,
                        int32_t* flat_to_sorted, hipStream_t s) {
  ProfScope prof("group", s);
  EXMOE_LAUNCH(prof, group_kernel, dim3(1), dim3(kGroupThreads), 0, s, ids, T * k, E, offsets,
                     sorted_flat, flat_to_sorted);
  return hipGetLastError();
}

}  // namespace exmoe
