// Sequential W4 reference path: the per-expert launch pair of moe_seq.hip.
#pragma once

#include "common.h"

namespace exmoe {

// An expert with at most kSeqMaxRows rows (sorted rows seg0 .. seg0 + cnt - 1): a gate/up
// and a down launch with many waves on each row block and a short latency chain.
constexpr int kSeqMaxRows = 16;
hipError_t launch_seq_expert(const MoeArgs& a, int e, int seg0, int cnt, hipStream_t s);

}  // namespace exmoe
