// Sequential W4 reference path (EXMOE_PATH_SEQUENTIAL): the active experts one after
// another in ascending id, each with a gate/up launch and a down launch of its own, the
// comparison point of the pages' fused kernel (ExactMoE, Abstract: fused against
// sequential execution of the same int4 experts at 16 tokens).
//
// One expert's weights are small (3.2 MB for the OLMoE shape): a per-expert launch is
// bound by its latency chain, not by the bytes. Each launch therefore puts many waves on
// every row block and keeps the chain short: workgroup = RB row blocks of 16 outputs x WPR
// waves each (16 waves), each wave taking gpw of the row block's input groups (one 1 KiB
// tile per output matrix and group) with every load issued at once, straight from memory
// into registers (weights, scales and the activation fragments of the rows); the waves'
// sums meet in LDS, added in wave order (fixed, so repeated calls are bit-identical), and
// the first wave of each row block finishes its rows: SiLU(gate) * up rounded to bf16
// (gate/up), or the routing weight times the row into y_perm (down). At most 16 rows per
// launch (one MFMA column block).
#include "device.h"
#include "moe_seq.h"

namespace exmoe {

constexpr int kSeqWaves = 16;

// Waves per row block (a power of two, at most 16), row blocks per workgroup and input
// groups per wave for a reduction of G groups.
static void seq_shape(int G, int& wpr, int& rbw, int& gpw) {
  wpr = 1;
  while (wpr < kSeqWaves && wpr < G) wpr *= 2;
  rbw = kSeqWaves / wpr;
  gpw = (G + wpr - 1) / wpr;
}

// GATEUP: outputs = the I rows of gate and up, reduction over H (x rows of the tokens);
// else outputs = the H rows of down, reduction over I (h rows). Rows seg0 .. seg0 + cnt - 1
// of the expert's sorted segment (cnt <= 16).
template <bool GATEUP>
__global__ __launch_bounds__(64 * kSeqWaves) void seq_expert_kernel(MoeArgs a, int e, int seg0, int cnt, int wpr,
                                                                  int gpw) {
  __shared__ f32x4 red[kSeqWaves][2][64];
  constexpr int NM = GATEUP ? 2 : 1;   // output matrices of a row block
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  span_begin(a.span);
  const int rbw = kSeqWaves / wpr;
  const int nrb = (GATEUP ? a.I : a.H) / kTileRows;
  const int rb = blockIdx.x * rbw + wave / wpr, kp = wave % wpr;
  const int K = GATEUP ? a.H : a.I;
  const int G = K / kGroup;
  const int slot = a.e2s ? __builtin_amdgcn_readfirstlane(a.e2s[e]) : e;
  if (slot < 0) {
    if (blockIdx.x == 0 && threadIdx.x == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
    return;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  const uint4* tiles = reinterpret_cast<const uint4*>(blob);
  const uint8_t* scales = blob + n_tiles(a.H, a.I) * kTileBytes;
  // tile of (matrix m, group g): gate/up tiles (2 rb + m) G + g; down tiles after them
  const int rbc = rb < nrb ? rb : nrb - 1;
  const size_t tb0 = GATEUP ? (size_t)(rbc * 2) * G : 2 * (size_t)(a.I / kTileRows) * (a.H / kGroup) + (size_t)rbc * G;

  // the lane's row (B operand column and C column) and its source row
  const int r = lane & 15, kq = lane >> 4;
  const bool live = r < cnt;
  int f = -1;
  if (live) f = a.sorted_flat[seg0 + r];
  const uint16_t* src = GATEUP ? a.x + (size_t)(live ? f / a.k : 0) * a.H : a.h + (size_t)(seg0 + (live ? r : 0)) * a.I;

  f32x4 acc[NM];
#pragma unroll
  for (int m = 0; m < NM; m++) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int g0 = kp * gpw;
  const int ng = rb < nrb ? (G - g0 < gpw ? G - g0 : gpw) : 0;
  for (int i = 0; i < ng; i++) {
    const int g = g0 + i;
    uint4 w[NM];
    uint2 sc[NM];
#pragma unroll
    for (int m = 0; m < NM; m++) {
      const size_t t = tb0 + (size_t)m * G + g;
      w[m] = tiles[t * (kTileBytes / 16) + lane];
      sc[m] = *reinterpret_cast<const uint2*>(scales + t * kScaleBytes + 8 * kq);
    }
    bf16x8 act[4];
#pragma unroll
    for (int q = 0; q < 4; q++)
      act[q] = live ? *reinterpret_cast<const bf16x8*>(src + g * kGroup + 32 * q + 8 * kq) : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    // -136 times the group's activation sum of the lane's column: the lane's 32 values,
    // then the four lanes of the column (each lane adds the same pairs, so all agree)
    float xs = 0.f;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const i32x4 v = __builtin_bit_cast(i32x4, act[q]);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        xs += __uint_as_float((uint32_t)v[j] << 16);
        xs += __uint_as_float((uint32_t)v[j] & 0xFFFF0000u);
      }
    }
    xs += __shfl_xor(xs, 16);
    xs += __shfl_xor(xs, 32);
    const float sd = -136.0f * xs;
#pragma unroll
    for (int m = 0; m < NM; m++) {
      f32x4 c = {sd, sd, sd, sd};
      c = mfma16(dequant_word(w[m].x), act[0], c);
      c = mfma16(dequant_word(w[m].y), act[1], c);
      c = mfma16(dequant_word(w[m].z), act[2], c);
      c = mfma16(dequant_word(w[m].w), act[3], c);
      scale_accum(acc[m], c, sc[m]);
    }
  }
  // the row block's waves' sums, added in wave order by its first wave
#pragma unroll
  for (int m = 0; m < NM; m++) red[wave][m][lane] = acc[m];
  __syncthreads();
  // exactness counter: the down launch's first workgroup counts the rows
  if (!GATEUP && a.rows_ctr && blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(a.rows_ctr + e, cnt);
  if (kp == 0 && rb < nrb) {
#pragma unroll
    for (int m = 0; m < NM; m++)
      for (int w2 = 1; w2 < wpr; w2++) acc[m] += red[wave + w2][m][lane];
    if (live) {
      if (GATEUP) {
        uint2 pk;
        pk.x = pack_bf16x2(silu_mul(acc[0][0], acc[NM - 1][0]), silu_mul(acc[0][1], acc[NM - 1][1]));
        pk.y = pack_bf16x2(silu_mul(acc[0][2], acc[NM - 1][2]), silu_mul(acc[0][3], acc[NM - 1][3]));
        *reinterpret_cast<uint2*>(a.h + (size_t)(seg0 + r) * a.I + rb * kTileRows + 4 * kq) = pk;
      } else {
        const float wt = a.w[f];
        *reinterpret_cast<float4*>(a.y_perm + (size_t)f * a.H + rb * kTileRows + 4 * kq) =
            make_float4(acc[0][0] * wt, acc[0][1] * wt, acc[0][2] * wt, acc[0][3] * wt);
      }
    }
  }
  span_end(a.span);
}

hipError_t launch_seq_expert(const MoeArgs& a, int e, int seg0, int cnt, hipStream_t st) {
  if (cnt <= 0 || cnt > kSeqMaxRows) return hipErrorInvalidValue;
  int wpr, rbw, gpw;
  {
    seq_shape(a.H / kGroup, wpr, rbw, gpw);
    const int nrb = a.I / kTileRows;
    ProfScope prof("seq_gateup", st);
    MoeArgs as = a;
    as.span = prof.span();
    EXMOE_LAUNCH(prof, seq_expert_kernel<true>, dim3((nrb + rbw - 1) / rbw), dim3(64 * kSeqWaves), 0, st, as, e, seg0,
                 cnt, wpr, gpw);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  {
    seq_shape(a.I / kGroup, wpr, rbw, gpw);
    const int nrb = a.H / kTileRows;
    ProfScope prof("seq_down", st);
    MoeArgs as = a;
    as.span = prof.span();
    EXMOE_LAUNCH(prof, seq_expert_kernel<false>, dim3((nrb + rbw - 1) / rbw), dim3(64 * kSeqWaves), 0, st, as, e, seg0,
                 cnt, wpr, gpw);
  }
  return hipGetLastError();
}

}  // namespace exmoe
