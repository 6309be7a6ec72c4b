// Prefill-sized expert layer (many tokens per expert): grouped GEMMs on bf16 MFMA, gfx950.
//
// Every selected expert runs over the tokens grouped to it (ExactMoE abstract; Fig. 1).
// One workgroup (8 waves) computes a 256-row x 128-token output tile of one expert:
//   gate/up: rows = 128 gate rows + the matching 128 up rows (one 128-wide slice of the
//            intermediate dimension), epilogue h = bf16(silu(g) * u) plus the fp32 sum of
//            each token's 128 rounded h values (the next kernel's dequant correction);
//   down:    rows = 256 output rows, epilogue y_perm = o * routing weight (fp32), stored in
//            flat (token, slot) order for the combine.
// The activation tile of each 128-input group is gathered (gate/up: through the token
// permutation) into LDS, double-buffered, rows padded to 272 B so that the 16 tokens of a
// fragment read hit distinct banks. Packed int4 tiles go straight from HBM to registers
// (one 1 KiB tile per wave-wide 128-bit load, prefetched a group ahead) and are turned
// into exact bf16 operands 128 + u in registers. Each group's MFMA chain starts from
// -136 * (group sum of the activations), so it ends at sum(x * q); the bf16 scale of the
// row is applied once per group in fp32. Waves: 4 along rows x 2 along tokens; each wave
// owns 4 x 4 tiles of 16 x 16.
#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kPfThreads = 512;
constexpr int kPfBN = 128;                 // tokens per workgroup tile
constexpr int kPfRows = 256;               // output rows per workgroup tile
constexpr int kLdsStride = kGroup + 8;     // bf16 elements per LDS row (272 B)

// All-zero row read for rows past a segment's end (device globals start zeroed; never
// written).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row_pf[kMaxDim];

// Which expert / token tile / row tile this workgroup owns. Token tiles are counted per
// expert (ceil(count / 128)); a single wave scans the counts (E <= 256).
struct PfTile {
  int e, seg0, cnt, tok0;
};

__device__ bool pf_resolve(const MoeArgs& a, int fixed_expert, int tt_lin, PfTile& t,
                           int* s_scan) {
  // s_scan: LDS int[kMaxExperts + 1] of exclusive token-tile prefix sums
  const int tid = threadIdx.x;
  if (fixed_expert >= 0) {
    t.e = fixed_expert;
    t.seg0 = a.offsets[t.e];
    t.cnt = a.offsets[t.e + 1] - t.seg0;
    t.tok0 = tt_lin * kPfBN;
    return t.tok0 < t.cnt;
  }
  if (tid < 64) {
    int v[4], run = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      int e = tid * 4 + q;
      v[q] = e < a.E ? (a.offsets[e + 1] - a.offsets[e] + kPfBN - 1) / kPfBN : 0;
      run += v[q];
    }
    int incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (tid >= off) incl += o;
    }
    int excl = incl - run;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      s_scan[tid * 4 + q] = excl;
      excl += v[q];
    }
    if (tid == 63) s_scan[kMaxExperts] = incl;
  }
  __syncthreads();
  if (tt_lin >= s_scan[kMaxExperts]) return false;
  // The owner is the largest e with s_scan[e] <= tt_lin: an empty expert shares its
  // prefix value with the next one, so the largest such e always has tiles.
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_scan[mid] <= tt_lin) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  t.e = e;
  t.seg0 = a.offsets[e];
  t.cnt = a.offsets[e + 1] - t.seg0;
  t.tok0 = (tt_lin - s_scan[e]) * kPfBN;
  return t.tok0 < t.cnt;
}

template <bool GATEUP>
__global__ __launch_bounds__(kPfThreads, 1) void prefill_kernel(MoeArgs a, int fixed_expert,
                                                               int n_row_tiles) {
  __shared__ __attribute__((aligned(16))) uint16_t s_act[2][kPfBN * kLdsStride];
  __shared__ int s_scan[kMaxExperts + 1];
  __shared__ float s_gsum[4][kPfBN];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wr = wave & 3, wt = wave >> 2;
  const int rt = blockIdx.x % n_row_tiles;
  const int tt_lin = blockIdx.x / n_row_tiles;
  PfTile pt;
  if (!pf_resolve(a, fixed_expert, tt_lin, pt, s_scan)) return;
  const int slot = a.e2s ? a.e2s[pt.e] : pt.e;
  if (slot < 0) {
    if (tid == 0) atomicOr(a.debug, 1u);
    return;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  const uint4* tiles = reinterpret_cast<const uint4*>(blob);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blob + n_tiles(a.H, a.I) * kTileBytes);
  const int K = GATEUP ? a.H : a.I;
  const int G = K / kGroup;
  const size_t tile_down0 = 2 * (size_t)(a.I / kTileRows) * (a.H / kGroup);

  // tile index (without the group) of this wave's 4 row subtiles
  size_t tbase[4];
  bool rvalid[4];
#pragma unroll
  for (int ai = 0; ai < 4; ai++) {
    rvalid[ai] = GATEUP || (rt * 16 + 4 * wr + ai) < a.H / kTileRows;
    if (GATEUP) {
      const int rbI = rt * 8 + 2 * wr + (ai >> 1);
      tbase[ai] = (size_t)(rbI * 2 + (ai & 1)) * G;
    } else {
      const int rbH = rt * 16 + 4 * wr + ai;
      tbase[ai] = tile_down0 + (size_t)(rvalid[ai] ? rbH : 0) * G;
    }
  }

  // ---- staging of the activation tile: thread -> (row, 4 chunks of 16 B)
  const int st_row = tid >> 2, st_c = tid & 3;
  const bool st_valid = pt.tok0 + st_row < pt.cnt;
  // Rows past the segment read the zero row: loads stay unconditional, so the compiler
  // counts them exactly and the prefetch stays in flight.
  const uint16_t* st_src = g_zero_row_pf;
  if (st_valid) {
    if (GATEUP)
      st_src = a.x + (size_t)(a.sorted_flat[pt.seg0 + pt.tok0 + st_row] / a.k) * a.H;
    else
      st_src = a.h + (size_t)(pt.seg0 + pt.tok0 + st_row) * a.I;
  }
  uint4 st_reg[4];
  auto stage_load = [&](int g) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      st_reg[i] = *reinterpret_cast<const uint4*>(st_src + g * kGroup + (st_c + 4 * i) * 8);
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; i++)
      *reinterpret_cast<uint4*>(&s_act[buf][st_row * kLdsStride + (st_c + 4 * i) * 8]) = st_reg[i];
  };

  // ---- per-lane token rows of the 4 token subtiles (for the correction sums)
  int crow[4];
  bool cval[4];
#pragma unroll
  for (int bj = 0; bj < 4; bj++) {
    const int r = pt.tok0 + wt * 64 + bj * 16 + (lane & 15);
    cval[bj] = r < pt.cnt;
    if (GATEUP)
      crow[bj] = cval[bj] ? a.sorted_flat[pt.seg0 + r] / a.k : 0;   // token
    else
      crow[bj] = pt.seg0 + (cval[bj] ? r : 0);                       // sorted row
  }
  const float* csum = GATEUP ? a.xsum : a.gsum;

  f32x4 acc[4][4];
#pragma unroll
  for (int ai = 0; ai < 4; ai++)
#pragma unroll
    for (int bj = 0; bj < 4; bj++) acc[ai][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 wcur[4], wnext[4];
  uint2 scur[4], snext[4];
  auto w_load = [&](int g, uint4* w, uint2* s) {
#pragma unroll
    for (int ai = 0; ai < 4; ai++) {
      const size_t t = tbase[ai] + g;
      w[ai] = tiles[t * 64 + lane];
      s[ai] = *reinterpret_cast<const uint2*>(scales + t * 16 + 4 * (lane >> 4));
    }
  };

  stage_load(0);
  w_load(0, wcur, scur);
  stage_store(0);
  __syncthreads();

  for (int g = 0; g < G; g++) {
    const int buf = g & 1;
    const int gn = g + 1 < G ? g + 1 : g;         // the last prefetch repeats a group, harmlessly
    stage_load(gn);
    w_load(gn, wnext, snext);
    // correction seeds: -136 * group sum of each token's activations
    f32x4 tmp[4][4];
#pragma unroll
    for (int bj = 0; bj < 4; bj++) {
      const float cs = csum[(size_t)crow[bj] * G + g];
      const float c = cval[bj] ? -136.0f * cs : 0.f;
#pragma unroll
      for (int ai = 0; ai < 4; ai++) tmp[ai][bj] = f32x4{c, c, c, c};
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      bf16x8 bfr[4];
#pragma unroll
      for (int bj = 0; bj < 4; bj++) {
        const int row = wt * 64 + bj * 16 + (lane & 15);
        const uint4 v = *reinterpret_cast<const uint4*>(&s_act[buf][row * kLdsStride + 32 * s + 8 * (lane >> 4)]);
        i32x4 iv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
        bfr[bj] = __builtin_bit_cast(bf16x8, iv);
      }
#pragma unroll
      for (int ai = 0; ai < 4; ai++) {
        const uint32_t word = s == 0 ? wcur[ai].x : s == 1 ? wcur[ai].y : s == 2 ? wcur[ai].z : wcur[ai].w;
        const bf16x8 afr = dequant_word(word);
#pragma unroll
        for (int bj = 0; bj < 4; bj++) tmp[ai][bj] = mfma16(afr, bfr[bj], tmp[ai][bj]);
      }
    }
#pragma unroll
    for (int ai = 0; ai < 4; ai++)
#pragma unroll
      for (int bj = 0; bj < 4; bj++) scale_accum(acc[ai][bj], tmp[ai][bj], scur[ai]);
    stage_store(buf ^ 1);
#pragma unroll
    for (int ai = 0; ai < 4; ai++) {
      wcur[ai] = wnext[ai];
      scur[ai] = snext[ai];
    }
    __syncthreads();
  }

  // ---- epilogue
  if (GATEUP) {
    float gpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rbl = 0; rbl < 2; rbl++) {
      const int col = (rt * 8 + 2 * wr + rbl) * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int bj = 0; bj < 4; bj++) {
        const f32x4 gv = acc[2 * rbl][bj], uv = acc[2 * rbl + 1][bj];
        uint16_t hb[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          hb[i] = f32_to_bf16(gv[i] / (1.0f + expf(-gv[i])) * uv[i]);
          gpart[bj] += bf16_to_f32(hb[i]);
        }
        const int r = pt.tok0 + wt * 64 + bj * 16 + (lane & 15);
        if (r < pt.cnt) {
          uint2 pk;
          pk.x = (uint32_t)hb[0] | ((uint32_t)hb[1] << 16);
          pk.y = (uint32_t)hb[2] | ((uint32_t)hb[3] << 16);
          *reinterpret_cast<uint2*>(a.h + (size_t)(pt.seg0 + r) * a.I + col) = pk;
        }
      }
    }
    // per-token sum over this workgroup's 128 intermediate columns (one down group)
#pragma unroll
    for (int bj = 0; bj < 4; bj++) {
      float v = gpart[bj];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (lane < 16) s_gsum[wr][wt * 64 + bj * 16 + lane] = v;
    }
    __syncthreads();
    if (tid < kPfBN) {
      const int r = pt.tok0 + tid;
      if (r < pt.cnt) {
        const float v = ((s_gsum[0][tid] + s_gsum[1][tid]) + s_gsum[2][tid]) + s_gsum[3][tid];
        a.gsum[(size_t)(pt.seg0 + r) * (a.I / kGroup) + rt] = v;
      }
    }
  } else {
#pragma unroll
    for (int bj = 0; bj < 4; bj++) {
      const int r = pt.tok0 + wt * 64 + bj * 16 + (lane & 15);
      if (r < pt.cnt) {
        const int f = a.sorted_flat[pt.seg0 + r];     // y_perm rows are in flat (token, slot) order
        const float wgt = a.w[f];
#pragma unroll
        for (int ai = 0; ai < 4; ai++) {
          if (!rvalid[ai]) continue;
          const int col = (rt * 16 + 4 * wr + ai) * 16 + 4 * (lane >> 4);
          const f32x4 o = acc[ai][bj];
          *reinterpret_cast<float4*>(a.y_perm + (size_t)f * a.H + col) =
              make_float4(o[0] * wgt, o[1] * wgt, o[2] * wgt, o[3] * wgt);
        }
      }
    }
  }
}

// Group sums of x in fp32 (one wave per token row of 128-wide groups): xsum[t, g].
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                   float* __restrict__ xsum) {
  const int G = H / kGroup;
  const int i = blockIdx.x * 256 + threadIdx.x;     // one (token, group) per thread
  if (i >= T * G) return;
  const int t = i / G, g = i % G;
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * H + g * kGroup);
  float s = 0.f;
#pragma unroll 4
  for (int c = 0; c < kGroup / 8; c++) {
    const uint4 v = p[c];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; q++) s += __uint_as_float(w[q] << 16) + __uint_as_float(w[q] & 0xFFFF0000u);
  }
  xsum[i] = s;
}

hipError_t launch_moe_prefill(const MoeArgs& a, hipStream_t s) {
  const int TK = a.T * a.k;
  const int max_tt = TK / kPfBN + (a.E < TK ? a.E : TK);
  const int G = a.H / kGroup;
  {
    ProfScope prof("xsum", s);
    hipLaunchKernelGGL(xsum_kernel, dim3((a.T * G + 255) / 256), dim3(256), 0, s, a.x, a.T, a.H, a.xsum);
  }
  const int rt_gu = a.I / 128;
  {
    ProfScope prof("prefill_gateup", s);
    hipLaunchKernelGGL(prefill_kernel<true>, dim3(max_tt * rt_gu), dim3(kPfThreads), 0, s, a, -1, rt_gu);
  }
  const int rt_d = (a.H + kPfRows - 1) / kPfRows;
  {
    ProfScope prof("prefill_down", s);
    hipLaunchKernelGGL(prefill_kernel<false>, dim3(max_tt * rt_d), dim3(kPfThreads), 0, s, a, -1, rt_d);
  }
  return launch_combine(a, s);
}

}  // namespace exmoe
