// Prefill-sized expert layer (many tokens per expert): grouped GEMMs on bf16 MFMA, gfx950.
//
// Every selected expert runs over the tokens grouped to it (ExactMoE abstract; Fig. 1).
// A workgroup computes a 256-row x BN-token output tile of one expert. int4 experts take
// BN = 64 on 4 waves (one per SIMD, two workgroups per compute unit), each wave owning 64
// rows (four 16-row subtiles) x all 64 tokens; the bf16 comparator takes BN = 128 on 8
// waves (two per SIMD), each owning 32 rows x all 128 tokens. The rows:
//   gate/up: rows = 128 gate rows + the matching 128 up rows (one 128-wide slice of the
//            intermediate dimension), epilogue h = bf16(silu(g) * u) plus the fp32 sum of
//            each token's 128 rounded h values (the down kernel's dequant correction);
//   down:    rows = 256 output rows, epilogue y_perm = o * routing weight (fp32), stored in
//            flat (token, slot) order for the combine.
// The activation tile of each 128-input group goes straight from memory into LDS
// (global_load_lds, gate/up gathered through the token permutation), double-buffered; the
// 16-byte chunks of row r sit at position chunk ^ (r mod 16), so the 16 rows of a fragment
// read hit distinct banks. Packed int4 tiles go from HBM to registers (one 1 KiB tile per
// wave-wide 128-bit load, prefetched a group ahead) and become exact bf16 operands 128 + u
// in registers. Each group's MFMA chain starts from -136 * (group sum of the activations:
// per token for gate/up, per routed row of h for down), so it ends at sum(x * q); the bf16
// scale of the row is applied once per group in fp32. A wave dequantizes its row subtiles
// of a group once and reuses them across all token subtiles of the tile (16 tokens each).
// Q4 = false runs the same loop on dense bf16 experts (the comparator): the weight
// fragments are loaded as they are, with no scales and no seeds.
#include <type_traits>

#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kPfBN = 128;                 // tokens per token tile of the bf16 comparator (and the down seeds' row padding)
constexpr int kPfWaves = 8;                // waves per workgroup of the bf16 comparator (2 row subtiles each)
constexpr int kPfRows = 256;               // output rows per workgroup tile
constexpr int kLdsStride = kGroup;         // bf16 elements per LDS row (256 B; 16-byte chunks swizzled)

// All-zero row read for rows past a segment's end (device globals start zeroed; never
// written).
__device__ __attribute__((aligned(16))) uint16_t g_zero_row_pf[kMaxDim];

// Which expert / token tile / row tile this workgroup owns. Token tiles are counted per
// expert (ceil(count / 128)); the full tiles of every expert come first (in expert
// order), then the ragged last tiles: workgroups are dispatched in index order, so the
// long ones start first and the short ones fill in behind them (under skewed routing
// the full tiles of the popular experts would otherwise end the launch alone). A single
// wave scans the counts (E <= 256).
struct PfTile {
  int e, seg0, cnt, tok0;
};

template <int BN>
__device__ bool pf_resolve(const MoeArgs& a, int fixed_expert, int tt_lin, PfTile& t,
                           int* s_full, int* s_part, int* s_off) {
  // s_full / s_part: LDS int[kMaxExperts + 1] of exclusive prefix sums of the full tiles
  // and of the ragged tiles (0 or 1) per expert; s_off: LDS int[kMaxExperts + 1], the
  // segment offsets (loaded once, all at a time)
  const int tid = threadIdx.x;
  if (fixed_expert >= 0) {
    t.e = fixed_expert;
    t.seg0 = a.offsets[t.e];
    t.cnt = a.offsets[t.e + 1] - t.seg0;
    t.tok0 = tt_lin * BN;
    return t.tok0 < t.cnt;
  }
  if (tid < 64) {
    int o[5];
#pragma unroll
    for (int q = 0; q < 5; q++) {   // offsets 4 tid .. 4 tid + 4, clamped: every load at once
      const int e = tid * 4 + q;
      o[q] = a.offsets[e <= a.E ? e : a.E];
    }
    int vf[4], vp[4], run_f = 0, run_p = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int e = tid * 4 + q;
      const int c = e < a.E ? o[q + 1] - o[q] : 0;
      vf[q] = c / BN;
      vp[q] = c % BN != 0 ? 1 : 0;
      run_f += vf[q];
      run_p += vp[q];
      s_off[e] = o[q];
    }
    if (tid == 63) s_off[kMaxExperts] = o[4];
    int incl_f = run_f, incl_p = run_p;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int uf = __shfl_up(incl_f, off, 64), up = __shfl_up(incl_p, off, 64);
      if (tid >= off) {
        incl_f += uf;
        incl_p += up;
      }
    }
    int ef = incl_f - run_f, ep = incl_p - run_p;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      s_full[tid * 4 + q] = ef;
      s_part[tid * 4 + q] = ep;
      ef += vf[q];
      ep += vp[q];
    }
    if (tid == 63) {
      s_full[kMaxExperts] = incl_f;
      s_part[kMaxExperts] = incl_p;
    }
  }
  __syncthreads();
  const int nfull = s_full[kMaxExperts];
  const bool full = tt_lin < nfull;
  const int idx = full ? tt_lin : tt_lin - nfull;
  const int* scan = full ? s_full : s_part;
  if (!full && idx >= s_part[kMaxExperts]) return false;
  // The owner is the largest e with scan[e] <= idx: an expert without such tiles shares
  // its prefix value with the next one, so the largest such e always has one.
  int lo = 0, hi = a.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (scan[mid] <= idx) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  t.e = e;
  t.seg0 = s_off[e];
  t.cnt = s_off[e + 1] - t.seg0;
  t.tok0 = full ? (idx - s_full[e]) * BN : t.cnt / BN * BN;
  return t.tok0 < t.cnt;
}

// One wave-wide global -> LDS copy (global_load_lds): lane l reads 16 (or 4) bytes at its
// own address; they land at dst + 16 l (or 4 l). Completion is counted like a load.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 4, 0, 0);
}

// NW waves per workgroup; each wave owns NA = 16 / NW row subtiles (of 16 rows) and all
// BN / 16 token subtiles of the 256 x BN tile. Tokens are the M operand of the MFMA and
// weight rows the N operand, so a lane's 4 accumulator values belong to one weight row
// (one scale) and 4 consecutive tokens (one float4 of correction seeds). 8 / NW waves per
// SIMD: with NW = 4, two workgroups share a compute unit.
// Q4 = false: the bank holds dense bf16 experts (the comparator), 1 KiB tiles of 16 rows x
// 32 columns in operand order, four per 128-column group; no scales and no seeds.
template <bool GATEUP, int NW, int BN, bool Q4>
__global__ __launch_bounds__(NW * 64, 8 / NW) void prefill_kernel(MoeArgs a, int fixed_expert,
                                                                int n_row_tiles) {
  constexpr int NT = NW * 64;            // threads
  constexpr int NA = 16 / NW;            // row subtiles per wave
  constexpr int NL = Q4 ? 1 : 4;         // 16-byte weight loads per lane, row subtile and group
  constexpr int NB = BN / 16;            // token subtiles per wave (all of the tile's tokens)
  constexpr int NP = NB / 2;             // token subtile pairs
  constexpr int kSeedWaves = BN / 64;    // waves that stage the correction seeds (64 each)
  // two buffers as separate arrays: the compiler then sees that reading one does not wait
  // for the copies into the other
  __shared__ __attribute__((aligned(16))) uint16_t s_act0[BN * kLdsStride], s_act1[BN * kLdsStride];
  __shared__ __attribute__((aligned(16))) float s_seed0[BN], s_seed1[BN];
  __shared__ int s_full[kMaxExperts + 1], s_part[kMaxExperts + 1], s_off[kMaxExperts + 1];
  __shared__ __attribute__((aligned(16))) float s_gsum[NW][BN];

  span_begin(a.span);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: tile addresses stay scalar
  const int rt = blockIdx.x % n_row_tiles;
  const int tt_lin = blockIdx.x / n_row_tiles;
  PfTile pt;
  if (!pf_resolve<BN>(a, fixed_expert, tt_lin, pt, s_full, s_part, s_off)) return;
  const int slot = a.e2s ? a.e2s[pt.e] : pt.e;
  if (slot < 0) {
    if (tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
    return;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  const uint4* tiles = reinterpret_cast<const uint4*>(blob);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(blob + (Q4 ? n_tiles(a.H, a.I) * kTileBytes : 0));
  const int K = GATEUP ? a.H : a.I;
  const int G = K / kGroup;
  const size_t tile_down0 = 2 * (size_t)(a.I / kTileRows) * (a.H / kGroup);
  const int rows_pad = a.T * a.k + kPfBN;          // row count of the down kernel's seed array

  // tile index (without the group) of this wave's NA row subtiles; gate/up subtiles come
  // in (gate, up) pairs of one 16-row block of the intermediate dimension
  size_t tbase[NA];
  bool rvalid[NA];
#pragma unroll
  for (int ai = 0; ai < NA; ai++) {
    if (GATEUP) {
      rvalid[ai] = true;
      const int rbI = rt * 8 + (NA / 2) * wave + (ai >> 1);
      tbase[ai] = (size_t)(rbI * 2 + (ai & 1)) * G;
    } else {
      const int rbH = rt * 16 + NA * wave + ai;
      rvalid[ai] = rbH < a.H / kTileRows;
      tbase[ai] = tile_down0 + (size_t)(rvalid[ai] ? rbH : 0) * G;
    }
  }

  // ---- staging of the activation tile (and the group's correction seeds), straight from
  // memory into LDS (global_load_lds, 16 bytes per lane): each wave moves kDmaPerWave
  // pieces of 4 rows x 256 bytes per group. Chunk c (16 bytes) of row r lands at position
  // c ^ (r mod 16) of the row, so that the 16 rows of a fragment read hit distinct banks.
  // Rows past the segment read the zero row.
  // (the gathered row indices are loaded at clamped positions, all at once, and the rows
  // past the segment are then pointed at the zero row)
  constexpr int kDmaPerWave = BN / 4 / NW;
  // Every index load of the set-up is issued at once, then the first group's weights
  // behind them, so that waiting for the indices leaves the weight loads in flight:
  //   gate/up: the gathered rows of the wave's copies and the token of the lane's seed row;
  //   down: the flat (token, slot) index of each of the tile's rows (for the epilogue).
  // (the clamped positions are hidden from the optimizer: where it can prove a position
  // unclamped it issues a second load there, late and waited for on its own)
  auto row_index = [&](int r) {
    int rr = r < pt.cnt ? r : pt.cnt - 1;
    asm volatile("" : "+v"(rr));
    return a.sorted_flat[pt.seg0 + rr];
  };
  int grow[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; i++)
    grow[i] = GATEUP ? row_index(pt.tok0 + (wave * kDmaPerWave + i) * 4 + (lane >> 4)) : 0;
  const int seed_r = pt.tok0 + (wave % kSeedWaves) * 64 + lane;
  int srow = 0;
  if (GATEUP && Q4) srow = row_index(seed_r);
  int fr_l = 0;
  if (!GATEUP && wave < BN / 64) fr_l = row_index(pt.tok0 + tid);

  uint4 wcur[NA][NL], wnext[NA][NL];
  uint32_t scur[NA], snext[NA];
#pragma unroll
  for (int ai = 0; ai < NA; ai++) {
    const size_t t = tbase[ai];
#pragma unroll
    for (int q = 0; q < NL; q++) wcur[ai][q] = tiles[(t * NL + q) * 64 + lane];
    if (Q4) scur[ai] = scales[t * 16 + (lane & 15)];
  }

  // flat (token, slot) index -> token: a high multiply by floor((2^32 - 1) / k) gives the
  // quotient or one less (for any 32-bit index), and one compare corrects it
  const uint32_t kmul = 0xFFFFFFFFu / (uint32_t)a.k;
  auto tok_of = [&](int flat) {
    uint32_t q = __umulhi((uint32_t)flat, kmul);
    if ((uint32_t)flat - q * (uint32_t)a.k >= (uint32_t)a.k) q++;
    return (int)q;
  };
  const uint16_t* drow[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; i++) {
    const int r = (wave * kDmaPerWave + i) * 4 + (lane >> 4);
    const uint16_t* src = g_zero_row_pf;
    if (pt.tok0 + r < pt.cnt) {
      if (GATEUP)
        src = a.x + (size_t)tok_of(grow[i]) * a.H;
      else
        src = a.h + (size_t)(pt.seg0 + pt.tok0 + r) * a.I;
    }
    drow[i] = src + (((lane & 15) ^ (r & 15)) * 8);
  }
  // correction seeds, already * -136: gate/up per token (xsum[group][token]), each lane
  // gathering its row's token (rows past the segment take token 0: their outputs are not
  // stored); down per sorted row (gsum[group][row], rows padded by one tile)
  const float* seed_src;
  size_t seed_stride;
  if (GATEUP) {
    seed_src = a.xsum + (seed_r < pt.cnt ? tok_of(srow) : 0);
    seed_stride = (size_t)a.T;
  } else {
    seed_src = a.gsum + pt.seg0 + pt.tok0 + (wave % kSeedWaves) * 64 + lane;
    seed_stride = (size_t)rows_pad;
  }
#define EXMOE_STAGE(g_, ACT, SEED)                                                                      \
  do {                                                                                                  \
    _Pragma("unroll") for (int i = 0; i < kDmaPerWave; i++)                                             \
        dma16(drow[i] + (g_) * kGroup, &ACT[(wave * kDmaPerWave + i) * 4 * kLdsStride]);                \
    if (Q4 && wave < kSeedWaves) dma4(seed_src + (size_t)(g_) * seed_stride, &SEED[wave * 64]);         \
  } while (0)

  f32x4 acc[NA][NB];
#pragma unroll
  for (int ai = 0; ai < NA; ai++)
#pragma unroll
    for (int bj = 0; bj < NB; bj++) acc[ai][bj] = f32x4{0.f, 0.f, 0.f, 0.f};

  EXMOE_STAGE(0, s_act0, s_seed0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // down: the tile's flat row indices and routing weights for the epilogue go to LDS (the
  // gate/up kernel's group-sum rows); the weights' loads run behind the first group
  int* const s_fr = reinterpret_cast<int*>(s_gsum[0]);
  float* const s_wr = s_gsum[1];
  float wr_l = 0.f;
  if (!GATEUP && wave < BN / 64) {
    s_fr[tid] = fr_l;
    wr_l = a.w[fr_l];
  }

  // Token subtile pairs (32 tokens) that hold rows of the segment: the last token tile of
  // an expert is often mostly padding, and its MFMAs on padding rows are skipped.
  const int npairs = pt.cnt - pt.tok0 >= BN ? NP : (pt.cnt - pt.tok0 + 31) / 32;

  // One group: compute it from (cact, cseed) while the next one lands in (nact, nseed).
  // full: every pair holds rows (no skip tests in the MFMA stream).
  auto group = [&](auto full, int g_, const uint16_t* cact, const float* cseed, uint16_t* nact, float* nseed) {
    const int gn = g_ + 1 < G ? g_ + 1 : g_;   // the last prefetch repeats a group, harmlessly
    // the next group's activations and seeds into the other buffer, its weights into
    // registers; everything is waited for once, at the end of this group
    EXMOE_STAGE(gn, nact, nseed);
#pragma unroll
    for (int ai = 0; ai < NA; ai++) {
      const size_t t = tbase[ai] + gn;
#pragma unroll
      for (int q = 0; q < NL; q++) wnext[ai][q] = tiles[(t * NL + q) * 64 + lane];
      if (Q4) snext[ai] = scales[t * 16 + (lane & 15)];
    }
    __builtin_amdgcn_sched_barrier(0);
    // weight fragments of the group (dequantized once): [row subtile][K step]
    bf16x8 wfr[NA][4];
#pragma unroll
    for (int ai = 0; ai < NA; ai++) {
      if (Q4) {
        wfr[ai][0] = dequant_word(wcur[ai][0].x);
        wfr[ai][1] = dequant_word(wcur[ai][0].y);
        wfr[ai][2] = dequant_word(wcur[ai][0].z);
        wfr[ai][3] = dequant_word(wcur[ai][0].w);
      } else {
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const uint4 v = wcur[ai][Q4 ? 0 : q];
          i32x4 iv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
          wfr[ai][q] = __builtin_bit_cast(bf16x8, iv);
        }
      }
    }
    float sc[NA];
#pragma unroll
    for (int ai = 0; ai < NA; ai++) sc[ai] = Q4 ? __uint_as_float(scur[ai] << 16) : 1.0f;
    // token subtiles in pairs: activation fragments of both for all 4 K steps
#pragma unroll
    for (int p = 0; p < NP; p++) {
      if constexpr (!decltype(full)::value) {
        if (p >= npairs) break;
      }
      bf16x8 xfr[2][4];
      f32x4 seed[2];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int row = (2 * p + j) * 16 + (lane & 15);
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) {
          const uint4 v = *reinterpret_cast<const uint4*>(
              &cact[row * kLdsStride + (((4 * s4 + (lane >> 4)) ^ (row & 15)) * 8)]);
          i32x4 iv = {(int)v.x, (int)v.y, (int)v.z, (int)v.w};
          xfr[j][s4] = __builtin_bit_cast(bf16x8, iv);
        }
        // seeds of tokens 4(l/16)+0..3 of the subtile: -136 * group sum of their activations
        if (Q4) seed[j] = *reinterpret_cast<const f32x4*>(&cseed[(2 * p + j) * 16 + 4 * (lane >> 4)]);
      }
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int bj = 2 * p + j;
#pragma unroll
        for (int ai = 0; ai < NA; ai++) {
          if (Q4) {
            f32x4 t = mfma16(xfr[j][0], wfr[ai][0], seed[j]);
            t = mfma16(xfr[j][1], wfr[ai][1], t);
            t = mfma16(xfr[j][2], wfr[ai][2], t);
            t = mfma16(xfr[j][3], wfr[ai][3], t);
#pragma unroll
            for (int i = 0; i < 4; i++) acc[ai][bj][i] += sc[ai] * t[i];
          } else {   // bf16 weights: one chain straight into the accumulator
            f32x4 t = mfma16(xfr[j][0], wfr[ai][0], acc[ai][bj]);
            t = mfma16(xfr[j][1], wfr[ai][1], t);
            t = mfma16(xfr[j][2], wfr[ai][2], t);
            acc[ai][bj] = mfma16(xfr[j][3], wfr[ai][3], t);
          }
        }
      }
    }
    // the next group has landed (LDS and registers) and every wave is done with this one
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int ai = 0; ai < NA; ai++) {
#pragma unroll
      for (int q = 0; q < NL; q++) wcur[ai][q] = wnext[ai][q];
      scur[ai] = snext[ai];
    }
  };
  if (npairs == NP) {
    for (int g = 0; g < G; g += 2) {
      group(std::true_type{}, g, s_act0, s_seed0, s_act1, s_seed1);
      if (g + 1 < G) group(std::true_type{}, g + 1, s_act1, s_seed1, s_act0, s_seed0);
    }
  } else {
    for (int g = 0; g < G; g += 2) {
      group(std::false_type{}, g, s_act0, s_seed0, s_act1, s_seed1);
      if (g + 1 < G) group(std::false_type{}, g + 1, s_act1, s_seed1, s_act0, s_seed0);
    }
  }
#undef EXMOE_STAGE

  // ---- epilogue: lane l holds weight row (l % 16) of each row subtile and tokens
  // bj*16 + 4(l/16) + i of each token subtile
  const int tl0 = 4 * (lane >> 4);
  if (GATEUP) {
    float gpart[NB][4];
#pragma unroll
    for (int bj = 0; bj < NB; bj++)
#pragma unroll
      for (int i = 0; i < 4; i++) gpart[bj][i] = 0.f;
#pragma unroll
    for (int rbl = 0; rbl < NA / 2; rbl++) {
      const int col = (rt * 8 + (NA / 2) * wave + rbl) * 16 + (lane & 15);
      // this lane's first h row; its other rows follow at multiples of I. A full tile
      // stores without row tests.
      uint16_t* hrow = a.h + (size_t)(pt.seg0 + pt.tok0 + tl0) * a.I + col;
      const int nv = pt.cnt - pt.tok0 - tl0;
      auto store = [&](auto full) {
#pragma unroll
        for (int bj = 0; bj < NB; bj++) {
          const f32x4 gv = acc[2 * rbl][bj], uv = acc[2 * rbl + 1][bj];
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const uint16_t hb = f32_to_bf16(silu_mul(gv[i], uv[i]));
            gpart[bj][i] += bf16_to_f32(hb);
            const int rr = bj * 16 + i;
            if (decltype(full)::value || rr < nv) hrow[(size_t)rr * a.I] = hb;
          }
        }
      };
      if (pt.cnt - pt.tok0 >= BN) store(std::true_type{});
      else store(std::false_type{});
    }
    // per-token sum over this workgroup's 128 intermediate columns (one down group):
    // the 16 lanes of a row hold 16 columns each (the int4 down kernel's correction)
    // (row rotations by 1, 2, 4 and 8, each step over all 32 values before the next, so
    // that the steps of different values interleave; lane 0 of each row then writes them)
    if (Q4) {
    auto rot_add = [&](auto ctrl) {
#pragma unroll
      for (int bj = 0; bj < NB; bj++)
#pragma unroll
        for (int i = 0; i < 4; i++)
          gpart[bj][i] += __uint_as_float(dpp_u32<decltype(ctrl)::value>(__float_as_uint(gpart[bj][i])));
    };
    rot_add(std::integral_constant<int, 0x121>{});
    rot_add(std::integral_constant<int, 0x122>{});
    rot_add(std::integral_constant<int, 0x124>{});
    rot_add(std::integral_constant<int, 0x128>{});
    if ((lane & 15) == 0) {
#pragma unroll
      for (int bj = 0; bj < NB; bj++)
        *reinterpret_cast<float4*>(&s_gsum[wave][bj * 16 + tl0]) =
            make_float4(gpart[bj][0], gpart[bj][1], gpart[bj][2], gpart[bj][3]);
    }
    __syncthreads();
    if (tid < BN) {
      const int r = pt.tok0 + tid;
      if (r < pt.cnt) {
        float v = s_gsum[0][tid];
#pragma unroll
        for (int w = 1; w < NW; w++) v += s_gsum[w][tid];
        a.gsum[(size_t)rt * rows_pad + pt.seg0 + r] = -136.0f * v;
      }
    }
    }
  } else {
    // y_perm rows are in flat (token, slot) order; the row indices and routing weights of
    // the tile's rows were loaded during the set-up (rows past the segment hold the last
    // row's, unused)
    if (wave < BN / 64) s_wr[tid] = wr_l;
    __syncthreads();
#pragma unroll
    for (int bj = 0; bj < NB; bj++) {
      const int4 fr4 = *reinterpret_cast<const int4*>(&s_fr[bj * 16 + tl0]);
      const f32x4 wr4 = *reinterpret_cast<const f32x4*>(&s_wr[bj * 16 + tl0]);
      const int fr[4] = {fr4.x, fr4.y, fr4.z, fr4.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = pt.tok0 + bj * 16 + tl0 + i;
        if (r < pt.cnt) {
#pragma unroll
          for (int ai = 0; ai < NA; ai++) {
            if (!rvalid[ai]) continue;
            const int col = (rt * 16 + NA * wave + ai) * 16 + (lane & 15);
            a.y_perm[(size_t)fr[i] * a.H + col] = acc[ai][bj][i] * wr4[i];
          }
        }
      }
    }
    // exactness counter: the first row tile of each token tile counts the tile's rows
    if (a.rows_ctr && rt == 0 && tid == 0) atomicAdd(a.rows_ctr + pt.e, min(BN, pt.cnt - pt.tok0));
  }
  span_end(a.span);
}

// Correction seeds of the gate/up kernel: xsum[g][t] = -136 * (sum over group g of the
// activations of token t), fp32, one thread per (token, group), in the order of
// chunk8_sum and row16_tree_sum (the routing kernels that also make these sums follow it).
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                   float* __restrict__ xsum) {
  const int G = H / kGroup;
  const int i = blockIdx.x * 256 + threadIdx.x;     // one (group, token) per thread
  if (i >= G * T) return;
  const int g = i / T, t = i % T;
  const uint4* p = reinterpret_cast<const uint4*>(x + (size_t)t * H + g * kGroup);
  float c[16];
#pragma unroll
  for (int j = 0; j < 16; j++) c[j] = chunk8_sum(p[j]);
#pragma unroll
  for (int w = 1; w < 16; w <<= 1)
#pragma unroll
    for (int j = 0; j < 16; j += 2 * w) c[j] += c[j + w];
  xsum[i] = -136.0f * c[0];
}

hipError_t launch_moe_prefill_xsum(const MoeArgs& a, hipStream_t s) {
  const int G = a.H / kGroup;
  ProfScope prof("xsum", s);
  EXMOE_LAUNCH(prof, xsum_kernel, dim3((G * a.T + 255) / 256), dim3(256), 0, s, a.x, a.T, a.H, a.xsum);
  return hipGetLastError();
}

// NW waves per workgroup and BN tokens per token tile; the row tile is 256 rows either way.
template <bool Q4, int NW, int BN>
static hipError_t launch_prefill_tiles(const MoeArgs& a, hipStream_t s) {
  const int TK = a.T * a.k;
  const int max_tt = TK / BN + (a.E < TK ? a.E : TK);
  const int rt_gu = a.I / 128;
  {
    ProfScope prof(Q4 ? "prefill_gateup" : "bf16_prefill_gateup", s);
    MoeArgs as = a;
    as.span = prof.span();
    EXMOE_LAUNCH(prof, (prefill_kernel<true, NW, BN, Q4>), dim3(max_tt * rt_gu), dim3(NW * 64), 0, s, as, -1,
                 rt_gu);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rt_d = (a.H + kPfRows - 1) / kPfRows;
  {
    ProfScope prof(Q4 ? "prefill_down" : "bf16_prefill_down", s);
    MoeArgs as = a;
    as.span = prof.span();
    EXMOE_LAUNCH(prof, (prefill_kernel<false, NW, BN, Q4>), dim3(max_tt * rt_d), dim3(NW * 64), 0, s, as, -1,
                 rt_d);
  }
  return hipGetLastError();
}

// int4 experts: 64-token tiles on 4-wave workgroups, two per compute unit, so that the
// waves sharing a SIMD belong to different workgroups and their barriers, memory round
// trips, unpacking and MFMAs overlap (against 128-token tiles on 8-wave workgroups:
// Zipf 512 tokens 0.164 -> 0.143 ms per layer, 2048 tokens 0.372 -> 0.342 ms, large layer
// 2.86 -> 2.85 ms). The bf16 comparator keeps the 128-token tiles: its 4-wave form runs
// out of registers (four 16-byte weight loads per row subtile and group).
template <bool Q4>
static hipError_t launch_prefill_experts(const MoeArgs& a, hipStream_t s) {
  if constexpr (Q4)
    return launch_prefill_tiles<Q4, 4, 64>(a, s);
  else
    return launch_prefill_tiles<Q4, kPfWaves, kPfBN>(a, s);
}

hipError_t launch_moe_prefill_experts(const MoeArgs& a, hipStream_t s) { return launch_prefill_experts<true>(a, s); }
hipError_t launch_bf16_prefill_experts(const MoeArgs& a, hipStream_t s) { return launch_prefill_experts<false>(a, s); }


}  // namespace exmoe
