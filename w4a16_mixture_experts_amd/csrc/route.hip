// BF16 router logits, top-k selection and routing weights (gfx950).
//
// ExactMoE keeps the router in BF16 and its top-k procedure unchanged (abstract; Fig. 1
// caption). Logits: exact bf16 x bf16 products (exact in fp32) accumulated in fp64 and
// rounded once to bf16, so that the selection made on them does not depend on the
// summation order. Selection: (logit descending, expert id ascending) on the bf16 logits.
#include "common.h"
#include "device.h"
#include "group_block.h"
#include "topk.h"
#include "route_wave.h"

namespace exmoe {

// ONE: H <= 8 LANES MC, one pass of loads per wave. XS: also the grouped GEMM's
// correction seeds (route_logits_wave).
template <int TB, int EB, int LANES, int MC, bool ONE, bool XS>
__global__ __launch_bounds__(64) void route_logits_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T,
                                                          int H, int E,
                                                          uint16_t* __restrict__ logits, float* __restrict__ xsum) {
  route_logits_wave<TB, EB, LANES, MC, false, ONE, XS>(x, wr, bias, T, H, E, logits,
                                                      blockIdx.x * (64 / LANES) + (int)lane_id() / LANES, xsum);
}

// ---------------------------------------------------------------------------------
// Logits of a few tokens, one logit per workgroup, with H split over its KW waves: one
// 16-byte chunk of the token row and of the router row per lane (H <= 512 KW), both
// loaded before any arithmetic; the chunk's 8 products are added in fp64 in element
// order, then the lanes of each 16-lane row (DPP rotations), the 4 rows of the wave (fixed
// order) and the KW waves (wave order, through LDS); one thread rounds once to bf16.
// ---------------------------------------------------------------------------------
template <int KW>
__global__ __launch_bounds__(64 * KW) void route_logits_split_kernel(const uint16_t* __restrict__ x,
                                                                     const uint16_t* __restrict__ wr,
                                                                     const float* __restrict__ bias, int T, int H,
                                                                     int E, uint16_t* __restrict__ logits) {
  __shared__ double red[KW];
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int t = (int)blockIdx.x / E, e = (int)blockIdx.x % E;
  const int chunks = H / 8;
  const int c = wave * 64 + lane;
  const bool on = c < chunks;
  const int cc = on ? c : chunks - 1;   // clamped: no load under a per-lane branch
  uint4 xu = reinterpret_cast<const uint4*>(x + (size_t)t * H)[cc];
  uint4 wu = reinterpret_cast<const uint4*>(wr + (size_t)e * H)[cc];
  // chunks past H become zeros (0 * 0 added to +0.0 leaves the sum's bits unchanged)
  xu = on ? xu : make_uint4(0u, 0u, 0u, 0u);
  wu = on ? wu : make_uint4(0u, 0u, 0u, 0u);
  const uint32_t xq[4] = {xu.x, xu.y, xu.z, xu.w}, wq[4] = {wu.x, wu.y, wu.z, wu.w};
  double a = 0.0;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    a = fma((double)__uint_as_float(xq[q] << 16), (double)__uint_as_float(wq[q] << 16), a);
    a = fma((double)__uint_as_float(xq[q] & 0xFFFF0000u), (double)__uint_as_float(wq[q] & 0xFFFF0000u), a);
  }
  double sv = row16_sum_f64(a);
  const long long b = __double_as_longlong(sv);
  const int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
  double r[4];
#pragma unroll
  for (int q = 0; q < 4; q++)
    r[q] = __longlong_as_double(((long long)(unsigned)__builtin_amdgcn_readlane(lo, 16 * q)) |
                                ((long long)__builtin_amdgcn_readlane(hi, 16 * q) << 32));
  sv = ((r[0] + r[1]) + r[2]) + r[3];
  if (lane == 0) red[wave] = sv;
  __syncthreads();
  if (threadIdx.x == 0) {
    double v = red[0];
#pragma unroll
    for (int w = 1; w < KW; w++) v += red[w];
    logits[(size_t)t * E + e] = f64_to_bf16(bias ? v + (double)bias[e] : v);
  }
}

// ---------------------------------------------------------------------------------
// Logits of many tokens on the fp64 matrix cores: a workgroup owns a tile of 16 tokens x
// 16 experts, each of its KW waves a strided share of the 32-column chunks of H, and the
// KW partial tiles are added in wave order through LDS. v_mfma_f64_16x16x4f64 takes A[m][k]
// from lane 16 k + m and B[k][n] from lane 16 k + n, and leaves C[g + 4 i][n] in value i of
// lane 16 g + n. Lane group g loads 8 bf16 of its row at columns 8 g .. 8 g + 7 of the
// chunk; MFMA j of the chunk multiplies element j of every lane, so that the 4 K slots of
// MFMA j are columns {8 g + j}. The products of bf16 values are exact in fp64 and the sum
// is rounded to bf16 once, as in the vector form.
// ---------------------------------------------------------------------------------
// XS (H <= kLgtXsMaxH): the workgroups also write the grouped GEMM's correction seeds of
// their 16 tokens, xsum[g][t] = -136 * (sum of group g of token t), from the activation
// chunks they load (group g by the workgroup of expert block g mod the block count), in
// the order of chunk8_sum and row16_tree_sum: each lane's 16-byte chunk sums go to LDS,
// and after the loop one thread per (group, token) adds the group's 16 in that tree.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kLgtXsMaxG = kLgtXsMaxH / kGroup;

template <int KW, bool XS>
__global__ __launch_bounds__(64 * KW) void route_logits_mfma_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wr,
                                                                    const float* __restrict__ bias, int T, int H,
                                                                    int E, uint16_t* __restrict__ logits,
                                                                    float* __restrict__ xsum) {
  __shared__ f64x4 red[KW][64];
  __shared__ float s_x16[XS ? kLgtXsMaxG : 1][16][16];   // [group][16-byte chunk of it][token]
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nEB = (E + 15) / 16;
  const int t0 = (blockIdx.x / nEB) * 16, e0 = (blockIdx.x % nEB) * 16;
  const int m = lane & 15, g = lane >> 4;
  const int t = t0 + m < T ? t0 + m : T - 1, e = e0 + m < E ? e0 + m : E - 1;   // clamped rows
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H) + g;
  const uint4* wrr = reinterpret_cast<const uint4*>(wr + (size_t)e * H) + g;
  const int nch = H / 32;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  const int xeb = (int)blockIdx.x % nEB;
  auto chunk = [&](const uint4 xu, const uint4 wu, int cc) {
    if (XS && (cc >> 2) % nEB == xeb) s_x16[cc >> 2][4 * (cc & 3) + g][m] = chunk8_sum(xu);   // wave-uniform test
    const uint32_t xq[4] = {xu.x, xu.y, xu.z, xu.w}, wq[4] = {wu.x, wu.y, wu.z, wu.w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(xq[q] << 16),
                                                 (double)__uint_as_float(wq[q] << 16), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)__uint_as_float(xq[q] & 0xFFFF0000u),
                                                 (double)__uint_as_float(wq[q] & 0xFFFF0000u), acc, 0, 0, 0);
    }
  };
  // two chunks in flight: the loads of chunk c + 2 KW go out before chunk c's MFMAs
  int c = wave;
  uint4 xa, wa, xb, wb;
  if (c < nch) { xa = xr[4 * c]; wa = wrr[4 * c]; }
  if (c + KW < nch) { xb = xr[4 * (c + KW)]; wb = wrr[4 * (c + KW)]; }
  for (; c < nch; c += 2 * KW) {
    const uint4 xc = xa, wc = wa;
    if (c + 2 * KW < nch) { xa = xr[4 * (c + 2 * KW)]; wa = wrr[4 * (c + 2 * KW)]; }
    chunk(xc, wc, c);
    if (c + KW < nch) {
      const uint4 xd = xb, wd = wb;
      if (c + 3 * KW < nch) { xb = xr[4 * (c + 3 * KW)]; wb = wrr[4 * (c + 3 * KW)]; }
      chunk(xd, wd, c + KW);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (XS) {
    for (int i = (int)threadIdx.x; i < (H / kGroup) * 16; i += 64 * KW) {
      const int gg = i / 16, mm = i % 16;
      if (gg % nEB == xeb && t0 + mm < T) {
        float c[16];
#pragma unroll
        for (int j = 0; j < 16; j++) c[j] = s_x16[gg][j][mm];
#pragma unroll
        for (int w = 1; w < 16; w <<= 1)
#pragma unroll
          for (int j = 0; j < 16; j += 2 * w) c[j] += c[j + w];
        xsum[(size_t)gg * T + t0 + mm] = -136.0f * c[0];
      }
    }
  }
  if (wave == 0) {
    f64x4 s = red[0][lane];
#pragma unroll
    for (int w = 1; w < KW; w++) s += red[w][lane];
    const int ee = e0 + m;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int tt = t0 + g + 4 * i;
      if (tt < T && ee < E) {
        const double v = bias ? s[i] + (double)bias[ee] : s[i];
        logits[(size_t)tt * E + ee] = f64_to_bf16(v);
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// The same split for 2 tokens x 2 experts per workgroup (prefill sizes up to 128 tokens).
// XS: the workgroups also write the grouped GEMM's correction seeds of their two tokens:
// row r of wave w holds the 16 chunks of group 4 w + r, which the workgroups of expert
// block g mod the block count sum (chunk8_sum, then row16_tree_sum over the row).
// ---------------------------------------------------------------------------------
template <int KW, bool XS>
__global__ __launch_bounds__(64 * KW) void route_logits_split2_kernel(const uint16_t* __restrict__ x,
                                                                      const uint16_t* __restrict__ wr,
                                                                      const float* __restrict__ bias, int T, int H,
                                                                      int E, uint16_t* __restrict__ logits,
                                                                      float* __restrict__ xsum) {
  __shared__ double red[KW][4];
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int nEB = (E + 1) / 2;
  const int eb = (int)blockIdx.x % nEB;
  const int t0 = ((int)blockIdx.x / nEB) * 2, e0 = eb * 2;
  const int chunks = H / 8;
  const int c = wave * 64 + lane;
  const bool on = c < chunks;
  const int cc = on ? c : chunks - 1;   // clamped: no load under a per-lane branch
  uint4 xu[2], wu[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int t = t0 + i < T ? t0 + i : T - 1;
    xu[i] = reinterpret_cast<const uint4*>(x + (size_t)t * H)[cc];
    const int e = e0 + i < E ? e0 + i : E - 1;
    wu[i] = reinterpret_cast<const uint4*>(wr + (size_t)e * H)[cc];
  }
  // chunks past H become zeros (0 * 0 added to +0.0 leaves the sum's bits unchanged)
#pragma unroll
  for (int i = 0; i < 2; i++) {
    xu[i] = on ? xu[i] : make_uint4(0u, 0u, 0u, 0u);
    wu[i] = on ? wu[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  if (XS) {
    const int g = c / 16;
    const bool mine = g % nEB == eb && (lane & 15) == 0 && on;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const float v = row16_tree_sum(chunk8_sum(xu[i]));
      if (mine && t0 + i < T) xsum[(size_t)g * T + t0 + i] = -136.0f * v;
    }
  }
  double xv[2][8], wv[2][8];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const uint32_t xq[4] = {xu[i].x, xu[i].y, xu[i].z, xu[i].w}, wq[4] = {wu[i].x, wu[i].y, wu[i].z, wu[i].w};
#pragma unroll
    for (int q = 0; q < 4; q++) {
      xv[i][2 * q] = (double)__uint_as_float(xq[q] << 16);
      xv[i][2 * q + 1] = (double)__uint_as_float(xq[q] & 0xFFFF0000u);
      wv[i][2 * q] = (double)__uint_as_float(wq[q] << 16);
      wv[i][2 * q + 1] = (double)__uint_as_float(wq[q] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      double a = 0.0;
#pragma unroll
      for (int q = 0; q < 8; q++) a = fma(xv[i][q], wv[j][q], a);
      double sv = row16_sum_f64(a);
      const long long b = __double_as_longlong(sv);
      const int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
      double r[4];
#pragma unroll
      for (int q = 0; q < 4; q++)
        r[q] = __longlong_as_double(((long long)(unsigned)__builtin_amdgcn_readlane(lo, 16 * q)) |
                                    ((long long)__builtin_amdgcn_readlane(hi, 16 * q) << 32));
      sv = ((r[0] + r[1]) + r[2]) + r[3];
      if (lane == 0) red[wave][2 * i + j] = sv;
    }
  __syncthreads();
  const int q = (int)threadIdx.x;
  if (q < 4) {
    const int t = t0 + q / 2, e = e0 + q % 2;
    double v = red[0][q];
#pragma unroll
    for (int w = 1; w < KW; w++) v += red[w][q];
    if (t < T && e < E) logits[(size_t)t * E + e] = f64_to_bf16(bias ? v + (double)bias[e] : v);
  }
}

// ---------------------------------------------------------------------------------
// Logits, top-k and the expert table of a few tokens (T <= 16) in one launch: the
// selection part (route_wave.h) with one wave per token of a 4-token block and one block
// of 2 experts per workgroup.
// ---------------------------------------------------------------------------------
__global__ __launch_bounds__(64 * kRouteSelTB) void route_sel_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias, int T, int H,
    int E, int k, int renormalize, uint16_t* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ w,
    uint8_t* __restrict__ sel, uint32_t* __restrict__ counters) {
  __shared__ RouteSelShared sh;
  route_sel_part<kRouteSelTB>(x, wr, bias, T, H, E, k, renormalize, logits, ids, w, sel, counters, blockIdx.x, sh);
}

__global__ __launch_bounds__(256) void topk_kernel(const uint16_t* __restrict__ logits,
                                                   const int32_t* __restrict__ given_ids, int T,
                                                   int E, int k, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ w) {
  const int lane = (int)lane_id();
  const int t = blockIdx.x * 4 + threadIdx.x / 64;
  if (t >= T) return;
  int id;
  float wt;
  topk_token(logits + (size_t)t * E, given_ids ? given_ids + (size_t)t * k : nullptr, E, k, renormalize, id, wt);
  if (lane < k) {
    if (ids) ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

// Top-k of every token and the grouping in one workgroup (small token counts): the ids
// stay in LDS between the two phases, saving a launch.
constexpr int kTopkGroupThreads = 256;
__global__ __launch_bounds__(kTopkGroupThreads) void topk_group_kernel(const uint16_t* __restrict__ logits,
                                                                  int T, int E, int k, int renormalize,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ w,
                                                                  int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted_flat,
                                                                  int32_t* __restrict__ flat_to_sorted) {
  __shared__ int32_t s_ids[kTopkGroupMaxRows];
  __shared__ GroupSharedT<kTopkGroupThreads> gs;
  const int lane = (int)lane_id(), wave = threadIdx.x >> 6;
  for (int t = wave; t < T; t += kTopkGroupThreads / 64) {
    int id;
    float wt;
    topk_token(logits + (size_t)t * E, nullptr, E, k, renormalize, id, wt);
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      w[(size_t)t * k + lane] = wt;
      s_ids[t * k + lane] = id;
    }
  }
  __syncthreads();
  group_block<kTopkGroupThreads>(s_ids, T * k, E, offsets, sorted_flat, flat_to_sorted, gs);
}


// ---------------------------------------------------------------------------------
// Whole routing of one token by one workgroup (decode sizes): its E logits with the
// same per-lane arithmetic as route_logits_kernel<.., .., 64, ..> (lanes split H in
// interleaved 16-byte chunks, ascending; fp64 partials added by DPP row sums and a
// fixed-order readlane combine), then the top-k selection and the weights from the bf16
// logits kept in LDS. Each wave takes 4 experts at a time and issues all loads of a
// 2048-column piece (the token's chunks and the 4 router rows) before the first FMA, so
// a piece costs one memory latency.
// ---------------------------------------------------------------------------------
constexpr int kRouteTokThreads = 1024;
constexpr int kRouteTokEB = 4;     // experts per wave at a time
constexpr int kRouteTokMC = 4;     // 16-byte chunks per lane per 2048-column piece
__global__ __launch_bounds__(kRouteTokThreads) void route_token_kernel(const uint16_t* __restrict__ x,
                                                                       const uint16_t* __restrict__ wr,
                                                                       const float* __restrict__ bias, int H, int E,
                                                                       int k, int renormalize,
                                                                       uint16_t* __restrict__ logits,
                                                                       int32_t* __restrict__ ids,
                                                                       float* __restrict__ w) {
  __shared__ uint16_t s_log[kMaxExperts];
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int t = blockIdx.x;
  const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * H);
  const int chunks = H / 8;
  constexpr int EB = kRouteTokEB, MC = kRouteTokMC;
  for (int e0 = wave * EB; e0 < E; e0 += EB * (kRouteTokThreads / 64)) {
    double acc[EB];
#pragma unroll
    for (int j = 0; j < EB; j++) acc[j] = 0.0;
    for (int c0 = 0; c0 < chunks; c0 += 64 * MC) {
      uint4 xu[MC], wu[EB][MC];
#pragma unroll
      for (int m = 0; m < MC; m++) {
        int c = c0 + lane + 64 * m;
        c = c < chunks ? c : chunks - 1;
        xu[m] = xr[c];
#pragma unroll
        for (int j = 0; j < EB; j++) {
          const int e = e0 + j < E ? e0 + j : E - 1;
          wu[j][m] = reinterpret_cast<const uint4*>(wr + (size_t)e * H)[c];
        }
      }
#pragma unroll
      for (int m = 0; m < MC; m++) {
        if (c0 + lane + 64 * m < chunks) {
          const uint32_t xq[4] = {xu[m].x, xu[m].y, xu[m].z, xu[m].w};
          double xv[8];
#pragma unroll
          for (int q = 0; q < 4; q++) {
            xv[2 * q] = (double)__uint_as_float(xq[q] << 16);
            xv[2 * q + 1] = (double)__uint_as_float(xq[q] & 0xFFFF0000u);
          }
#pragma unroll
          for (int j = 0; j < EB; j++) {
            const uint32_t q4[4] = {wu[j][m].x, wu[j][m].y, wu[j][m].z, wu[j][m].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
              acc[j] = fma(xv[2 * q], (double)__uint_as_float(q4[q] << 16), acc[j]);
              acc[j] = fma(xv[2 * q + 1], (double)__uint_as_float(q4[q] & 0xFFFF0000u), acc[j]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < EB; j++) {
      const double s16 = row16_sum_f64(acc[j]);
      const long long b = __double_as_longlong(s16);
      const int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
      double r[4];
#pragma unroll
      for (int q = 0; q < 4; q++)
        r[q] = __longlong_as_double(((long long)(unsigned)__builtin_amdgcn_readlane(lo, 16 * q)) |
                                    ((long long)__builtin_amdgcn_readlane(hi, 16 * q) << 32));
      const double sum = ((r[0] + r[1]) + r[2]) + r[3];
      const int e = e0 + j;
      if (lane == 0 && e < E) s_log[e] = f64_to_bf16(bias ? sum + (double)bias[e] : sum);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += kRouteTokThreads) logits[(size_t)t * E + i] = s_log[i];
  if (wave == 0) {
    int id;
    float wt;
    topk_token(s_log, nullptr, E, k, renormalize, id, wt);
    if (lane < k) {
      ids[(size_t)t * k + lane] = id;
      w[(size_t)t * k + lane] = wt;
    }
  }
}

hipError_t launch_route_token(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                              int k, int renormalize, uint16_t* logits, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  ProfScope prof("route_token", s);
  EXMOE_LAUNCH(prof, route_token_kernel, dim3(T), dim3(kRouteTokThreads), 0, s, x, wr, bias, H, E, k, renormalize,
               logits, ids, w);
  return hipGetLastError();
}

hipError_t launch_route_sel(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E, int k,
                            int renormalize, uint16_t* logits, int32_t* ids, float* w, uint8_t* sel,
                            uint32_t* counters, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (T > kRouteSelMaxTok || H > kRouteSelMaxH || k > 64) return hipErrorInvalidValue;
  ProfScope prof("route_sel", s);
  const int blocks = ((T + kRouteSelTB - 1) / kRouteSelTB) * ((E + kRouteSelEB - 1) / kRouteSelEB);
  EXMOE_LAUNCH(prof, route_sel_kernel, dim3(blocks), dim3(64 * kRouteSelTB), 0, s, x, wr, bias, T, H, E, k, renormalize, logits, ids,
               w, sel, counters);
  return hipGetLastError();
}

hipError_t launch_route_logits(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H,
                               int E, uint16_t* logits, hipStream_t s, float* xsum) {
  if (T == 0) return hipSuccess;
  if (xsum && H > kLgtXsMaxH) return hipErrorInvalidValue;   // the seed sums' LDS rows
  ProfScope prof("route_logits", s);
  if (T <= 16 && !xsum && H <= 4096) {
    // one logit per workgroup, H split over its waves (16 tokens and 64 experts: layer
    // 44.2 -> 43.5 us; one token 23.7 -> 22.7 us; against a wave per 2 tokens x 2 experts)
    const int kw = (H + 511) / 512;
    if (kw <= 2)
      EXMOE_LAUNCH(prof, route_logits_split_kernel<2>, dim3(T * E), dim3(128), 0, s, x, wr, bias, T, H, E, logits);
    else if (kw <= 4)
      EXMOE_LAUNCH(prof, route_logits_split_kernel<4>, dim3(T * E), dim3(256), 0, s, x, wr, bias, T, H, E, logits);
    else
      EXMOE_LAUNCH(prof, route_logits_split_kernel<8>, dim3(T * E), dim3(512), 0, s, x, wr, bias, T, H, E, logits);
  } else if (T <= 128 && H <= 4096) {
    // 2 tokens x 2 experts per workgroup, H split over its waves
    const int kw = (H + 511) / 512;
    const int blocks = ((T + 1) / 2) * ((E + 1) / 2);
#define EXMOE_SPLIT2(KW_)                                                                                        \
  do {                                                                                                           \
    if (xsum)                                                                                                    \
      EXMOE_LAUNCH(prof, (route_logits_split2_kernel<KW_, true>), dim3(blocks), dim3(64 * KW_), 0, s, x, wr, bias, \
                   T, H, E, logits, xsum);                                                                       \
    else                                                                                                         \
      EXMOE_LAUNCH(prof, (route_logits_split2_kernel<KW_, false>), dim3(blocks), dim3(64 * KW_), 0, s, x, wr,      \
                   bias, T, H, E, logits, nullptr);                                                              \
  } while (0)
    if (kw <= 2) EXMOE_SPLIT2(2);
    else if (kw <= 4) EXMOE_SPLIT2(4);
    else EXMOE_SPLIT2(8);
#undef EXMOE_SPLIT2
  } else if (T <= 128) {
    // one wave per 2 tokens x 2 experts, the whole wave on H: a row in one round trip
    const int blocks = ((T + 1) / 2) * ((E + 1) / 2);
    const bool one = H <= kRouteSelMaxH;
    if (one && xsum)
      EXMOE_LAUNCH(prof, (route_logits_kernel<2, 2, 64, 4, true, true>), dim3(blocks), dim3(64), 0, s, x, wr, bias, T,
                   H, E, logits, xsum);
    else if (one)
      EXMOE_LAUNCH(prof, (route_logits_kernel<2, 2, 64, 4, true, false>), dim3(blocks), dim3(64), 0, s, x, wr, bias,
                   T, H, E, logits, nullptr);
    else if (xsum)
      EXMOE_LAUNCH(prof, (route_logits_kernel<2, 2, 64, 4, false, true>), dim3(blocks), dim3(64), 0, s, x, wr, bias,
                   T, H, E, logits, xsum);
    else
      EXMOE_LAUNCH(prof, (route_logits_kernel<2, 2, 64, 4, false, false>), dim3(blocks), dim3(64), 0, s, x, wr, bias,
                   T, H, E, logits, nullptr);
  } else {
    // 16 x 16 tiles on the fp64 matrix cores (H is a multiple of 128), H split over 8
    // waves. Measured against four 4 x 4 blocks of vector FMAs per wave: 2048 tokens and
    // 64 experts 30.9 -> 15.5 us, 512 tokens 12.4 -> 8.8 us.
    const int tiles = ((T + 15) / 16) * ((E + 15) / 16);
    if (xsum)
      EXMOE_LAUNCH(prof, (route_logits_mfma_kernel<8, true>), dim3(tiles), dim3(512), 0, s, x, wr, bias, T, H, E,
                   logits, xsum);
    else
      EXMOE_LAUNCH(prof, (route_logits_mfma_kernel<8, false>), dim3(tiles), dim3(512), 0, s, x, wr, bias, T, H, E,
                   logits, nullptr);
  }
  return hipGetLastError();
}

// One workgroup for both steps saves a launch for a few tokens; its four waves take the
// tokens one after another, so from kTopkGroupMaxTok tokens on the top-k runs one token
// per wave over the whole chip and the grouping in a launch of its own.
constexpr int kTopkGroupMaxTok = 16;
hipError_t launch_topk_group(const uint16_t* logits, int T, int E, int k, int renormalize, int32_t* ids,
                             float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                             int32_t* group_ws, hipStream_t s) {
  if (T * k > kTopkGroupMaxRows || T > kTopkGroupMaxTok) {
    hipError_t e = launch_topk(logits, nullptr, T, E, k, renormalize, ids, w, s);
    if (e != hipSuccess) return e;
    return launch_group(ids, T, k, E, offsets, sorted_flat, flat_to_sorted, group_ws, s);
  }
  ProfScope prof("topk_group", s);
  EXMOE_LAUNCH(prof, topk_group_kernel, dim3(1), dim3(kTopkGroupThreads), 0, s, logits, T, E, k, renormalize, ids, w,
                     offsets, sorted_flat, flat_to_sorted);
  return hipGetLastError();
}

hipError_t launch_topk(const uint16_t* logits, const int32_t* given_ids, int T, int E, int k,
                       int renormalize, int32_t* ids, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  ProfScope prof("topk", s);
  EXMOE_LAUNCH(prof, topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits, given_ids, T, E, k,
                     renormalize, ids, w);
  return hipGetLastError();
}

}  // namespace exmoe
