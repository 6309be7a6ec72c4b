// Device helpers for the gfx950 kernels: MFMA operand types, int4 dequantization into
// bf16 MFMA operands, bf16 conversions and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "common.h"

namespace exmoe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// v_mfma_f32_16x16x32_bf16: A 16x32 (lane l: row l%16, k = 8(l/16)+0..7), B 32x16 (lane l:
// column l%16, same k), C 16x16 (lane l: column l%16, rows 4(l/16)+0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Compile-time constants hidden from constant folding, so that (a & m) | o below is
// selected as one v_and_or_b32 (m in an SGPR, o in a VGPR: one constant-bus read)
// instead of v_and + v_or with literals. The asm only moves constants; its VGPR result
// feeds VALU ops alone (no VALU-to-MFMA hazard hides behind it, since the compiler's
// hazard checks do not see through asm).
__device__ __forceinline__ uint32_t opaque_sgpr(uint32_t v) {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(v));
  return r;
}
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t v) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(v));
  return r;
}

// One packed word (8 nibbles u = q + 8, input j at bit 4(j/2) for even j, 16 + 4(j/2) for
// odd j) -> 8 bf16 operand values 128 + u, exact, in 7 VALU ops. Register p holds inputs
// 2p (low half) and 2p+1 (high half). The "+128 + 8" offset is removed by the -136
// correction of the group's MFMA chain.
__device__ __forceinline__ bf16x8 dequant_word(uint32_t w) {
  const uint32_t m = opaque_sgpr(0x000F000Fu), magic = opaque_vgpr(0x43004300u);  // bf16 128.0 x2
  i32x4 r;
  r[0] = (int)((w & m) | magic);
  r[1] = (int)(((w >> 4) & m) | magic);
  r[2] = (int)(((w >> 8) & m) | magic);
  r[3] = (int)(((w >> 12) & m) | magic);
  return __builtin_bit_cast(bf16x8, r);
}

// Operand of -136.0 in every element: an MFMA chain of it against the activation
// fragments yields -136 * (sum of the activations of the group), which turns the
// 128 + u operand values into the signed codes q = u - 8.
__device__ __forceinline__ bf16x8 neg136_operand() {
  i32x4 r;
  r[0] = r[1] = r[2] = r[3] = (int)0xC308C308u;          // bf16 -136.0
  return __builtin_bit_cast(bf16x8, r);
}

// acc[i] += scale(row i) * c[i]; sc holds the 4 bf16 scales of the lane's rows 4(l/16)+0..3.
__device__ __forceinline__ void scale_accum(f32x4& acc, const f32x4& c, uint2 sc) {
  acc[0] += __uint_as_float(sc.x << 16) * c[0];
  acc[1] += __uint_as_float(sc.x & 0xFFFF0000u) * c[1];
  acc[2] += __uint_as_float(sc.y << 16) * c[2];
  acc[3] += __uint_as_float(sc.y & 0xFFFF0000u) * c[3];
}

// Launch span stamps (benchmark timing, off when sp is null): the first thread of every
// workgroup folds the GPU's constant-rate clock into its sub-slot of the launch's slot
// (kSpanSub sub-slots, by workgroup index, so that few workgroups share an address):
// minimum at its start, maximum after all of its waves' memory operations have completed.
// The launch's duration is the largest end minus the smallest start, inside a replayed
// graph too.
__device__ __forceinline__ void span_begin(unsigned long long* sp) {
  if (sp && threadIdx.x == 0)
    atomicMin(sp + 2 * (blockIdx.x % kSpanSub), (unsigned long long)__builtin_amdgcn_s_memrealtime());
}
__device__ __forceinline__ void span_end(unsigned long long* sp) {
  if (sp) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
      atomicMax(sp + 2 * (blockIdx.x % kSpanSub) + 1, (unsigned long long)__builtin_amdgcn_s_memrealtime());
  }
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two fp32 values -> packed bf16 pair (lo in bits 0..15), round to nearest even, one
// instruction.
typedef float exmoe_f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 exmoe_bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const exmoe_f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, exmoe_bf16x2));
}

// silu(g) * u = g / (1 + e^-g) * u in fp32, from the hardware 2^x and reciprocal (each
// within about one ulp); g -> -inf gives -0, g -> +inf gives g * u.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * g);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// fp64 -> bf16 with a single rounding (nearest even), no detour through fp32.
__device__ __forceinline__ uint16_t f64_to_bf16(double v) {
  if (v == 0.0) return __double_as_longlong(v) < 0 ? 0x8000 : 0;
  int e;
  (void)frexp(v, &e);                      // v = m 2^e, 0.5 <= |m| < 1
  int qe = e - 1 - 7;
  if (qe < -133) qe = -133;
  double r = ldexp(rint(ldexp(v, -qe)), qe);
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// Cross-lane reductions on DPP row rotations (within 16-lane rows) plus four readlanes
// across the rows; the result is wave-uniform. Much shorter latency than LDS permutes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
// Group sums of the activations (the grouped GEMM's correction seeds) in one order for
// every kernel that makes them, so that they agree bit for bit: the 8 bf16 of a 16-byte
// chunk in element order, then the 16 chunk sums of a 128-input group in a balanced
// pairwise tree in chunk order, ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)) + ...
__device__ __forceinline__ float chunk8_sum(uint4 v) {
  const uint32_t q[4] = {v.x, v.y, v.z, v.w};
  float s = __uint_as_float(q[0] << 16);
  s += __uint_as_float(q[0] & 0xFFFF0000u);
#pragma unroll
  for (int i = 1; i < 4; i++) {
    s += __uint_as_float(q[i] << 16);
    s += __uint_as_float(q[i] & 0xFFFF0000u);
  }
  return s;
}
// The tree over the chunk sums held by the 16 lanes of a row (lane l of the row: chunk l),
// in every lane of the row: partners at lane distance 1 and 2 (quad permutes), then the
// other quad of the half row and the other half row (mirrors); each step adds two equal
// subtrees, so every lane ends with the same bits.
__device__ __forceinline__ float row16_tree_sum(float v) {
  v += __uint_as_float(dpp_u32<0xB1>(__float_as_uint(v)));    // quad_perm [1, 0, 3, 2]
  v += __uint_as_float(dpp_u32<0x4E>(__float_as_uint(v)));    // quad_perm [2, 3, 0, 1]
  v += __uint_as_float(dpp_u32<0x141>(__float_as_uint(v)));   // row_half_mirror
  v += __uint_as_float(dpp_u32<0x140>(__float_as_uint(v)));   // row_mirror
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t o;
  o = dpp_u32<0x121>(v); v = o > v ? o : v;   // row_ror:1
  o = dpp_u32<0x122>(v); v = o > v ? o : v;   // row_ror:2
  o = dpp_u32<0x124>(v); v = o > v ? o : v;   // row_ror:4
  o = dpp_u32<0x128>(v); v = o > v ? o : v;   // row_ror:8
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), e = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  a = a > b ? a : b;
  c = c > e ? c : e;
  return a > c ? a : c;
}
__device__ __forceinline__ float wave_max_f32(float v) {
  float o;
  o = __uint_as_float(dpp_u32<0x121>(__float_as_uint(v))); v = fmaxf(v, o);
  o = __uint_as_float(dpp_u32<0x122>(__float_as_uint(v))); v = fmaxf(v, o);
  o = __uint_as_float(dpp_u32<0x124>(__float_as_uint(v))); v = fmaxf(v, o);
  o = __uint_as_float(dpp_u32<0x128>(__float_as_uint(v))); v = fmaxf(v, o);
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, e));
}
// Sum in a fixed order (deterministic): row rotations, then rows 0+1+2+3.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __uint_as_float(dpp_u32<0x121>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x122>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x124>(__float_as_uint(v)));
  v += __uint_as_float(dpp_u32<0x128>(__float_as_uint(v)));
  float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return ((a + b) + c) + e;
}
__device__ __forceinline__ double dpp_f64_ror(double v, int which) {
  const long long b = __double_as_longlong(v);
  int lo = (int)(b & 0xFFFFFFFFll), hi = (int)(b >> 32);
  switch (which) {
    case 1: lo = __builtin_amdgcn_update_dpp(0, lo, 0x121, 0xF, 0xF, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x121, 0xF, 0xF, false); break;
    case 2: lo = __builtin_amdgcn_update_dpp(0, lo, 0x122, 0xF, 0xF, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x122, 0xF, 0xF, false); break;
    case 4: lo = __builtin_amdgcn_update_dpp(0, lo, 0x124, 0xF, 0xF, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x124, 0xF, 0xF, false); break;
    default: lo = __builtin_amdgcn_update_dpp(0, lo, 0x128, 0xF, 0xF, false); hi = __builtin_amdgcn_update_dpp(0, hi, 0x128, 0xF, 0xF, false); break;
  }
  return __longlong_as_double(((long long)(unsigned)lo) | ((long long)hi << 32));
}
// fp64 sum over each 16-lane row (every lane of the row gets the row's sum).
__device__ __forceinline__ double row16_sum_f64(double v) {
  v += dpp_f64_ror(v, 1);
  v += dpp_f64_ror(v, 2);
  v += dpp_f64_ror(v, 4);
  v += dpp_f64_ror(v, 8);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    T o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The a-th (0-based) expert with a non-empty segment, or -1; also returns the count of
// non-empty segments. Called by a whole wave; E <= 256.
__device__ __forceinline__ int nth_active_expert(const int32_t* __restrict__ offsets, int E, int a,
                                                 int* n_active) {
  int lane = (int)lane_id();
  int found = -1, base = 0;
  for (int c0 = 0; c0 < E; c0 += 64) {
    int e = c0 + lane;
    bool act = e < E && offsets[e + 1] > offsets[e];
    uint64_t m = __ballot(act);
    int rank = base + __popcll(m & ((1ull << lane) - 1ull));
    uint64_t hit = __ballot(act && rank == a);
    if (hit) found = c0 + (int)__ffsll((long long)hit) - 1;
    base += __popcll(m);
  }
  *n_active = base;
  return found;
}

}  // namespace exmoe
