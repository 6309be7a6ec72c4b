// Dense bf16 expert layer for decode sizes (the comparator of the int4 layer), gfx950.
//
// ExactMoE's measurements set the int4 expert layer against the same model with its
// experts left in bf16 (abstract; Tab. 1 and Tab. 4, the "BF16" rows). That baseline is
// built here with the same routing, grouping and combine, so the two layers differ only
// in the expert weights: 2 bytes per weight instead of half a byte plus a scale per 128.
//
// Bank layout (exmoe_bf16_pack): per expert, gate and up row blocks interleaved as in the
// int4 blob, then the down row blocks; each row block is a run of 1 KiB tiles of 16 rows
// x 32 columns in the MFMA operand order (lane l holds row l % 16, columns 8 (l / 16) ..
// + 7), so that one wave-wide 16-byte load is one operand of v_mfma_f32_16x16x32_bf16.
//
// bf16_decode_kernel streams those tiles like the int4 decode kernels: a workgroup owns one
// expert and a slice of output rows, each wave two row blocks (gate and up of one block of
// I, or two blocks of H), kBfRing K steps ahead in registers; the expert's tokens (16 per
// pass) sit in LDS and ride in the N dimension. gate/up writes h = bf16(silu(g) * u);
// down writes y_perm = o * routing weight for the combine.
#include "common.h"
#include "device.h"

namespace exmoe {

constexpr int kBfWaves = 8;
constexpr int kBfThreads = 64 * kBfWaves;
constexpr int kBfTok = 16;                 // tokens per pass: the MFMA N dimension
constexpr int kBfKC = 2048;                // reduction columns staged in LDS at a time
constexpr int kBfXS = kBfKC + 8;           // LDS row stride (bf16): 16-byte skew per row
constexpr int kBfRing = 4;                 // K steps (32 columns, two tiles) in flight per wave
constexpr int kBfTileBytes = 1024;         // 16 rows x 32 columns x 2 bytes
constexpr int kBfCpol = 2;                 // weight loads non-temporal (nt), as in the int4 decode kernels

template <bool GATEUP>
__global__ __launch_bounds__(kBfThreads) void bf16_decode_kernel(MoeArgs a, int per) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[(kBfTok + 1) * kBfXS];   // rows + one zero row
  __shared__ int32_t pf[kBfTok];
  span_begin(a.span);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e = blockIdx.x / per, chunk = blockIdx.x % per;
  const int seg0 = a.offsets[e], cnt = a.offsets[e + 1] - seg0;
  if (cnt <= 0) return;
  const int slot = a.e2s ? a.e2s[e] : e;
  if (slot < 0) {
    if (tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
    return;
  }
  const int K = GATEUP ? a.H : a.I;
  const int KS = K / 32;                   // K steps of this projection
  // the wave's two tile rows (tile index of K step 0) and output row blocks
  int rb0, rb1;
  bool live0 = true, live1 = true;
  uint32_t t0, t1;
  if (GATEUP) {
    rb0 = rb1 = chunk * kBfWaves + wave;   // one block of I: its gate and its up rows
    t0 = (uint32_t)(rb0 * 2) * KS;
    t1 = (uint32_t)(rb0 * 2 + 1) * KS;
  } else {
    const int nrb = a.H / kTileRows;
    rb0 = (chunk * kBfWaves + wave) * 2;
    rb1 = rb0 + 1;
    live0 = rb0 < nrb;
    live1 = rb1 < nrb;
    const uint32_t dbase = 2u * (uint32_t)(a.I / kTileRows) * (uint32_t)(a.H / 32);
    t0 = dbase + (uint32_t)(live0 ? rb0 : nrb - 1) * KS;
    t1 = dbase + (uint32_t)(live1 ? rb1 : nrb - 1) * KS;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  const int nbytes = (int)bf16_expert_bytes(a.H, a.I);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_none = __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, 0, 0x00020000);
  const uint32_t lo = (uint32_t)lane * 16u;
  const int npass = (cnt + kBfTok - 1) / kBfTok;
  const int total = npass * KS;            // ring positions: pass-major, K step minor
  uint4 R0[kBfRing], R1[kBfRing];
  // positions past the last pass load nothing (a zero-length resource returns zeros)
  auto issue = [&](int s, int j) {
    const __amdgpu_buffer_rsrc_t& rs = s < total ? rsrc : rsrc_none;
    const uint32_t kk = (uint32_t)(s % KS);
    R0[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, (int)((t0 + kk) * kBfTileBytes), kBfCpol));
    R1[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo, (int)((t1 + kk) * kBfTileBytes), kBfCpol));
  };
  // the weight stream starts first; the activation rows are staged while it is in flight
#pragma unroll
  for (int j = 0; j < kBfRing; j++) issue(j, j);
  for (int i = tid; i < kBfXS / 8; i += kBfThreads)
    *reinterpret_cast<uint4*>(xs + kBfTok * kBfXS + i * 8) = make_uint4(0u, 0u, 0u, 0u);

  for (int p = 0; p < npass; p++) {
    const int nrow = cnt - p * kBfTok < kBfTok ? cnt - p * kBfTok : kBfTok;
    __syncthreads();   // previous pass done with the row list
    if (tid < kBfTok) {
      const int r = p * kBfTok + tid;
      pf[tid] = r < cnt ? (GATEUP ? a.sorted_flat[seg0 + r] / a.k : seg0 + r) : -1;   // x row or h row
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    for (int kc0 = 0; kc0 < K; kc0 += kBfKC) {
      const int kcw = K - kc0 < kBfKC ? K - kc0 : kBfKC;
      __syncthreads();   // previous chunk consumed; row list visible
      const int cw8 = kcw / 8;
      for (int q = tid; q < nrow * cw8; q += kBfThreads) {
        const int r = q / cw8, c8 = q - r * cw8;
        const uint16_t* src = (GATEUP ? a.x + (size_t)pf[r] * a.H : a.h + (size_t)pf[r] * a.I) + kc0 + c8 * 8;
        *reinterpret_cast<uint4*>(xs + r * kBfXS + c8 * 8) = *reinterpret_cast<const uint4*>(src);
      }
      __syncthreads();
      const uint16_t* xrow = xs + ((lane & 15) < nrow ? (lane & 15) : kBfTok) * kBfXS + 8 * (lane >> 4);
      const int nks = kcw / 32;            // a multiple of 4 = kBfRing
      const int sbase = p * KS + kc0 / 32;
      for (int i0 = 0; i0 < nks; i0 += kBfRing) {
#pragma unroll
        for (int j = 0; j < kBfRing; j++) {
          const bf16x8 act = *reinterpret_cast<const bf16x8*>(xrow + (i0 + j) * 32);
          i32x4 v0 = {(int)R0[j].x, (int)R0[j].y, (int)R0[j].z, (int)R0[j].w};
          i32x4 v1 = {(int)R1[j].x, (int)R1[j].y, (int)R1[j].z, (int)R1[j].w};
          acc0 = mfma16(__builtin_bit_cast(bf16x8, v0), act, acc0);
          acc1 = mfma16(__builtin_bit_cast(bf16x8, v1), act, acc1);
          issue(sbase + i0 + j + kBfRing, j);
        }
      }
    }
    // lane l holds token l % 16 and weight rows 4 (l / 16) + 0..3 of each row block
    const int tok = lane & 15, r4 = 4 * (lane >> 4);
    if (tok < nrow) {
      const int row = seg0 + p * kBfTok + tok;   // sorted row
      if (GATEUP) {
        uint2 pk;
        pk.x = pack_bf16x2(silu_mul(acc0[0], acc1[0]), silu_mul(acc0[1], acc1[1]));
        pk.y = pack_bf16x2(silu_mul(acc0[2], acc1[2]), silu_mul(acc0[3], acc1[3]));
        *reinterpret_cast<uint2*>(a.h + (size_t)row * a.I + rb0 * kTileRows + r4) = pk;
      } else {
        const int f = a.sorted_flat[row];
        const float wgt = a.w[f];
        float* dst = a.y_perm + (size_t)f * a.H;
        if (live0) *reinterpret_cast<float4*>(dst + rb0 * kTileRows + r4) =
            make_float4(acc0[0] * wgt, acc0[1] * wgt, acc0[2] * wgt, acc0[3] * wgt);
        if (live1) *reinterpret_cast<float4*>(dst + rb1 * kTileRows + r4) =
            make_float4(acc1[0] * wgt, acc1[1] * wgt, acc1[2] * wgt, acc1[3] * wgt);
      }
    }
  }
  if (!GATEUP && a.rows_ctr && chunk == 0 && tid == 0) atomicAdd(a.rows_ctr + e, cnt);   // exactness counter
  span_end(a.span);
}

hipError_t launch_bf16_decode_experts(const MoeArgs& a, hipStream_t s) {
  {
    ProfScope prof("bf16_decode_gateup", s);
    MoeArgs as = a;
    as.span = prof.span();
    const int per = a.I / (kTileRows * kBfWaves);
    EXMOE_LAUNCH(prof, bf16_decode_kernel<true>, dim3(a.E * per), dim3(kBfThreads), 0, s, as, per);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope prof("bf16_decode_down", s);
    MoeArgs as = a;
    as.span = prof.span();
    const int per = (a.H / kTileRows + 2 * kBfWaves - 1) / (2 * kBfWaves);
    EXMOE_LAUNCH(prof, bf16_decode_kernel<false>, dim3(a.E * per), dim3(kBfThreads), 0, s, as, per);
  }
  return hipGetLastError();
}

}  // namespace exmoe
