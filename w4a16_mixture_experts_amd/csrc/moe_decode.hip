// Decode-sized expert layer (a few tokens per expert), gfx950.
//
// Every selected expert runs (ExactMoE abstract; Fig. 1). With a handful of tokens per
// expert the layer is bound by streaming the packed int4 weights from HBM, so the expert
// kernels are laid out for bandwidth:
//  * a workgroup owns one active expert and a slice of output rows; each wave streams
//    whole 1 KiB tiles (one wave-wide 128-bit load each), two tiles per 128-input group,
//    kDecRing groups ahead in registers;
//  * the expert's tokens (up to 16 per pass) are staged in LDS and ride in the N
//    dimension of v_mfma_f32_16x16x32_bf16; the activation operand comes from LDS (rows
//    skewed by 16 bytes, so the 16 token rows hit distinct banks).
// Dequantization is exact: a packed word becomes bf16 operands 128 + u (u = q + 8) with
// two bitwise ops per pair; each group's accumulator is seeded with -136 * (sum of that
// group's activations of the token), so the chain ends at sum(x * q); the bf16 row scale
// is applied once per group in fp32.
//
// decode_fused_kernel (most batches): gate/up, SiLU * up and down in one kernel; the
//   workgroup keeps h of its slice of I in LDS and writes fp32 down outputs per slice,
//   which combine_parts_kernel adds in a fixed order with the routing weights. Above 16
//   tokens every 16-row pass of an active expert has workgroups of its own.
// decode_narrow_kernel (a few routed rows): the same in slices of 32 rows of I, so that a
//   single token's experts still cover the chip.
// decode_expert_kernel (shapes the fused kernels do not take): gate/up into h, then down
//   into y_perm (already weighted), then combine_kernel.
// Routing sources: the caller's grouping, the top-k ids (grouped here: histogram, scan
// and ballot over at most kDecMaxRows rows in LDS, and published by the first workgroup
// of each expert), or the routing kernel's per-expert token table (no grouping here; a
// publisher workgroup writes the caller's grouping outputs).
// Workgroups of these kernels never wait on each other.
#include "common.h"
#include "device.h"
#include "group_block.h"
#include "topk.h"

namespace exmoe {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTok = 16;                  // tokens per pass: the MFMA N dimension
constexpr int kDecKC = 2048;                 // reduction columns staged in LDS at a time
constexpr int kDecKG = kDecKC / kGroup;      // 128-input groups per staged chunk
constexpr int kDecXS = kDecKC + 8;           // LDS row stride (bf16): 16-byte skew per row
constexpr int kDecRing = 4;                  // weight groups in flight per wave
constexpr int kSelStride = kSelRowBytes;     // bytes per expert row of the routing table (T <= 16)
// Cache policy of the weight and scale loads of table-routed launches (T <= 16):
// non-temporal (the nt bit of gfx950 buffer loads). There every byte of the packed
// experts is read once per launch; streaming ~190 MB with nt loads measured about 10%
// faster than with default-policy loads on MI355X. Launches whose passes re-read an
// expert (more than 16 rows) keep the default policy, so that the re-reads hit in L2.
constexpr int kWeightCpol = 2;


// In the routing set-up the staging area holds the ids; afterwards the staged rows, and at
// the end of a pass the partial-sum reduction. Row kDecTok stays zero: token slots past
// the expert's rows read it.
struct DecLDS {
  uint16_t xs[(kDecTok + 1) * kDecXS];       // staged activation rows + one zero row
  float seed[(kDecTok + 1) * kDecKG];        // -136 * group sums of the staged rows (+ zeros)
  int32_t cnt[kMaxExperts];
  int32_t off[kMaxExperts + 1];
  int32_t act[kMaxExperts];
  int32_t rows[kDecMaxRows];                 // flat indices of this expert's rows (grouped here)
  int32_t pf[kDecTok];                       // flat indices of the current pass (-1: padding)
  int32_t srows[kDecTok];                    // this expert's flat indices (table routing)
  int32_t n_act;
  int32_t pp_idx, pp_pass;                   // pass-parallel launch: active-expert index and pass
};

struct DecExpert {
  int e, seg0, cnt;
  int row0;   // first of the expert's rows this workgroup takes (pass-parallel launches)
  const uint4* tiles;
  const uint16_t* scales;
};

// Routing source of the expert kernels. kSrcGiven: offsets and permutation come from the
// caller. kSrcIds: top-k ids given; the rows are grouped here and the first workgroup of
// each expert publishes its segment (workgroup 0 the offsets). kSrcSel (T <= 16, H <=
// kDecKC): the routing kernel's table sel[e][t] = slot + 1 when token t selected expert
// e, else 0; every token row of x is staged before the weight stream starts, and a
// publisher workgroup (the grid's last) groups the ids for the caller's outputs.
// kSrcLgt (T <= 16, H <= kDecKC, E <= 64): the routing kernel wrote only the bf16 logits.
// Every workgroup makes the top-k selection itself (one wave per token, ranks by readlane
// compares: the selection of topk_rank_token), exchanges the table columns in LDS and
// finds its expert and tokens by ballots; the publisher workgroup also writes the ids and
// routing weights. This removes the routing kernel's arrival count and read-back.
constexpr int kSrcGiven = 0, kSrcIds = 1, kSrcSel = 2, kSrcLgt = 3;
__host__ __device__ constexpr bool is_sel(int src) { return src == kSrcSel || src == kSrcLgt; }
__host__ __device__ constexpr int weight_cpol(int src) { return is_sel(src) ? kWeightCpol : 0; }
struct DecPublish {
  const uint8_t* sel;        // [E][kSelStride] bytes (kSrcSel)
  int32_t* offsets;
  int32_t* sorted_flat;
  int32_t* flat_to_sorted;
  const uint16_t* logits;    // bf16 [T][E] (kSrcLgt)
  int32_t* ids;              // [T][k], written by the publisher (kSrcLgt)
  float* w;                  // [T][k], written by the publisher (kSrcLgt)
  int renormalize;
};

// The routing inputs of the set-up (ids, offsets or the table), loaded into registers as
// the kernel's very first loads: a wave's vector loads complete in issue order, so these
// must not queue behind the weight prefetch. Unconditional loads at clamped indices.
constexpr int kDecPre = 4;   // per thread: ids <= 2 * 512, offsets <= 257, one 16-byte table row
struct DecPre {
  int32_t v[kDecPre];
};
template <int SRC, int NT>
__device__ __forceinline__ DecPre dec_preload(const MoeArgs& a, const DecPublish& pub) {
  DecPre pr;
  const int tid = threadIdx.x;
  if (SRC == kSrcSel) {
    const int e = tid < a.E ? tid : a.E - 1;
    const uint4 u = *reinterpret_cast<const uint4*>(pub.sel + (size_t)e * kSelStride);
    pr.v[0] = (int32_t)u.x; pr.v[1] = (int32_t)u.y; pr.v[2] = (int32_t)u.z; pr.v[3] = (int32_t)u.w;
    return pr;
  }
  const int n = SRC == kSrcIds ? a.T * a.k : a.E + 1;
#pragma unroll
  for (int m = 0; m < kDecPre; m++) {
    int i = tid + m * NT;
    i = i < n ? i : n - 1;
    pr.v[m] = SRC == kSrcIds ? a.ids[i] : a.offsets[i];
  }
  return pr;
}

// Every token row of x (T <= kDecTok, H <= kDecKC) into the staging rows, indexed by
// token: all loads in flight at once, then the stores. Pieces past the last row load and
// store the last row's piece again (the same value to the same place), so that no load
// sits under a branch, where it would be waited for one at a time.
template <int NT>
__device__ __forceinline__ void dec_prestage_x(const MoeArgs& a, DecLDS& L) {
  constexpr int SQ = kDecTok * (kDecKC / 8) / NT;
  const int tid = threadIdx.x;
  const int cw8 = a.H / 8;
  uint4 v[SQ];
  int dst[SQ];
#pragma unroll
  for (int m = 0; m < SQ; m++) {
    const int q = tid + m * NT;
    int r = q / cw8;
    const int c8 = q - r * cw8;
    r = r < a.T ? r : a.T - 1;
    v[m] = *reinterpret_cast<const uint4*>(a.x + (size_t)r * a.H + c8 * 8);
    dst[m] = r * kDecXS + c8 * 8;
  }
#pragma unroll
  for (int m = 0; m < SQ; m++) *reinterpret_cast<uint4*>(L.xs + dst[m]) = v[m];
}

// The same staging straight from memory into LDS (buffer loads to LDS, 16 bytes per
// lane): no registers are held, so the first weight ring can be issued behind these loads
// at once. Wave w copies staging rows w, w + NW, ... (kDecTok rows); a wave-wide copy
// moves 512 consecutive activations. The count is fixed (kDecTok / NW rows x kDecKC / 512
// copies per wave), with no branch: rows past T copy token T - 1 and columns past H copy
// the row's last 8 values, into staging positions nothing reads. The caller waits for
// completion (the copies count in vmcnt and complete in issue order with the other vector
// loads) and synchronizes the workgroup before reading the rows. (The buffer form, unlike
// the global one, lets the compiler count the loads issued before the copies exactly.)
template <int NW>
__device__ __forceinline__ void dec_dma_x(const MoeArgs& a, DecLDS& L, int wave, int lane) {
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void*)a.x, (short)0, a.T * a.H * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < kDecTok / NW; i++) {
    const int r = wave + i * NW;
    const int src = (r < a.T ? r : a.T - 1) * a.H;
#pragma unroll
    for (int c0 = 0; c0 < kDecKC; c0 += 512) {
      const int c = c0 + 8 * lane < a.H ? c0 + 8 * lane : a.H - 8;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (__attribute__((address_space(3))) void*)(L.xs + r * kDecXS + c0), 16,
                                               2 * (src + c), 0, 0, 0);
    }
  }
}

// kSrcLgt: the logits of the tokens a wave ranks (tokens w, w + NW, ...; lane e: expert
// e, clamped) and the slot of expert `lane`, loaded as the kernel's first loads (through
// zero-length resources where there is nothing to read).
template <int NW>
struct DecLgt {
  uint16_t lg[(kDecTok + NW - 1) / NW];
  int slot;
};
template <int NW>
__device__ __forceinline__ DecLgt<NW> dec_lgt_load(const MoeArgs& a, const DecPublish& pub, int wave, int lane) {
  const int e = lane < a.E ? lane : a.E - 1;
  const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc((void*)pub.logits, (short)0, a.T * a.E * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc((void*)a.e2s, (short)0, a.e2s ? 4 * a.E : 0, 0x00020000);
  DecLgt<NW> r;
#pragma unroll
  for (int i = 0; i < (kDecTok + NW - 1) / NW; i++) {
    const int t = wave + i * NW < a.T ? wave + i * NW : a.T - 1;
    r.lg[i] = __builtin_amdgcn_raw_buffer_load_b16(lr, 2 * (t * a.E + e), 0, 0);
  }
  r.slot = __builtin_amdgcn_raw_buffer_load_b32(er, 4 * e, 0, 0);
  return r;
}

// kSrcLgt: byte t of expert e's table row for each token t < T the wave ranks: rank + 1
// when expert e is among token t's top k (its rank in (logit descending, id ascending)
// order is its slot), else 0 — the selection of topk_rank_token. Lane e computes expert
// e's byte and hands it to put(slot i of the wave's tokens, token, byte).
// The 64 keys go through the wave's own LDS row (skeys: 64 words per wave), where every
// lane reads all of them with broadcast 16-byte reads: no scalar round trip per key. (A
// wave's LDS operations complete in order, so no barrier is needed.)
__device__ __forceinline__ int dec_lgt_byte(const MoeArgs& a, uint16_t lg, int lane, uint32_t* row) {
  const uint32_t key = lane < a.E ? order_key(lg, lane) : 0u;
  row[lane] = key;
  int rank = 0;
#pragma unroll
  for (int q = 0; q < 16; q++) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + 4 * q);
    rank += (v.x > key ? 1 : 0) + (v.y > key ? 1 : 0) + (v.z > key ? 1 : 0) + (v.w > key ? 1 : 0);
  }
  return lane < a.E && rank < a.k ? rank + 1 : 0;
}
template <int NW, class Put>
__device__ __forceinline__ void dec_lgt_ranks(const MoeArgs& a, const DecLgt<NW>& r, int wave, int lane,
                                              uint32_t* skeys, Put put) {
#pragma unroll
  for (int i = 0; i < (kDecTok + NW - 1) / NW; i++) {
    const int t = wave + i * NW;
    if (t >= a.T) break;   // uniform
    put(i, t, dec_lgt_byte(a, r.lg[i], lane, skeys + wave * 64));
  }
}

// kSrcLgt, launches of the active experts: the table row of expert `lane`. With one token
// every wave ranks it itself (its logits are what every wave loaded); otherwise wave w
// ranks tokens w, w + NW, ..., the columns meet in LDS (stab: 64 rows of kDecTok bytes)
// and every wave reads the rows after a barrier.
template <int NW>
__device__ __forceinline__ uint4 dec_lgt_rows(const MoeArgs& a, const DecLgt<NW>& r, int wave, int lane,
                                              uint32_t* skeys, uint8_t* stab) {
  if (a.T == 1) return make_uint4((uint32_t)dec_lgt_byte(a, r.lg[0], lane, skeys + wave * 64), 0u, 0u, 0u);
  dec_lgt_ranks<NW>(a, r, wave, lane, skeys, [&](int, int t, int b) { stab[lane * kDecTok + t] = (uint8_t)b; });
  __syncthreads();
  return *reinterpret_cast<const uint4*>(&stab[lane * kDecTok]);
}

// The table row of expert `lane` and that expert's slot.
struct DecSelRow {
  uint4 row;
  int slot;
};

// kSrcLgt: the workgroup's expert is the ai-th active one in ascending id order (active:
// at least one of the T tokens selected it). Its tokens, ascending, are L.srows: lane t <
// T of wave 0 holds in `tok` its position in that list and its flat index when token t
// selected the expert (else -1); the caller writes them once the activation copies have
// landed (an LDS store before that would wait for them) and its barrier publishes them.
// Returns false when there is no ai-th active expert. Every wave computes the same
// uniform values from the same rows.
struct DecSelTok {
  int pos, flat;
};
__device__ __forceinline__ bool dec_sel_pick(const MoeArgs& a, const DecSelRow& r, int ai, int lane, DecExpert& ex,
                                             int& slot, DecSelTok& tok) {
  const uint32_t w4[4] = {r.row.x, r.row.y, r.row.z, r.row.w};
  int c = 0;
#pragma unroll
  for (int q = 0; q < kDecTok; q++) c += (q < a.T && ((w4[q >> 2] >> (8 * (q & 3))) & 0xFFu)) ? 1 : 0;
  const bool on = lane < a.E && c > 0;
  const uint64_t m = __ballot(on);
  if (ai >= __popcll(m)) return false;
  const uint64_t pick = __ballot(on && __popcll(m & ((1ull << lane) - 1ull)) == ai);
  const int e = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(pick));
  ex.e = e;
  ex.cnt = __builtin_amdgcn_readlane(c, e);
  ex.seg0 = 0;
  ex.row0 = 0;
  slot = a.e2s ? __builtin_amdgcn_readlane(r.slot, e) : e;
  const uint32_t rw[4] = {(uint32_t)__builtin_amdgcn_readlane((int)r.row.x, e), (uint32_t)__builtin_amdgcn_readlane((int)r.row.y, e),
                          (uint32_t)__builtin_amdgcn_readlane((int)r.row.z, e), (uint32_t)__builtin_amdgcn_readlane((int)r.row.w, e)};
  const int tq = lane & 15;
  const uint32_t wd = tq < 4 ? rw[0] : tq < 8 ? rw[1] : tq < 12 ? rw[2] : rw[3];
  const int sb = lane < a.T ? (int)((wd >> (8 * (lane & 3))) & 0xFFu) : 0;
  const uint64_t mt = __ballot(sb > 0);
  tok.pos = sb > 0 ? __popcll(mt & ((1ull << lane) - 1ull)) : -1;
  tok.flat = lane * a.k + sb - 1;
  return true;
}

// Publisher of a table-routed launch (the grid's last workgroup): stable grouping of the
// ids, into the caller's offsets / sorted_flat / flat_to_sorted. kSrcSel: the ids the
// routing kernel wrote; kSrcLgt: the top-k selection and weights of every token made here
// from the logits (one wave per token), also written to the caller's ids and weights.
template <int SRC, int NT>
__device__ void dec_publish(const MoeArgs& a, DecLDS& L, const DecPublish& pub) {
  int32_t* ids_l = reinterpret_cast<int32_t*>(L.xs);
  auto& gs = *reinterpret_cast<GroupSharedT<NT>*>(L.xs + 2 * kDecMaxRows);
  static_assert(2 * kDecMaxRows * 2 + sizeof(GroupSharedT<NT>) <= sizeof(L.xs), "publisher scratch exceeds the staging rows");
  const int TK = a.T * a.k;
  if (SRC == kSrcLgt) {
    const int lane = (int)lane_id(), wave = threadIdx.x >> 6;
    for (int t = wave; t < a.T; t += NT / 64) {
      int id;
      float wt;
      topk_rank_token(pub.logits + (size_t)t * a.E, a.E, a.k, pub.renormalize, id, wt);
      if (lane < a.k) {
        ids_l[t * a.k + lane] = id;
        pub.ids[t * a.k + lane] = id;
        pub.w[t * a.k + lane] = wt;
      }
    }
  } else {
    for (int f = threadIdx.x; f < TK; f += NT) ids_l[f] = a.ids[f];
  }
  __syncthreads();
  group_block<NT>(ids_l, TK, a.E, pub.offsets, pub.sorted_flat, pub.flat_to_sorted, gs);
}

// The publisher's work done by a workgroup that also runs an expert slice (logit routing,
// E <= 64): wave t ranks token t from the logits it loaded first (lane e: expert e) through
// an LDS row of its own, writes ids and weights, and the workgroup groups the ids. Called
// once the slice's weight loads are in flight, so that it runs while they land.
template <int NT>
struct DecPubLDS {
  uint16_t lg[kDecTok][64];
  int32_t ids[kDecTok * 64];
  GroupSharedT<NT> gs;
};
template <int NW, int NT>
__device__ void dec_publish_lgt(const MoeArgs& a, const DecLgt<NW>& lgt, int wave, int lane, const DecPublish& pub,
                                DecPubLDS<NT>& P) {
  static_assert(NW * 64 == NT && (kDecTok + NW - 1) / NW == 1, "one token per wave");
  if (wave < a.T) {
    if (lane < a.E) P.lg[wave][lane] = lgt.lg[0];
    int id;
    float wt;
    topk_rank_token(P.lg[wave], a.E, a.k, pub.renormalize, id, wt);
    if (lane < a.k) {
      P.ids[wave * a.k + lane] = id;
      pub.ids[wave * a.k + lane] = id;
      pub.w[wave * a.k + lane] = wt;
    }
  }
  __syncthreads();
  group_block<NT>(P.ids, a.T * a.k, a.E, pub.offsets, pub.sorted_flat, pub.flat_to_sorted, P.gs);
}

// pp (pass-parallel, not ALL): aidx counts 16-row passes over the active experts in
// ascending order instead of the experts themselves, so that a hot expert's passes run in
// workgroups of their own; ex.row0 / ex.cnt are then this pass's rows.
template <int SRC, bool ALL, int NT>
__device__ bool dec_setup(const MoeArgs& a, DecLDS& L, const DecPublish& pub, const DecPre& pr, int fixed_expert,
                          int aidx, bool first_of_expert, int slot_known, DecExpert& ex, bool pp = false) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int TK = a.T * a.k;
  int32_t* ids_l = reinterpret_cast<int32_t*>(L.xs);            // staging rows are free (ids mode)
  uint8_t* selb = reinterpret_cast<uint8_t*>(L.rows);            // table rows (sel mode)
  if (SRC == kSrcSel) {
    if (tid < a.E) {
      const uint4 u = make_uint4((uint32_t)pr.v[0], (uint32_t)pr.v[1], (uint32_t)pr.v[2], (uint32_t)pr.v[3]);
      *reinterpret_cast<uint4*>(selb + tid * kSelStride) = u;
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
      int c = 0;
#pragma unroll
      for (int q = 0; q < 16; q++) c += (q < a.T && ((w4[q >> 2] >> (8 * (q & 3))) & 0xFFu)) ? 1 : 0;
      L.cnt[tid] = c;
    }
  } else if (SRC == kSrcIds) {
#pragma unroll
    for (int m = 0; m < kDecPre; m++)
      if (tid + m * NT < TK) ids_l[tid + m * NT] = pr.v[m];
  }
  if (SRC != kSrcGiven) {
    if (SRC == kSrcIds) {
      for (int i = tid; i < a.E; i += NT) L.cnt[i] = 0;
      __syncthreads();
      for (int f = tid; f < TK; f += NT) {
        const int e = ids_l[f];
        if ((unsigned)e < (unsigned)a.E) atomicAdd(&L.cnt[e], 1);
      }
    }
    __syncthreads();
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 < a.E; c0 += 64) {
        const int e = c0 + lane;
        const int v = e < a.E ? L.cnt[e] : 0;
        int incl = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(incl, d);
          if (lane >= d) incl += u;
        }
        if (e < a.E) L.off[e] = base + incl - v;
        base += __shfl(incl, 63);
      }
      if (lane == 0) L.off[a.E] = base;
    }
  } else {
    if (tid <= a.E) L.off[tid] = pr.v[0];
  }
  __syncthreads();
  if (!ALL && wave == 0) {
    if (fixed_expert >= 0) {
      if (lane == 0) {
        L.act[0] = fixed_expert;
        L.n_act = 1;
      }
    } else {
      int base = 0;
      for (int c0 = 0; c0 < a.E; c0 += 64) {
        const int e = c0 + lane;
        const bool on = e < a.E && L.off[e + 1] > L.off[e];
        const uint64_t m = __ballot(on);
        if (on) L.act[base + __popcll(m & ((1ull << lane) - 1ull))] = e;
        base += __popcll(m);
      }
      if (lane == 0) L.n_act = base;
    }
  }
  __syncthreads();
  if (!ALL && pp) {
    if (wave == 0) {
      if (lane == 0) L.pp_idx = -1;   // past the last pass: nothing to do
      int base = 0;
      for (int i0 = 0; i0 < L.n_act; i0 += 64) {
        const int i = i0 + lane;
        const int e = i < L.n_act ? L.act[i] : 0;
        const int np = i < L.n_act ? (L.off[e + 1] - L.off[e] + kDecTok - 1) / kDecTok : 0;
        int incl = np;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int u = __shfl_up(incl, d);
          if (lane >= d) incl += u;
        }
        const int excl = base + incl - np;
        if (np > 0 && aidx >= excl && aidx < excl + np) {
          L.pp_idx = i;
          L.pp_pass = aidx - excl;
        }
        base += __shfl(incl, 63);
      }
    }
    __syncthreads();
  }
  const int ai = !ALL && pp ? L.pp_idx : aidx;
  const int pass = !ALL && pp ? L.pp_pass : 0;
  if (!ALL && (ai < 0 || ai >= L.n_act)) return false;
  // uniform values: keep them (and the addresses built from them) in scalar registers
  ex.e = ALL ? aidx : __builtin_amdgcn_readfirstlane(L.act[ai]);
  ex.seg0 = __builtin_amdgcn_readfirstlane(L.off[ex.e]);
  ex.cnt = __builtin_amdgcn_readfirstlane(L.off[ex.e + 1]) - ex.seg0;
  ex.row0 = 0;
  if (SRC == kSrcSel) {
    // the tokens that selected this expert, ascending (the table gives each one's slot)
    if (wave == 0) {
      const int sb = lane < a.T ? selb[ex.e * kSelStride + lane] : 0;
      const uint64_t m = __ballot(sb > 0);
      if (sb > 0) L.srows[__popcll(m & ((1ull << lane) - 1ull))] = lane * a.k + sb - 1;
    }
    __syncthreads();
  }
  if (SRC == kSrcIds) {
    if (wave == 0) {
      int base = 0;
      for (int c0 = 0; c0 < TK; c0 += 64) {
        const int f = c0 + lane;
        const bool on = f < TK && ids_l[f] == ex.e;
        const uint64_t m = __ballot(on);
        if (on) L.rows[base + __popcll(m & ((1ull << lane) - 1ull))] = f;
        base += __popcll(m);
      }
    }
    __syncthreads();
    if (first_of_expert && pass == 0) {
      for (int r = tid; r < ex.cnt; r += NT) {
        const int f = L.rows[r];
        pub.sorted_flat[ex.seg0 + r] = f;
        pub.flat_to_sorted[f] = ex.seg0 + r;
      }
    }
    if (blockIdx.x == 0)
      for (int i = tid; i <= a.E; i += NT) pub.offsets[i] = L.off[i];
  }
  if (ex.cnt <= 0) return false;
  if (pass > 0 || pp) {   // this pass's rows only
    ex.row0 = __builtin_amdgcn_readfirstlane(pass * kDecTok);
    ex.cnt = ex.cnt - ex.row0 < kDecTok ? ex.cnt - ex.row0 : kDecTok;
  }
  const int slot = ALL ? slot_known : a.e2s ? __builtin_amdgcn_readfirstlane(a.e2s[ex.e]) : ex.e;
  if (slot < 0) {
    if (tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
    return false;
  }
  const uint8_t* blob = a.base + a.stride * (size_t)slot;
  ex.tiles = reinterpret_cast<const uint4*>(blob);
  ex.scales = reinterpret_cast<const uint16_t*>(blob + n_tiles(a.H, a.I) * kTileBytes);
  return true;
}

struct WSlot2 {
  uint4 w[2];
  uint2 s[2];
};

// ------------------------------------------------------------------------------------
// One kernel body for both projections. GATEUP: wave row = one 16-row block of I, its
// gate and up tiles; reduction over H. DOWN: wave row = two 16-row blocks of H; reduction
// over I. Workgroup = (active expert, chunk of output rows); KS waves per wave row split
// the groups of each staged chunk (g = kpart, kpart + KS, ...).
// ------------------------------------------------------------------------------------
template <bool GATEUP, int SRC, int KS, bool ALL>
__global__ __launch_bounds__(kDecThreads, 4) void decode_expert_kernel(MoeArgs a, DecPublish pub, int fixed_expert,
                                                                    int nchunk) {
  __shared__ DecLDS L;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  span_begin(a.span);
  const int tid = threadIdx.x;
  const int aidx = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;

  constexpr int RBW = kDecWaves / KS;           // wave rows per workgroup
  constexpr int PER = kDecKG / KS;              // groups of a staged chunk per wave
  const int wrow = wave / KS, kpart = wave % KS;
  const int K = GATEUP ? a.H : a.I;
  const int G = K / kGroup;
  const int nK = (K + kDecKC - 1) / kDecKC;
  int rb0, rb1;
  bool live0, live1;
  size_t t0, t1;
  if (GATEUP) {
    rb0 = chunk * RBW + wrow;
    rb1 = rb0;
    live0 = live1 = rb0 < a.I / kTileRows;
    const int rbc = live0 ? rb0 : a.I / kTileRows - 1;
    t0 = (size_t)(rbc * 2) * G;
    t1 = (size_t)(rbc * 2 + 1) * G;
  } else {
    const int nrb = a.H / kTileRows;
    rb0 = (chunk * RBW + wrow) * 2;
    rb1 = rb0 + 1;
    live0 = rb0 < nrb;
    live1 = rb1 < nrb;
    const size_t dbase = 2 * (size_t)(a.I / kTileRows) * (a.H / kGroup);
    t0 = dbase + (size_t)(live0 ? rb0 : nrb - 1) * G;
    t1 = dbase + (size_t)(live1 ? rb1 : nrb - 1) * G;
  }
  // The blob through a buffer resource: uniform byte offsets of the wave's two tile rows
  // go in scalar registers, the lane's offset in one vector register.
  const uint32_t sc_base = (uint32_t)(n_tiles(a.H, a.I) * kTileBytes);
  const int nbytes = (int)packed_bytes(a.H, a.I);
  const uint32_t lo_t = (uint32_t)lane * 16u, lo_s = (uint32_t)(lane >> 4) * 8u;
  const uint32_t t0b = (uint32_t)t0 * kTileBytes, t1b = (uint32_t)t1 * kTileBytes;
  const uint32_t s0b = sc_base + (uint32_t)t0 * kScaleBytes, s1b = sc_base + (uint32_t)t1 * kScaleBytes;
  // Sequence index s -> group: staged chunk c = s / PER holds ngc groups, split in KS
  // contiguous runs of pg; positions past a run repeat its last group (cache hits).
  auto gof = [&](int s) {
    const int c = s / PER, i = s % PER;
    const int ngc = G - c * kDecKG < kDecKG ? G - c * kDecKG : kDecKG;
    const int pg = (ngc + KS - 1) / KS;
    const int g = c * kDecKG + kpart * pg + (i < pg ? i : pg - 1);
    return g < G ? (g >= 0 ? g : 0) : G - 1;
  };
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, int s, WSlot2& w) {
    const uint32_t g = (uint32_t)gof(s);
    w.w[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo_t, (int)(t0b + g * kTileBytes), weight_cpol(SRC)));
    w.w[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo_t, (int)(t1b + g * kTileBytes), weight_cpol(SRC)));
    w.s[0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, lo_s, (int)(s0b + g * kScaleBytes), weight_cpol(SRC)));
    w.s[1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, lo_s, (int)(s1b + g * kScaleBytes), weight_cpol(SRC)));
  };

  for (int i = tid; i < kDecXS / 8; i += kDecThreads)
    *reinterpret_cast<uint4*>(L.xs + kDecTok * kDecXS + i * 8) = make_uint4(0u, 0u, 0u, 0u);
  if (tid < kDecKG) L.seed[kDecTok * kDecKG + tid] = 0.f;

  // all-experts launch: the expert's slot, loaded first so that its latency overlaps the
  // activation loads (the publisher's index is clamped; it returns before using it)
  // (a vector load: a scalar one would be waited for with the kernel arguments)
  // (a resident bank has no slot table: the slot is the expert, and nothing waits for it)
  int slot = aidx;
  if (ALL && a.e2s) {
    const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc((void*)a.e2s, (short)0, 4 * a.E, 0x00020000);
    slot = __builtin_amdgcn_raw_buffer_load_b32(er, 4 * (aidx < a.E ? aidx : a.E - 1), 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep the load here, ahead of the others
  }
  const DecPre pre = dec_preload<SRC, kDecThreads>(a, pub);
  if (GATEUP && SRC == kSrcSel && blockIdx.x == gridDim.x - 1) {
    dec_publish<SRC, kDecThreads>(a, L, pub);
    return;
  }
  if (GATEUP && SRC == kSrcSel) dec_prestage_x<kDecThreads>(a, L);
  // ALL: the grid covers every expert, so the expert (hence its weights) is known at once:
  // the first ring of weight loads goes out right behind the routing inputs and arrives
  // while the routing is worked out. Loads through a resource of zero length (expert
  // without a slot, or no next pass) return zeros without touching memory; issuing them
  // anyway keeps every wave's load count fixed, so the waits stay exact.
  WSlot2 W[kDecRing];
  __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a.base, (short)0, 0, 0x00020000);
  if (ALL) {
    if (a.e2s) slot = __builtin_amdgcn_readfirstlane(slot);
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.base + a.stride * (size_t)(slot >= 0 ? slot : 0)), (short)0,
                                             slot >= 0 ? nbytes : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < kDecRing; j++) issue(rsrc, j, W[j]);
  }
  DecExpert ex;
  if (!dec_setup<SRC, ALL, kDecThreads>(a, L, pub, pre, fixed_expert, aidx, chunk == 0, slot, ex)) return;
  if (!ALL) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < kDecRing; j++) issue(rsrc, j, W[j]);
  }
  const __amdgpu_buffer_rsrc_t rsrc_none = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, 0, 0x00020000);

  const int npass = (ex.cnt + kDecTok - 1) / kDecTok;
  for (int p = 0; p < npass; p++) {
    const int nrow = ex.cnt - p * kDecTok < kDecTok ? ex.cnt - p * kDecTok : kDecTok;
    if (GATEUP && tid < kDecTok) {
      const int r = p * kDecTok + tid;
      L.pf[tid] = r < ex.cnt ? (SRC == kSrcSel ? L.srows[r] : SRC == kSrcIds ? L.rows[r] : a.sorted_flat[ex.seg0 + r])
                             : -1;
    }
    // down: the rows to stage are contiguous in h; the flat index is needed only at the end
    int f_out = -1;
    if (!GATEUP && (lane & 15) < nrow) f_out = a.sorted_flat[ex.seg0 + p * kDecTok + (lane & 15)];
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nK; c++) {
      const int kc0 = c * kDecKC;
      const int kcw = K - kc0 < kDecKC ? K - kc0 : kDecKC;
      const int ngc = kcw / kGroup;
      __syncthreads();   // previous chunk consumed; pass row list visible
      if (!(GATEUP && SRC == kSrcSel)) {   // table routing: every token row is already staged
        const int cw8 = kcw / 8;
        for (int q = tid; q < nrow * cw8; q += kDecThreads) {
          const int r = q / cw8, c8 = q - r * cw8;
          const size_t row = GATEUP ? (size_t)(L.pf[r] / a.k) * a.H : (size_t)(ex.seg0 + p * kDecTok + r) * a.I;
          *reinterpret_cast<uint4*>(L.xs + r * kDecXS + c8 * 8) =
              *reinterpret_cast<const uint4*>((GATEUP ? a.x : a.h) + row + kc0 + c8 * 8);
        }
      }
      __syncthreads();
      const int nstaged = GATEUP && SRC == kSrcSel ? a.T : nrow;   // rows indexed by token or by slot
      for (int q = tid; q < nstaged * ngc * 2; q += kDecThreads) {
        const int r = q / (ngc * 2), gg = (q >> 1) % ngc, half = q & 1;
        const uint16_t* src = L.xs + r * kDecXS + gg * kGroup + half * 64;
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const uint4 u = *reinterpret_cast<const uint4*>(src + 8 * i);
          const uint32_t q4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int m = 0; m < 4; m++) {
            s += __uint_as_float(q4[m] << 16);
            s += __uint_as_float(q4[m] & 0xFFFF0000u);
          }
        }
        const float o = __shfl_xor(s, 1);
        if (!half) L.seed[r * kDecKG + gg] = -136.0f * (s + o);
      }
      __syncthreads();

      const int pg = (ngc + KS - 1) / KS;
      // padding slots read the zero row; table routing stages rows by token
      const int myrow = (lane & 15) < nrow ? (GATEUP && SRC == kSrcSel ? L.pf[lane & 15] / a.k : (lane & 15)) : kDecTok;
      const uint16_t* xrow = L.xs + myrow * kDecXS + 8 * (lane >> 4);
      const float* srow = L.seed + myrow * kDecKG;
#pragma unroll
      for (int i0 = 0; i0 < PER; i0 += kDecRing) {
#pragma unroll
        for (int j = 0; j < kDecRing; j++) {
          const int gl = kpart * pg + i0 + j;
          if (i0 + j < pg && gl < ngc) {
            bf16x8 act[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) act[s4] = *reinterpret_cast<const bf16x8*>(xrow + gl * kGroup + 32 * s4);
            const float sd = srow[gl];
            f32x4 c0 = {sd, sd, sd, sd}, c1 = c0;
            c0 = mfma16(dequant_word(W[j].w[0].x), act[0], c0);
            c1 = mfma16(dequant_word(W[j].w[1].x), act[0], c1);
            c0 = mfma16(dequant_word(W[j].w[0].y), act[1], c0);
            c1 = mfma16(dequant_word(W[j].w[1].y), act[1], c1);
            c0 = mfma16(dequant_word(W[j].w[0].z), act[2], c0);
            c1 = mfma16(dequant_word(W[j].w[1].z), act[2], c1);
            c0 = mfma16(dequant_word(W[j].w[0].w), act[3], c0);
            c1 = mfma16(dequant_word(W[j].w[1].w), act[3], c1);
            scale_accum(acc0, c0, W[j].s[0]);
            scale_accum(acc1, c1, W[j].s[1]);
          }
          // past this pass's last group the ring runs on into the next pass (the same
          // groups again); after the last pass it loads nothing
          const int sn = c * PER + i0 + j + kDecRing, wrap = sn >= nK * PER;
          issue(wrap ? (p + 1 < npass ? rsrc : rsrc_none) : rsrc, wrap ? sn - nK * PER : sn, W[j]);
        }
      }
    }

    if (KS > 1) {
      __syncthreads();   // every wave done with the staged rows: reuse them for partial sums
      f32x4* red = reinterpret_cast<f32x4*>(L.xs);
      red[(wave * 2 + 0) * 64 + lane] = acc0;
      red[(wave * 2 + 1) * 64 + lane] = acc1;
      __syncthreads();
      if (kpart == 0) {
#pragma unroll
        for (int kp = 1; kp < KS; kp++) {
          acc0 += red[((wave + kp) * 2 + 0) * 64 + lane];
          acc1 += red[((wave + kp) * 2 + 1) * 64 + lane];
        }
      }
    }
    if (kpart == 0) {
      const int r = lane & 15;
      const int f = GATEUP ? L.pf[r] : f_out;
      if (f >= 0) {
        if (GATEUP) {
          if (live0) {
            uint2 pk;
            pk.x = pack_bf16x2(silu_mul(acc0[0], acc1[0]), silu_mul(acc0[1], acc1[1]));
            pk.y = pack_bf16x2(silu_mul(acc0[2], acc1[2]), silu_mul(acc0[3], acc1[3]));
            *reinterpret_cast<uint2*>(a.h + (size_t)(ex.seg0 + p * kDecTok + r) * a.I + rb0 * 16 + 4 * (lane >> 4)) = pk;
          }
        } else {
          const float wt = a.w[f];
          float* yrow = a.y_perm + (size_t)f * a.H + 4 * (lane >> 4);
          if (live0)
            *reinterpret_cast<float4*>(yrow + rb0 * 16) = make_float4(acc0[0] * wt, acc0[1] * wt, acc0[2] * wt, acc0[3] * wt);
          if (live1)
            *reinterpret_cast<float4*>(yrow + rb1 * 16) = make_float4(acc1[0] * wt, acc1[1] * wt, acc1[2] * wt, acc1[3] * wt);
        }
      }
    }
    __syncthreads();   // pass row list and reduction space free for the next pass
  }
  // exactness counter: the down projection's first chunk counts the rows it wrote
  if (!GATEUP && a.rows_ctr && chunk == 0 && tid == 0) atomicAdd(a.rows_ctr + ex.e, ex.cnt);
  span_end(a.span);
}

// ------------------------------------------------------------------------------------
// Fused gate/up + down, NW = 8 or 16 waves. Workgroup = (expert, slice c of RS = 16 NW
// rows of I); wave w owns row block NW c + w of I. Phase 1 computes h for the slice (gate
// and up tiles, reduction over H) into LDS; phase 2 applies the slice's RS columns of
// W_down, which are exactly input groups NCG c .. NCG c + NCG - 1 (NCG = NW / 8) of every
// down tile row, to all H outputs: each wave streams those tiles for its share of the H
// row blocks. The result goes to part[c][f][H]; the combine adds the slices and applies
// the routing weight. h never leaves the chip, and one kernel boundary (its ramp, set-up
// and tail) disappears. One weight ring runs through both phases: slots 0 .. S1-1 hold
// gate/up groups, then two down tiles each (two row blocks at NW = 8, the slice's two
// groups of one row block at NW = 16).
// With 16 waves one workgroup fills a compute unit: two 8-wave workgroups sharing one do
// not stream evenly (the older one's waves win the issue arbitration and the younger one
// ends far later), while the waves of one workgroup meet at its barriers; the token rows
// are also staged once per compute unit instead of twice, and the slices are twice as
// wide, which halves the partial outputs the combine reads.
// ------------------------------------------------------------------------------------
template <int SRC, bool ALL, int NW>
__global__ __launch_bounds__(64 * NW) void decode_fused_kernel(MoeArgs a, DecPublish pub, int fixed_expert, int pp) {
  static_assert(NW == 8 || NW == 16, "8 or 16 waves");
  constexpr int NT = 64 * NW, RS = kTileRows * NW, NCG = NW / 8;
  __shared__ DecLDS L;
  const int lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  span_begin(a.span);
  const int tid = threadIdx.x;
  const int nslice = a.I / RS;
  const int aidx = blockIdx.x / nslice, cs = blockIdx.x % nslice;

  const int G = a.H / kGroup;                  // gate/up groups
  const int nK = (a.H + kDecKC - 1) / kDecKC;  // staged chunks of x
  const int S1 = nK * kDecKG;                  // phase-1 ring positions
  const int nrbd = a.H / kTileRows;            // down row blocks
  const int per_w = (nrbd + NW - 1) / NW;      // down row blocks per wave
  const int npos2 = NCG == 1 ? (per_w + 1) / 2 : per_w;          // phase-2 positions in use
  const int S2 = (npos2 + kDecRing - 1) / kDecRing * kDecRing;   // phase-2 ring positions
  const int ST = S1 + S2;
  const int rb = cs * NW + wave;               // gate/up row block of this wave
  const int rbd_base = wave * per_w;
  const int Gd = a.I / kGroup;
  const uint32_t sc_base = (uint32_t)(n_tiles(a.H, a.I) * kTileBytes);
  const uint32_t dbase = 2u * (uint32_t)(a.I / kTileRows) * (uint32_t)G;
  const int nbytes = (int)packed_bytes(a.H, a.I);
  const uint32_t lo_t = (uint32_t)lane * 16u, lo_s = (uint32_t)(lane >> 4) * 8u;
  const uint32_t tg0 = (uint32_t)(rb * 2) * G, tg1 = (uint32_t)(rb * 2 + 1) * G;
  const bf16x8 n136 = neg136_operand();
  // tile indices of ring position s (uniform): gate/up group, or two down tiles
  auto tiles_of = [&](int s, uint32_t& ta, uint32_t& tb) {
    if (s < S1) {
      const int c = s / kDecKG, i = s % kDecKG;
      int g = c * kDecKG + i;
      g = g < G ? g : G - 1;
      ta = tg0 + g;
      tb = tg1 + g;
    } else {
      const int pi = s - S1;
      const int rmax = rbd_base + per_w - 1 < nrbd - 1 ? rbd_base + per_w - 1 : nrbd - 1;
      if (NCG == 1) {
        int r0 = rbd_base + 2 * pi, r1 = r0 + 1;
        r0 = r0 < rmax ? r0 : rmax;
        r1 = r1 < rmax ? r1 : rmax;
        ta = dbase + (uint32_t)r0 * Gd + cs;
        tb = dbase + (uint32_t)r1 * Gd + cs;
      } else {
        int r = rbd_base + pi;
        r = r < rmax ? r : rmax;
        ta = dbase + (uint32_t)r * Gd + 2 * cs;
        tb = ta + 1;
      }
    }
  };
  auto issue = [&](const __amdgpu_buffer_rsrc_t& rs, int s, WSlot2& w) {
    uint32_t ta, tb;
    tiles_of(s, ta, tb);
    w.w[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo_t, (int)(ta * kTileBytes), weight_cpol(SRC)));
    w.w[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, lo_t, (int)(tb * kTileBytes), weight_cpol(SRC)));
    w.s[0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, lo_s, (int)(sc_base + ta * kScaleBytes), weight_cpol(SRC)));
    w.s[1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, lo_s, (int)(sc_base + tb * kScaleBytes), weight_cpol(SRC)));
  };

  for (int i = tid; i < kDecXS / 8; i += NT)
    *reinterpret_cast<uint4*>(L.xs + kDecTok * kDecXS + i * 8) = make_uint4(0u, 0u, 0u, 0u);

  // all-experts launch: the expert's slot, loaded first so that its latency overlaps the
  // activation loads (the publisher's index is clamped; it returns before using it)
  // (a vector load: a scalar one would be waited for with the kernel arguments)
  // (a resident bank has no slot table: the slot is the expert, and nothing waits for it)
  int slot = aidx;
  if (ALL && a.e2s) {
    const __amdgpu_buffer_rsrc_t er = __builtin_amdgcn_make_buffer_rsrc((void*)a.e2s, (short)0, 4 * a.E, 0x00020000);
    slot = __builtin_amdgcn_raw_buffer_load_b32(er, 4 * (aidx < a.E ? aidx : a.E - 1), 0, 0);
    __builtin_amdgcn_sched_barrier(0);   // keep the load here, ahead of the others
  }
  // table routing with every expert launched: this expert's 16-byte table row in every
  // lane (a vector load, like the slot's), or (logit routing) the logits of the wave's
  // tokens, from which that row is made here
  constexpr bool kSelAll = SRC == kSrcSel && ALL;
  constexpr bool kLgt = SRC == kSrcLgt;
  constexpr bool kTabAll = (SRC == kSrcSel || kLgt) && ALL;   // the token list from one table row
  constexpr int TPW = (kDecTok + NW - 1) / NW;                // tokens ranked per wave
  __shared__ __attribute__((aligned(16))) uint8_t s_tab[64 * kDecTok];   // logit routing: table rows
  __shared__ __attribute__((aligned(16))) uint32_t s_keys[kLgt && !ALL ? NW * 64 : 4];   // logit routing: keys
  uint4 selrow = make_uint4(0u, 0u, 0u, 0u);
  DecPre pre;
  DecLgt<NW> lgt;
  DecSelTok stok;
  if (kSelAll) {
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void*)pub.sel, (short)0, a.E * kSelStride, 0x00020000);
    selrow = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(sr, (aidx < a.E ? aidx : a.E - 1) * kSelStride, 0, 0));
  } else if (kLgt) {
    lgt = dec_lgt_load<NW>(a, pub, wave, lane);
  } else {
    pre = dec_preload<SRC, NT>(a, pub);
  }
  if (is_sel(SRC) && blockIdx.x == gridDim.x - 1) {
    dec_publish<SRC, NT>(a, L, pub);
    return;
  }
  // every token row of x straight into LDS; with every expert launched the first weight
  // ring goes out right behind those copies
  if (kTabAll) dec_dma_x<NW>(a, L, wave, lane);
  else if (SRC == kSrcSel) dec_prestage_x<NT>(a, L);
  __builtin_amdgcn_sched_barrier(0);
  WSlot2 W[kDecRing];
  __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)a.base, (short)0, 0, 0x00020000);
  if (ALL) {
    if (a.e2s) slot = __builtin_amdgcn_readfirstlane(slot);
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.base + a.stride * (size_t)(slot >= 0 ? slot : 0)), (short)0,
                                             slot >= 0 ? nbytes : 0, 0x00020000);
#pragma unroll
    for (int j = 0; j < kDecRing; j++) issue(rsrc, j, W[j]);
  }
  if (kTabAll) {
    // logit routing: this expert's byte of each of the wave's tokens (uniform), while the
    // copies and the ring are in flight
    // (one expert's rank per token: the number of experts whose key is above its own, by one
    // ballot; the same order as the full ranks)
    uint8_t tb[TPW];
    if (kLgt) {
#pragma unroll
      for (int i = 0; i < TPW; i++) {
        const uint32_t key = lane < a.E ? order_key(lgt.lg[i], lane) : 0u;
        const uint32_t mine = (uint32_t)__builtin_amdgcn_readlane((int)key, aidx < a.E ? aidx : 0);
        const int rank = __popcll(__ballot(key > mine));
        tb[i] = (uint8_t)(rank < a.k ? rank + 1 : 0);
      }
    }
    // the activation copies are older than the 4 x 4 ring loads: vmcnt(16) is their
    // completion (expcnt and lgkmcnt left at their maxima); the barrier below (token list)
    // publishes every wave's rows
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x4F70);
    static_assert(kDecRing * 4 == 16, "the wait above counts 16 ring loads");
    if (kLgt) {
      // (stored after that wait: an LDS store before it would wait for the copies)
#pragma unroll
      for (int i = 0; i < TPW; i++)
        if (lane == 0 && wave + i * NW < a.T) s_tab[wave + i * NW] = tb[i];
      __syncthreads();
      selrow = *reinterpret_cast<const uint4*>(s_tab);
    }
  }
  DecExpert ex;
  if (kTabAll) {
    // the expert's tokens, ascending, straight from its table row: no grouping needed
    const uint32_t wd = (lane & 15) < 4 ? selrow.x : (lane & 15) < 8 ? selrow.y : (lane & 15) < 12 ? selrow.z : selrow.w;
    const int sb = lane < a.T ? (int)((wd >> (8 * (lane & 3))) & 0xFFu) : 0;
    const uint64_t m = __ballot(sb > 0);
    if (wave == 0 && sb > 0) L.srows[__popcll(m & ((1ull << lane) - 1ull))] = lane * a.k + sb - 1;
    ex.e = aidx;
    ex.seg0 = 0;
    ex.row0 = 0;
    ex.cnt = __popcll(m);
    __syncthreads();   // token list and activation rows visible
    if (ex.cnt == 0) return;
    if (slot < 0) {
      if (tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
      return;
    }
    ex.tiles = reinterpret_cast<const uint4*>(a.base + a.stride * (size_t)slot);
    ex.scales = nullptr;
  } else if (kLgt) {
    // the table rows (lane e: row e), then the workgroup's expert by ballots
    const DecSelRow srow{dec_lgt_rows<NW>(a, lgt, wave, lane, s_keys, s_tab), lgt.slot};
    if (!dec_sel_pick(a, srow, aidx, lane, ex, slot, stok)) return;
    if (slot < 0) {
      if (tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
      return;
    }
    ex.tiles = reinterpret_cast<const uint4*>(a.base + a.stride * (size_t)slot);
    ex.scales = nullptr;
    dec_dma_x<NW>(a, L, wave, lane);   // the token rows straight into LDS, then the weights
  } else if (!dec_setup<SRC, ALL, NT>(a, L, pub, pre, fixed_expert, aidx, cs == 0, slot, ex, pp != 0)) {
    return;
  }
  if (!ALL) {
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, nbytes, 0x00020000);
#pragma unroll
    for (int j = 0; j < kDecRing; j++) issue(rsrc, j, W[j]);
  }
  if (kLgt && !ALL) {
    // as above: vmcnt(16) is the completion of the activation copies; the barrier
    // publishes every wave's rows and wave 0's token list
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x4F70);
    if (wave == 0 && stok.pos >= 0) L.srows[stok.pos] = stok.flat;
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t rsrc_none = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, 0, 0x00020000);

  const int npass = (ex.cnt + kDecTok - 1) / kDecTok;
  for (int p = 0; p < npass; p++) {
    const int nrow = ex.cnt - p * kDecTok < kDecTok ? ex.cnt - p * kDecTok : kDecTok;
    if (tid < kDecTok) {
      const int r = p * kDecTok + tid;
      L.pf[tid] = r < ex.cnt ? (is_sel(SRC) ? L.srows[r] : SRC == kSrcIds ? L.rows[ex.row0 + r]
                                                                          : a.sorted_flat[ex.seg0 + ex.row0 + r])
                             : -1;
    }
    auto next_issue = [&](int sn, WSlot2& w) {
      // past this pass's last position the ring runs on into the next pass; after the
      // last pass it loads nothing
      const int wrap = sn >= ST;
      issue(wrap ? (p + 1 < npass ? rsrc : rsrc_none) : rsrc, wrap ? sn - ST : sn, w);
    };
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // ---- phase 1: gate/up over H, activations staged chunk by chunk
    for (int c = 0; c < nK; c++) {
      const int kc0 = c * kDecKC;
      const int kcw = a.H - kc0 < kDecKC ? a.H - kc0 : kDecKC;
      const int ngc = kcw / kGroup;
      __syncthreads();   // previous chunk consumed; pass row list visible
      if (!is_sel(SRC)) {   // table routing: every token row is already staged
        const int cw8 = kcw / 8;
        for (int q = tid; q < nrow * cw8; q += NT) {
          const int r = q / cw8, c8 = q - r * cw8;
          *reinterpret_cast<uint4*>(L.xs + r * kDecXS + c8 * 8) = *reinterpret_cast<const uint4*>(
              a.x + (size_t)(L.pf[r] / a.k) * a.H + kc0 + c8 * 8);
        }
      }
      __syncthreads();
      const int myrow = (lane & 15) < nrow ? (is_sel(SRC) ? L.pf[lane & 15] / a.k : (lane & 15)) : kDecTok;
      const uint16_t* xrow = L.xs + myrow * kDecXS + 8 * (lane >> 4);
#pragma unroll
      for (int i0 = 0; i0 < kDecKG; i0 += kDecRing) {
#pragma unroll
        for (int j = 0; j < kDecRing; j++) {
          const int gl = i0 + j;
          if (gl < ngc) {
            bf16x8 act[4];
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) act[s4] = *reinterpret_cast<const bf16x8*>(xrow + gl * kGroup + 32 * s4);
            // seed: -136 * (sum of the group's activations of the token), by MFMA
            f32x4 sd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) sd = mfma16(n136, act[s4], sd);
            f32x4 c0 = sd, c1 = sd;
            c0 = mfma16(dequant_word(W[j].w[0].x), act[0], c0);
            c1 = mfma16(dequant_word(W[j].w[1].x), act[0], c1);
            c0 = mfma16(dequant_word(W[j].w[0].y), act[1], c0);
            c1 = mfma16(dequant_word(W[j].w[1].y), act[1], c1);
            c0 = mfma16(dequant_word(W[j].w[0].z), act[2], c0);
            c1 = mfma16(dequant_word(W[j].w[1].z), act[2], c1);
            c0 = mfma16(dequant_word(W[j].w[0].w), act[3], c0);
            c1 = mfma16(dequant_word(W[j].w[1].w), act[3], c1);
            scale_accum(acc0, c0, W[j].s[0]);
            scale_accum(acc1, c1, W[j].s[1]);
          }
          next_issue(c * kDecKG + i0 + j + kDecRing, W[j]);
        }
      }
    }
    // ---- h of the slice into LDS (bf16, [token][RS + skew]), and its correction seeds
    __syncthreads();   // all waves done with the staged activations
    constexpr int kHS = RS + 8;
    uint16_t* hs = L.xs;
    {
      // padding token slots computed from the zero row: their h is 0
      uint2 pk;
      pk.x = pack_bf16x2(silu_mul(acc0[0], acc1[0]), silu_mul(acc0[1], acc1[1]));
      pk.y = pack_bf16x2(silu_mul(acc0[2], acc1[2]), silu_mul(acc0[3], acc1[3]));
      *reinterpret_cast<uint2*>(hs + (lane & 15) * kHS + wave * 16 + 4 * (lane >> 4)) = pk;
    }
    __syncthreads();
    // ---- phase 2: the slice's down column groups over all H rows of this wave's share;
    // the seeds -136 * (sum of h over each group) come from the same MFMA against -136
    bf16x8 acth[NCG][4];
    f32x4 sdh[NCG];
#pragma unroll
    for (int g = 0; g < NCG; g++) {
      sdh[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        acth[g][s4] = *reinterpret_cast<const bf16x8*>(hs + (lane & 15) * kHS + g * kGroup + 32 * s4 + 8 * (lane >> 4));
        sdh[g] = mfma16(n136, acth[g][s4], sdh[g]);
      }
    }
    const int f = L.pf[lane & 15];
    float* prow = a.part + ((size_t)cs * a.T * a.k + (f >= 0 ? f : 0)) * a.H + 4 * (lane >> 4);
    const int lim = rbd_base + per_w < nrbd ? rbd_base + per_w : nrbd;
#pragma unroll
    for (int i0 = 0; i0 < S2; i0 += kDecRing) {
#pragma unroll
      for (int j = 0; j < kDecRing; j++) {
        const int pi = i0 + j;
        if (pi < npos2) {
          // NW = 8: tiles of row blocks r0, r0 + 1, one group each; NW = 16: the two
          // groups of row block r0, summed into one output
          const bf16x8* o1 = acth[NCG - 1];
          f32x4 c0 = sdh[0], c1 = sdh[NCG - 1];
          c0 = mfma16(dequant_word(W[j].w[0].x), acth[0][0], c0);
          c1 = mfma16(dequant_word(W[j].w[1].x), o1[0], c1);
          c0 = mfma16(dequant_word(W[j].w[0].y), acth[0][1], c0);
          c1 = mfma16(dequant_word(W[j].w[1].y), o1[1], c1);
          c0 = mfma16(dequant_word(W[j].w[0].z), acth[0][2], c0);
          c1 = mfma16(dequant_word(W[j].w[1].z), o1[2], c1);
          c0 = mfma16(dequant_word(W[j].w[0].w), acth[0][3], c0);
          c1 = mfma16(dequant_word(W[j].w[1].w), o1[3], c1);
          f32x4 oa = {0.f, 0.f, 0.f, 0.f}, ob = oa;
          scale_accum(oa, c0, W[j].s[0]);
          scale_accum(NCG == 1 ? ob : oa, c1, W[j].s[1]);
          if (f >= 0) {
            if (NCG == 1) {
              const int r0 = rbd_base + 2 * pi, r1 = r0 + 1;
              if (r0 < lim) *reinterpret_cast<float4*>(prow + r0 * 16) = make_float4(oa[0], oa[1], oa[2], oa[3]);
              if (r1 < lim) *reinterpret_cast<float4*>(prow + r1 * 16) = make_float4(ob[0], ob[1], ob[2], ob[3]);
            } else {
              const int r0 = rbd_base + pi;
              if (r0 < lim) *reinterpret_cast<float4*>(prow + r0 * 16) = make_float4(oa[0], oa[1], oa[2], oa[3]);
            }
          }
        }
        next_issue(S1 + i0 + j + kDecRing, W[j]);
      }
    }
    __syncthreads();   // pass row list and LDS free for the next pass
  }
  // exactness counter: the rows this expert ran (once per row: slice 0 counts them)
  if (a.rows_ctr && cs == 0 && tid == 0) atomicAdd(a.rows_ctr + ex.e, ex.cnt);
  span_end(a.span);
}

// ------------------------------------------------------------------------------------
// Narrow fused gate/up + down for very few routed rows (T <= 16, H <= kDecKC), when the
// 8-wave fused kernel would leave most compute units idle (one token routes to k experts:
// k x I/128 workgroups). A compute unit streams about 30 GB/s however deep its queue of
// loads, so the expert is cut four times finer: workgroup = (expert, slice c of 32 rows of
// I), 16 waves. Phase 1: wave w computes tile row w % 4 (gate and up of the slice's two
// row blocks) over quarter w / 4 of the input groups; the quarters are added in LDS and
// h of the slice (32 columns) goes to LDS as bf16. Phase 2: the slice is one 32-input
// step (word c % 4 of group c / 4) of every down tile; wave w applies it to row blocks
// kNarD w .. kNarD w + kNarD - 1 and writes fp32 partial outputs part[c][f][H]. Every
// weight load of the workgroup is issued at once, right after the expert is known.
// ------------------------------------------------------------------------------------
constexpr int kNarRows = 32;                          // rows of I per workgroup
constexpr int kNarQ = 4;                              // input quarters of the gate/up phase
constexpr int kNarG = kDecKG / kNarQ;                 // groups per quarter (H <= kDecKC)
constexpr int kNarD = kDecKC / kTileRows / 16;        // down row blocks per wave (H <= kDecKC)

template <int SRC>
__global__ __launch_bounds__(1024) void decode_narrow_kernel(MoeArgs a, DecPublish pub) {
  constexpr int NW = 16, NT = 64 * NW;
  __shared__ DecLDS L;
  __shared__ f32x4 red[NW][64];
  __shared__ __attribute__((aligned(16))) uint16_t hs[kDecTok][kNarRows + 8];
  const int tid = threadIdx.x, lane = (int)lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  span_begin(a.span);
  const int nslice = a.I / kNarRows;
  // Workgroups are handed to the 8 XCDs in turn (workgroup b to XCD b % 8), and the four
  // slices 4j .. 4j + 3 of an expert read the same down tiles (a word each). The logical
  // order is therefore transposed so that each XCD takes a contiguous run of workgroups:
  // the slices of one expert share that XCD's L2.
  // With logit routing the grid's last workgroup is also the publisher (after its slice's
  // weight loads); otherwise a workgroup of its own follows the slices.
  constexpr bool kPubFold = SRC == kSrcLgt;
  const bool pub_wg = kPubFold && blockIdx.x == gridDim.x - 1;
  const int nwk = gridDim.x - (is_sel(SRC) && !kPubFold ? 1 : 0);
  int b = blockIdx.x;
  if (b < nwk && (nwk & 7) == 0) b = (b & 7) * (nwk >> 3) + (b >> 3);
  const int aidx = b / nslice, cs = b % nslice;
  const int G = a.H / kGroup, GQ = (G + kNarQ - 1) / kNarQ;
  const int nrbd = a.H / kTileRows, Gd = a.I / kGroup;
  const int tr = wave & 3, q = wave >> 2;               // tile row (row block 2c + tr / 2, gate / up), quarter
  const uint32_t tbase = (uint32_t)((cs * 2 + (tr >> 1)) * 2 + (tr & 1)) * G;
  const uint32_t dbase = 2u * (uint32_t)(a.I / kTileRows) * (uint32_t)G;
  const uint32_t sc_base = (uint32_t)(n_tiles(a.H, a.I) * kTileBytes);
  const int nbytes = (int)packed_bytes(a.H, a.I);
  const uint32_t lo_t = (uint32_t)lane * 16u, lo_s = (uint32_t)(lane >> 4) * 8u;
  const uint32_t lo_w = lo_t + 4u * (uint32_t)(cs & 3);  // the slice's word of a down tile
  const bf16x8 n136 = neg136_operand();

  for (int i = tid; i < kDecXS / 8; i += NT)
    *reinterpret_cast<uint4*>(L.xs + kDecTok * kDecXS + i * 8) = make_uint4(0u, 0u, 0u, 0u);
  constexpr bool kLgt = SRC == kSrcLgt;
  __shared__ __attribute__((aligned(16))) uint8_t s_tab[64 * kDecTok];   // logit routing: table rows
  __shared__ __attribute__((aligned(16))) uint32_t s_keys[kLgt ? NW * 64 : 4];   // logit routing: keys
  __shared__ DecPubLDS<kPubFold ? NT : 64> s_pub;                               // the folded publisher
  DecPre pre;
  DecLgt<NW> lgt;
  if (kLgt) lgt = dec_lgt_load<NW>(a, pub, wave, lane);
  else pre = dec_preload<SRC, NT>(a, pub);
  if (is_sel(SRC) && !kPubFold && blockIdx.x == gridDim.x - 1) {
    dec_publish<SRC, NT>(a, L, pub);
    return;
  }
  if (SRC == kSrcSel) dec_prestage_x<NT>(a, L);
  DecExpert ex;
  DecSelTok stok;
  if (kLgt) {
    // the table rows (lane e: row e), then the workgroup's expert by ballots
    const DecSelRow srow{dec_lgt_rows<NW>(a, lgt, wave, lane, s_keys, s_tab), lgt.slot};
    int slot = 0;
    const bool has = dec_sel_pick(a, srow, aidx, lane, ex, slot, stok);
    if (!has || slot < 0) {
      if (has && tid == 0 && !a.skip_absent) atomicOr(a.debug, 1u);   // routed expert without a slot
      if constexpr (kPubFold) {
        if (pub_wg) dec_publish_lgt<NW, NT>(a, lgt, wave, lane, pub, s_pub);
      }
      return;
    }
    ex.tiles = reinterpret_cast<const uint4*>(a.base + a.stride * (size_t)slot);
    ex.scales = nullptr;
    dec_dma_x<NW>(a, L, wave, lane);   // the token rows straight into LDS, then the weights
    __builtin_amdgcn_sched_barrier(0);
  } else if (!dec_setup<SRC, false, NT>(a, L, pub, pre, -1, aidx, cs == 0, 0, ex)) {
    return;
  }

  // every weight load at once (positions past the data load through a zero-length resource)
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, nbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rnone = __builtin_amdgcn_make_buffer_rsrc((void*)ex.tiles, (short)0, 0, 0x00020000);
  uint4 w1[kNarG];
  uint2 s1[kNarG];
  uint32_t w2[kNarD];
  uint2 s2[kNarD];
#pragma unroll
  for (int i = 0; i < kNarG; i++) {
    const int g = q * GQ + i;
    const bool on = i < GQ && g < G;
    const uint32_t t = tbase + (uint32_t)(on ? g : 0);
    w1[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(on ? rsrc : rnone, lo_t, (int)(t * kTileBytes), weight_cpol(SRC)));
    s1[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(on ? rsrc : rnone, lo_s, (int)(sc_base + t * kScaleBytes), weight_cpol(SRC)));
  }
#pragma unroll
  for (int i = 0; i < kNarD; i++) {
    const int r = wave * kNarD + i;
    const bool on = r < nrbd;
    const uint32_t t = dbase + (uint32_t)(on ? r : 0) * Gd + (uint32_t)(cs >> 2);
    // (default cache policy: the four slices of a word group read these lines)
    w2[i] = __builtin_amdgcn_raw_buffer_load_b32(on ? rsrc : rnone, lo_w, (int)(t * kTileBytes), 0);
    s2[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(on ? rsrc : rnone, lo_s, (int)(sc_base + t * kScaleBytes), 0));
  }
  if (kLgt) {
    // the activation copies are older than the 24 weight loads: vmcnt(24) is their
    // completion; the barrier below publishes the rows and wave 0's token list
    static_assert(2 * kNarG + 2 * kNarD == 24, "the wait counts 24 weight loads");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x4F78);
    if (wave == 0 && stok.pos >= 0) L.srows[stok.pos] = stok.flat;
    if constexpr (kPubFold) {
      if (pub_wg) dec_publish_lgt<NW, NT>(a, lgt, wave, lane, pub, s_pub);   // while the weights land
    }
  }

  // the expert's rows (at most T <= kDecTok: one pass)
  const int nrow = ex.cnt;
  if (tid < kDecTok)
    L.pf[tid] = tid < nrow ? (is_sel(SRC) ? L.srows[tid] : SRC == kSrcIds ? L.rows[tid] : a.sorted_flat[ex.seg0 + tid])
                           : -1;
  __syncthreads();
  if (!is_sel(SRC)) {   // table routing: every token row is already staged
    const int cw8 = a.H / 8;
    for (int i = tid; i < nrow * cw8; i += NT) {
      const int r = i / cw8, c8 = i - r * cw8;
      *reinterpret_cast<uint4*>(L.xs + r * kDecXS + c8 * 8) =
          *reinterpret_cast<const uint4*>(a.x + (size_t)(L.pf[r] / a.k) * a.H + c8 * 8);
    }
    __syncthreads();
  }
  // ---- phase 1: this wave's tile row over its quarter of the input groups
  const int myrow = (lane & 15) < nrow ? (is_sel(SRC) ? L.pf[lane & 15] / a.k : (lane & 15)) : kDecTok;
  const uint16_t* xrow = L.xs + myrow * kDecXS + 8 * (lane >> 4);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kNarG; i++) {
    const int g = q * GQ + i;
    if (i < GQ && g < G) {
      bf16x8 act[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) act[s4] = *reinterpret_cast<const bf16x8*>(xrow + g * kGroup + 32 * s4);
      f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) c = mfma16(n136, act[s4], c);   // seed: -136 * group sum
      c = mfma16(dequant_word(w1[i].x), act[0], c);
      c = mfma16(dequant_word(w1[i].y), act[1], c);
      c = mfma16(dequant_word(w1[i].z), act[2], c);
      c = mfma16(dequant_word(w1[i].w), act[3], c);
      scale_accum(acc, c, s1[i]);
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave < 2) {   // row block 2c + wave: gate tile row 2 wave, up tile row 2 wave + 1
    f32x4 g = red[2 * wave][lane], u = red[2 * wave + 1][lane];
#pragma unroll
    for (int qq = 1; qq < kNarQ; qq++) {
      g += red[2 * wave + 4 * qq][lane];
      u += red[2 * wave + 1 + 4 * qq][lane];
    }
    uint2 pk;
    pk.x = pack_bf16x2(silu_mul(g[0], u[0]), silu_mul(g[1], u[1]));
    pk.y = pack_bf16x2(silu_mul(g[2], u[2]), silu_mul(g[3], u[3]));
    *reinterpret_cast<uint2*>(&hs[lane & 15][wave * 16 + 4 * (lane >> 4)]) = pk;
  }
  __syncthreads();
  // ---- phase 2: the slice's 32 inputs of this wave's down row blocks
  const bf16x8 acth = *reinterpret_cast<const bf16x8*>(&hs[lane & 15][8 * (lane >> 4)]);
  const f32x4 sdh = mfma16(n136, acth, f32x4{0.f, 0.f, 0.f, 0.f});
  const int f = L.pf[lane & 15];
  float* prow = a.part + ((size_t)cs * a.T * a.k + (f >= 0 ? f : 0)) * a.H + 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < kNarD; i++) {
    const int r = wave * kNarD + i;
    if (r < nrbd) {
      const f32x4 c = mfma16(dequant_word(w2[i]), acth, sdh);
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      scale_accum(o, c, s2[i]);
      if (f >= 0) *reinterpret_cast<float4*>(prow + r * 16) = make_float4(o[0], o[1], o[2], o[3]);
    }
  }
  if (a.rows_ctr && cs == 0 && tid == 0) atomicAdd(a.rows_ctr + ex.e, ex.cnt);   // exactness counter
  span_end(a.span);
}

// ------------------------------------------------------------------------------------
// combine: y[t, rows] = bf16(sum_j y_perm[t k + j, rows]) in slot order
// ------------------------------------------------------------------------------------
// Workgroup = (token, 256 M float4 columns: grid x = token, y = column block); thread = M float4 columns 256 apart (every
// load instruction of the workgroup covers 4 KiB in a row), with 16 / M slots of them in
// flight at a time. M = 4 for many tokens (fewer, longer workgroups), 1 for few.
// A grouping that misses rows (an id outside [0, E) counted nowhere: offsets[E] < T k)
// leaves their outputs unwritten; the combine's first thread records it.
__device__ __forceinline__ void check_grouped_rows(const MoeArgs& a) {
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0 && a.offsets[a.E] != a.T * a.k)
    atomicOr(a.debug, (uint32_t)EXMOE_FLAG_ROWS_UNGROUPED);
}

template <int M>
__global__ __launch_bounds__(256) void combine_kernel(MoeArgs a) {
  span_begin(a.span);
  check_grouped_rows(a);
  const int t = blockIdx.x;
  const int nv = a.H >> 2;                               // float4 per row
  const int q0 = blockIdx.y * (256 * M) + (int)threadIdx.x;
  const float* src = a.y_perm + (size_t)t * a.k * a.H;
  constexpr int JB = 16 / M;
  float4 s[M];
#pragma unroll
  for (int m = 0; m < M; m++) s[m] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < a.k; j0 += JB) {
    float4 v[JB][M];
#pragma unroll
    for (int u = 0; u < JB; u++)
#pragma unroll
      for (int m = 0; m < M; m++) {
        const int q = q0 + 256 * m;
        v[u][m] = (j0 + u < a.k && q < nv) ? *reinterpret_cast<const float4*>(src + (size_t)(j0 + u) * a.H + 4 * q)
                                           : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < JB; u++)
      if (j0 + u < a.k) {   // added in slot order
#pragma unroll
        for (int m = 0; m < M; m++) {
          s[m].x += v[u][m].x; s[m].y += v[u][m].y; s[m].z += v[u][m].z; s[m].w += v[u][m].w;
        }
      }
  }
#pragma unroll
  for (int m = 0; m < M; m++) {
    const int q = q0 + 256 * m;
    if (q < nv) {
      uint2 pk;
      pk.x = pack_bf16x2(s[m].x, s[m].y);
      pk.y = pack_bf16x2(s[m].z, s[m].w);
      *reinterpret_cast<uint2*>(a.y + (size_t)t * a.H + 4 * q) = pk;
    }
  }
  span_end(a.span);
}

// combine of the fused decode: y[t] = bf16(sum over slots j in order of w[t k + j] times
// (sum over I-slices q in order of part[q][t k + j])). Workgroup = (token, CC columns);
// thread = (4 columns, slot j) adds the slices of its slot, then the slots are added
// through LDS. CC shrinks for few tokens so that the partial sums (slices x slots x H
// floats per token) are read by enough workgroups. Every load of a thread (QB slices at a
// time, at clamped positions, and the routing weight) is issued unconditionally before the
// first add, so that they share one memory latency; a position past the last slice adds
// +0.0, which leaves the sum's bits unchanged (the sum starts at +0.0 and never becomes
// -0.0).
template <int CC, int QB>
__global__ __launch_bounds__(256) void combine_parts_kernel(MoeArgs a) {
  constexpr int kCombCols = CC;
  __shared__ float4 red[kMaxK][kCombCols / 4];
  span_begin(a.span);
  const int t = blockIdx.y;
  const int col0 = blockIdx.x * kCombCols;
  const size_t slice = (size_t)a.T * a.k * a.H;
  const int nq = a.nparts;
  for (int i = threadIdx.x; i < a.k * (kCombCols / 4); i += blockDim.x) {
    const int j = i / (kCombCols / 4), cq = i % (kCombCols / 4);
    const int c = col0 + 4 * cq;
    const bool cin = c < a.H;
    const float* src = a.part + ((size_t)t * a.k + j) * a.H + (cin ? c : 0);
    const float wt = a.w[t * a.k + j];
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < nq; q0 += QB) {
      float4 v[QB];
#pragma unroll
      for (int u = 0; u < QB; u++) {
        const int q = q0 + u < nq ? q0 + u : nq - 1;
        v[u] = *reinterpret_cast<const float4*>(src + (size_t)q * slice);
      }
#pragma unroll
      for (int u = 0; u < QB; u++) {
        const bool on = q0 + u < nq;
        s.x += on ? v[u].x : 0.f;
        s.y += on ? v[u].y : 0.f;
        s.z += on ? v[u].z : 0.f;
        s.w += on ? v[u].w : 0.f;
      }
    }
    s.x *= wt; s.y *= wt; s.z *= wt; s.w *= wt;
    red[j][cq] = cin ? s : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __syncthreads();
  if (threadIdx.x < kCombCols / 4) {
    const int cq = threadIdx.x, c = col0 + 4 * cq;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; j++) {
      const float4 v = red[j][cq];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (c < a.H) {
      uint2 pk;
      pk.x = pack_bf16x2(s.x, s.y);
      pk.y = pack_bf16x2(s.z, s.w);
      *reinterpret_cast<uint2*>(a.y + (size_t)t * a.H + c) = pk;
    }
  }
  check_grouped_rows(a);   // (after the sums: its load does not delay them)
  span_end(a.span);
}

// The same sums for many tokens (the pass-parallel decode): workgroup = (token, 1024
// columns), thread = one float4 column over every slot and slice, 16 loads in flight; the
// slot and slice order and the roundings (slot sum, times the weight, then added) are the
// ones of combine_parts_kernel.
template <int NP>
__global__ __launch_bounds__(256) void combine_parts_tok_kernel(MoeArgs a) {
#pragma clang fp contract(off)   // the slot sum times the weight is rounded before it is added
  span_begin(a.span);
  check_grouped_rows(a);
  const int t = blockIdx.x;
  const int q4 = blockIdx.y * 256 + (int)threadIdx.x;   // float4 column
  if (q4 < (a.H >> 2)) {
    const size_t slice = (size_t)a.T * a.k * a.H;
    const float* src = a.part + (size_t)t * a.k * a.H + 4 * q4;
    constexpr int JB = 16 / NP;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < a.k; j0 += JB) {
      float4 v[JB][NP];
#pragma unroll
      for (int u = 0; u < JB; u++)
#pragma unroll
        for (int q = 0; q < NP; q++)
          v[u][q] = j0 + u < a.k ? *reinterpret_cast<const float4*>(src + (size_t)(j0 + u) * a.H + q * slice)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < JB; u++)
        if (j0 + u < a.k) {
          float4 sj = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int q = 0; q < NP; q++) {
            sj.x += v[u][q].x; sj.y += v[u][q].y; sj.z += v[u][q].z; sj.w += v[u][q].w;
          }
          const float wt = a.w[t * a.k + j0 + u];
          acc.x += sj.x * wt; acc.y += sj.y * wt;
          acc.z += sj.z * wt; acc.w += sj.w * wt;
        }
    }
    uint2 pk;
    pk.x = pack_bf16x2(acc.x, acc.y);
    pk.y = pack_bf16x2(acc.z, acc.w);
    *reinterpret_cast<uint2*>(a.y + (size_t)t * a.H + 4 * q4) = pk;
  }
  span_end(a.span);
}

// ------------------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------------------
// Smallest reduction split that gives the launch enough workgroups to cover the chip.
static int pick_ks(int wgs_at_ks1) {
  int ks = 1;
  while (ks < 4 && wgs_at_ks1 * ks < 320) ks *= 2;
  return ks;
}

template <bool GATEUP, int SRC>
static void launch_expert(ProfScope& prof, const MoeArgs& a, const DecPublish& pub, int fixed_expert, int ny,
                          hipStream_t s) {
  // workgroups per expert at KS = 1: gate/up 8 row blocks of I each; down 16 row blocks of H
  const int per1 = GATEUP ? a.I / (kTileRows * kDecWaves) : (a.H / kTileRows + 2 * kDecWaves - 1) / (2 * kDecWaves);
  const dim3 block(kDecThreads);
  const int extra = GATEUP && SRC == kSrcSel ? 1 : 0;   // the publisher workgroup
  MoeArgs as = a;
  as.span = prof.span();
  if (fixed_expert < 0 && (long long)a.T * a.k >= 2LL * a.E) {
    // most experts active: one row of workgroups per expert (no active-expert list)
    EXMOE_LAUNCH(prof, (decode_expert_kernel<GATEUP, SRC, 1, true>), dim3(a.E * per1 + extra), block, 0, s, as, pub,
                 fixed_expert, per1);
    return;
  }
  const int ks = pick_ks(ny * per1);
  const int nchunk = per1 * ks;
  const dim3 grid(ny * nchunk + extra);
  if (ks == 1)
    EXMOE_LAUNCH(prof, (decode_expert_kernel<GATEUP, SRC, 1, false>), grid, block, 0, s, as, pub, fixed_expert, nchunk);
  else if (ks == 2)
    EXMOE_LAUNCH(prof, (decode_expert_kernel<GATEUP, SRC, 2, false>), grid, block, 0, s, as, pub, fixed_expert, nchunk);
  else
    EXMOE_LAUNCH(prof, (decode_expert_kernel<GATEUP, SRC, 4, false>), grid, block, 0, s, as, pub, fixed_expert, nchunk);
}

// Workgroups per slice of I of a fused launch: every expert (T <= 16 and most experts
// active), one per active expert (T <= 16), or one per 16-row pass of an active expert
// (more tokens: at most T k / 16 + min(E, T k) passes).
static long long fused_units(int T, int E, int k) {
  const long long tk = (long long)T * k;
  const long long ny = E < tk ? E : tk;
  if (T > kDecTok) return (tk + kDecTok - 1) / kDecTok + ny;
  return tk >= 2LL * E ? E : ny;
}

int decode_fused_waves(int T, int H, int I, int E, int k) {
  const long long tk = (long long)T * k;
  const long long units = fused_units(T, E, k);
  // most experts active (or many passes) and one 16-wave workgroup per compute unit or
  // more: 16 waves
  if ((tk >= 2LL * E || T > kDecTok) && I % (2 * kGroup) == 0 && I / (2 * kGroup) <= 8 &&
      units * (I / (2 * kGroup)) >= 256)
    return 16;
  if (I / kGroup <= 16 && units * (I / kGroup) >= 256) return 8;
  // a few routed rows: the narrow kernel (32-row slices; reported as 2 waves' worth of rows)
  if (T <= kDecTok && H <= kDecKC && tk < 2LL * E) return kNarRows / kTileRows;
  return 0;
}

// One fused launch: grid (pass-parallel units, every expert, or the active ones) x slices,
// plus the publisher of a table-routed launch.
template <int SRC>
static void launch_fused(ProfScope& prof, const MoeArgs& as, const DecPublish& P, int fixed_expert, int ny, int units,
                         bool pp, bool all, hipStream_t s) {
  const int nw = as.I / (kTileRows * as.nparts);   // the workspace layout chose the width
  const int extra = is_sel(SRC) ? 1 : 0;           // the publisher workgroup
  const dim3 grid((pp ? units : all ? as.E : ny) * as.nparts + extra);
  if (nw == kNarRows / kTileRows) {
    // with logit routing the last slice's workgroup also publishes
    EXMOE_LAUNCH(prof, decode_narrow_kernel<SRC>, dim3(ny * as.nparts + (SRC == kSrcLgt ? 0 : extra)), dim3(1024), 0, s,
                 as, P);
    return;
  }
  {
    if (all) {
      if (nw == 16) EXMOE_LAUNCH(prof, (decode_fused_kernel<SRC, true, 16>), grid, dim3(1024), 0, s, as, P, fixed_expert, 0);
      else EXMOE_LAUNCH(prof, (decode_fused_kernel<SRC, true, 8>), grid, dim3(512), 0, s, as, P, fixed_expert, 0);
      return;
    }
  }
  if (nw == 16) EXMOE_LAUNCH(prof, (decode_fused_kernel<SRC, false, 16>), grid, dim3(1024), 0, s, as, P, fixed_expert, pp);
  else EXMOE_LAUNCH(prof, (decode_fused_kernel<SRC, false, 8>), grid, dim3(512), 0, s, as, P, fixed_expert, pp);
}

static hipError_t launch_decode_experts(const MoeArgs& a, const DecPublish* pub, int fixed_expert, int ny,
                                        hipStream_t s) {
  if (a.nparts > 0 && fixed_expert < 0) {
    ProfScope prof("decode_fused", s);
    const bool pp = a.T > kDecTok && !(pub && (pub->sel || pub->logits));   // pass-parallel: one workgroup per 16-row pass
    const bool all = !pp && (long long)a.T * a.k >= 2LL * a.E;
    const int units = (int)fused_units(a.T, a.E, a.k);
    MoeArgs as = a;
    as.span = prof.span();
    if (!pub) launch_fused<kSrcGiven>(prof, as, DecPublish{}, fixed_expert, ny, units, pp, all, s);
    else if (pub->logits) launch_fused<kSrcLgt>(prof, as, *pub, fixed_expert, ny, units, pp, all, s);
    else if (pub->sel) launch_fused<kSrcSel>(prof, as, *pub, fixed_expert, ny, units, pp, all, s);
    else launch_fused<kSrcIds>(prof, as, *pub, fixed_expert, ny, units, pp, all, s);
    return hipGetLastError();
  }
  {
    ProfScope prof("decode_gateup", s);
    if (!pub)
      launch_expert<true, kSrcGiven>(prof, a, DecPublish{}, fixed_expert, ny, s);
    else if (pub->sel)
      launch_expert<true, kSrcSel>(prof, a, *pub, fixed_expert, ny, s);
    else
      launch_expert<true, kSrcIds>(prof, a, *pub, fixed_expert, ny, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope prof("decode_down", s);
    launch_expert<false, kSrcGiven>(prof, a, DecPublish{}, fixed_expert, ny, s);
  }
  return hipGetLastError();
}

hipError_t launch_moe_decode_experts(const MoeArgs& a, hipStream_t s) {
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  return launch_decode_experts(a, nullptr, -1, ny, s);
}

hipError_t launch_moe_decode(const MoeArgs& a, hipStream_t s) {
  hipError_t e = launch_moe_decode_experts(a, s);
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

bool decode_table_routing_ok(int T, int H, int E, int k) {
  return T >= 1 && T <= kDecTok && H <= kDecKC && E <= 256 && E * kSelStride <= kDecMaxRows * 4 &&
         T * k <= kDecMaxRows;
}

hipError_t launch_moe_decode_routed(const MoeArgs& a, const uint8_t* sel, int32_t* offsets, int32_t* sorted_flat,
                                    int32_t* flat_to_sorted, hipStream_t s) {
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  const DecPublish pub{sel, offsets, sorted_flat, flat_to_sorted};
  hipError_t e = launch_decode_experts(a, &pub, -1, ny, s);
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

bool decode_logit_routing_ok(int T, int H, int I, int E, int k) {
  return decode_table_routing_ok(T, H, E, k) && E <= 64 && decode_fused_waves(T, H, I, E, k) != 0;
}

hipError_t launch_moe_decode_logit_routed(const MoeArgs& a, const uint16_t* logits, int renormalize, int32_t* ids,
                                          float* w, int32_t* offsets, int32_t* sorted_flat, int32_t* flat_to_sorted,
                                          hipStream_t s) {
  if (a.nparts <= 0 || a.E > 64) return hipErrorInvalidValue;
  const int ny = a.E < a.T * a.k ? a.E : a.T * a.k;
  const DecPublish pub{nullptr, offsets, sorted_flat, flat_to_sorted, logits, ids, w, renormalize};
  hipError_t e = launch_decode_experts(a, &pub, -1, ny, s);
  if (e != hipSuccess) return e;
  return launch_combine(a, s);
}

hipError_t launch_moe_expert_range(const MoeArgs& a, int expert, int rows, hipStream_t s) {
  (void)rows;
  return launch_decode_experts(a, nullptr, expert, 1, s);
}

hipError_t launch_combine(const MoeArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  ProfScope prof("combine", s);
  MoeArgs as = a;
  as.span = prof.span();
  if (a.nparts > 0) {
    const dim3 tok_grid(a.T, (a.H / 4 + 255) / 256);
    if (a.T > kDecTok && a.nparts == 4)
      EXMOE_LAUNCH(prof, combine_parts_tok_kernel<4>, tok_grid, dim3(256), 0, s, as);
    else if (a.T > kDecTok && a.nparts == 8)
      EXMOE_LAUNCH(prof, combine_parts_tok_kernel<8>, tok_grid, dim3(256), 0, s, as);
    else {
      // widest column block that still gives 128 workgroups; threads: k slots x CC / 4
      int cc = 128;
      while (cc > 16 && (long long)a.T * ((a.H + cc - 1) / cc) < 128) cc /= 2;
      const int nth = a.k * (cc / 4) < 256 ? (a.k * (cc / 4) + 63) / 64 * 64 : 256;
      const dim3 grid((a.H + cc - 1) / cc, a.T);
      // slices in flight per thread: the slice count rounded up to 4, 8, 16 or 32
      const int qb = a.nparts <= 4 ? 4 : a.nparts <= 8 ? 8 : a.nparts <= 16 ? 16 : 32;
#define EXMOE_COMB(CC)                                                                            \
  do {                                                                                            \
    if (qb == 4) EXMOE_LAUNCH(prof, (combine_parts_kernel<CC, 4>), grid, dim3(nth), 0, s, as);    \
    else if (qb == 8) EXMOE_LAUNCH(prof, (combine_parts_kernel<CC, 8>), grid, dim3(nth), 0, s, as); \
    else if (qb == 16) EXMOE_LAUNCH(prof, (combine_parts_kernel<CC, 16>), grid, dim3(nth), 0, s, as); \
    else EXMOE_LAUNCH(prof, (combine_parts_kernel<CC, 32>), grid, dim3(nth), 0, s, as);           \
  } while (0)
      if (cc == 128) EXMOE_COMB(128);
      else if (cc == 64) EXMOE_COMB(64);
      else if (cc == 32) EXMOE_COMB(32);
      else EXMOE_COMB(16);
#undef EXMOE_COMB
    }
    return hipGetLastError();
  }
  const int nv = a.H / 4;
  if (a.T >= 512)
    EXMOE_LAUNCH(prof, combine_kernel<4>, dim3(a.T, (nv + 1023) / 1024), dim3(256), 0, s, as);
  else
    EXMOE_LAUNCH(prof, combine_kernel<1>, dim3(a.T, (nv + 255) / 256), dim3(256), 0, s, as);
  return hipGetLastError();
}

}  // namespace exmoe
