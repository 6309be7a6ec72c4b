/*
 * exmoe.h -- C ABI of libexmoe, a fused grouped W4A16 mixture-of-experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes follows "Every Expert Counts: ExactMoE for Memory-Efficient
 * W4A16 Inference": routed experts carry symmetric group-128 int4 weights packed once
 * into a kernel-native form (abstract; Fig. 1 caption), the BF16 router and its top-k
 * procedure are unchanged (abstract; Fig. 1), tokens are grouped by selected expert and
 * every selected expert runs (Fig. 1), and packed experts live in a pinned host pool
 * behind a configurable GPU slot cache (abstract; Fig. 1; Tab. 1).
 *
 * Conventions shared by every entry point
 *  - Return value: EXMOE_OK (0) or a negative exmoe_status. exmoe_last_error() returns a
 *    thread-local message for the last failing call on the calling thread. Nothing throws
 *    or aborts across this boundary.
 *  - Validation happens before anything is enqueued: on an error no work is launched and
 *    outputs are untouched. Faults of already-enqueued device work surface as
 *    EXMOE_ERR_HIP on a later synchronizing call.
 *  - Ownership: the caller owns every buffer passed in. The library owns only slot-cache
 *    handles (pinned pool, device slots, copy streams, events).
 *  - Device calls are asynchronous on the caller's stream unless stated otherwise.
 *  - bf16 values travel as raw uint16_t bit patterns; indices are int32; routing weights
 *    are fp32. Device buffers must be 16-byte aligned.
 *  - Shapes: H % 128 == 0, I % 128 == 0, group size 128, 1 <= k <= E <= 256. T == 0 is a
 *    valid no-op.
 *  - Integer outputs are deterministic; y is bitwise reproducible for fixed inputs and
 *    path (no floating-point atomics).
 */
#ifndef EXMOE_H
#define EXMOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EXMOE_ABI_VERSION 1

typedef uint16_t exmoe_bf16;

typedef enum exmoe_status {
  EXMOE_OK = 0,
  EXMOE_ERR_INVALID_ARGUMENT = -1, /* bad pointer, shape, alignment or flag */
  EXMOE_ERR_UNSUPPORTED = -2,      /* valid request this build does not implement */
  EXMOE_ERR_WORKSPACE = -3,        /* workspace missing or smaller than the query says */
  EXMOE_ERR_HIP = -4,              /* a HIP runtime call failed */
  EXMOE_ERR_OUT_OF_MEMORY = -5,    /* a library-owned allocation failed */
  EXMOE_ERR_CACHE = -6             /* slot-cache misuse: too many active experts, bad layer */
} exmoe_status;

const char* exmoe_status_string(int status);
/* Thread-local message of the calling thread's last failing call ("" if none). */
const char* exmoe_last_error(void);
int exmoe_abi_version(void);

/* ------------------------------------------------------------------------------------
 * Offline quantize + pack (host memory, synchronous, runs on the CPU).
 * Abstract and Fig. 1: routed expert projections are quantized (symmetric, group 128,
 * four bits) and packed once into the form the expert kernels consume.
 *
 * Quantization per output row n and input group g (inputs 128g..128g+127):
 *   s = bf16_round_nearest_even(fp32(absmax / 7)), 0 for an all-zero group;
 *   q = clamp(round_half_even(w / s), -8, 7) with the quotient formed in fp64; q = 0 if s = 0.
 * Packed blob of one expert (exmoe_packed_expert_bytes(H, I) = 3HI/2 + 3HI/64 bytes):
 *   [n_tiles x 1024 B int4 tiles][n_tiles x 32 B bf16 scales],
 *   n_tiles = 2(I/16)(H/128) + (H/16)(I/128).
 *   Tile order: for row block b < I/16: gate tiles g < H/128, then up tiles g < H/128;
 *   then for row block b < H/16: down tiles g < I/128. A tile holds rows 16b..16b+15 and
 *   inputs 128g..128g+127 of its matrix. Byte 16l+4s of a tile (lane l < 64, word s < 4)
 *   starts a little-endian word with row 16b + l%16, inputs 128g + 32s + 8(l/16) + j
 *   (j < 8) as nibbles u = q + 8; input j sits at bit 4(j/2) for even j and 16 + 4(j/2)
 *   for odd j. The 16 scales of tile t (its rows in order) start at byte
 *   1024 n_tiles + 32 t.
 * ---------------------------------------------------------------------------------- */
size_t exmoe_packed_expert_bytes(int H, int I);

/* w_gate, w_up: fp32 [I, H] row-major; w_down: fp32 [H, I]; group_size must be 128.
 * packed: host buffer of packed_bytes >= exmoe_packed_expert_bytes(H, I).
 * Non-finite weights are EXMOE_ERR_INVALID_ARGUMENT. */
int exmoe_quantize_pack(const float* w_gate, const float* w_up, const float* w_down, int H, int I,
                        int group_size, void* packed, size_t packed_bytes);

/* Inverse of the packing (not of the rounding): codes q int8 ([I,H], [I,H], [H,I]) and
 * scales bf16 ([I,H/128], [I,H/128], [H,I/128]). Any output pointer may be NULL. */
int exmoe_unpack_expert(const void* packed, size_t packed_bytes, int H, int I, int8_t* q_gate,
                        int8_t* q_up, int8_t* q_down, exmoe_bf16* s_gate, exmoe_bf16* s_up,
                        exmoe_bf16* s_down);

/* Dense bf16 expert of the comparator layer (abstract; Tab. 1 and Tab. 4: the same model
 * with its experts left in bf16). A bf16 blob (exmoe_bf16_expert_bytes(H, I) = 6HI bytes)
 * holds 1 KiB tiles of 16 rows x 32 inputs, no scales:
 *   tile order: for row block b < I/16: gate tiles c < H/32, then up tiles c < H/32; then
 *   for row block b < H/16: down tiles c < I/32. Bytes 16l..16l+15 of a tile (lane l < 64)
 *   hold row 16b + l%16, inputs 32c + 8(l/16) + j (j < 8) as little-endian bf16.
 * exmoe_bf16_pack only reorders: w_gate, w_up bf16 [I, H], w_down bf16 [H, I] row-major
 * (host) into out (host, out_bytes >= exmoe_bf16_expert_bytes). A bank of such blobs runs
 * with the flag EXMOE_WEIGHTS_BF16 on exmoe_moe_forward, exmoe_moe_layer and
 * exmoe_moe_forward_cached. 0 for H or I not a positive multiple of 128. */
size_t exmoe_bf16_expert_bytes(int H, int I);
int exmoe_bf16_pack(const exmoe_bf16* w_gate, const exmoe_bf16* w_up, const exmoe_bf16* w_down, int H, int I,
                    void* out, size_t out_bytes);

/* ------------------------------------------------------------------------------------
 * Routing (device, asynchronous). Abstract and Fig. 1: the original BF16 router selects
 * the experts and the top-k procedure is unchanged.
 *   logits[t,e] = bf16_round_nearest_even(sum_h x[t,h] * w_router[e,h] + bias[e]), the
 *     exact bf16 products summed in fp64 (order-insensitive in practice), rounded once;
 *   topk_ids[t, 0..k-1]: experts ordered by (logit descending, expert id ascending),
 *     -0 and +0 equal;
 *   topk_weights[t,j]: renormalize != 0 -> softmax over the k selected logits;
 *     renormalize == 0 -> full-softmax probability of the selected expert (fp32 expf).
 * x bf16 [T,H]; w_router bf16 [E,H]; logit_bias fp32 [E] or NULL; logits bf16 [T,E] or
 * NULL (not written); topk_ids int32 [T,k]; topk_weights fp32 [T,k]. All device memory.
 * ---------------------------------------------------------------------------------- */
int exmoe_route_topk(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias,
                     int T, int H, int E, int k, int renormalize, exmoe_bf16* logits,
                     int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Top-k and weights from given bf16 logits [T,E] (same rules as exmoe_route_topk). */
int exmoe_topk_from_logits(const exmoe_bf16* logits, int T, int E, int k, int renormalize,
                           int32_t* topk_ids, float* topk_weights, hipStream_t stream);

/* Weights for externally chosen experts (a routing trace): topk_ids int32 [T,k] holds k
 * distinct ids per token; weights follow the renormalize rule above over those ids. */
int exmoe_route_weights(const exmoe_bf16* logits, const int32_t* topk_ids, int T, int E, int k,
                        int renormalize, float* topk_weights, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Grouping (device, asynchronous). Fig. 1: tokens are grouped by selected expert.
 * Flat index f = t*k + j. expert_offsets int32 [E+1] is the exclusive prefix sum of the
 * per-expert counts (offsets[E] = T*k, unpadded); sorted_flat int32 [T*k] lists, expert by
 * expert ascending and within an expert in ascending f, every f routed there;
 * flat_to_sorted int32 [T*k] is its inverse. Ids outside [0, E) are a caller error: such a
 * row is counted nowhere and gets flat_to_sorted = -1, so expert_offsets[E] falls short of
 * T*k (the expert layer flags that grouping: EXMOE_FLAG_ROWS_UNGROUPED); sorted_flat is
 * then written only up to expert_offsets[E], and no memory is touched out of range. The workspace may be NULL when exmoe_group_workspace_bytes returns 0; it is
 * (T*k + 1023) / 1024 * E * 4 bytes of device scratch (4-byte aligned) above 4096 routed
 * rows, where the grouping runs in chunks over several workgroups; its contents need no
 * initialization and are not kept.
 * ---------------------------------------------------------------------------------- */
size_t exmoe_group_workspace_bytes(int T, int k, int E);
int exmoe_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                       int32_t* sorted_flat, int32_t* flat_to_sorted, void* workspace,
                       size_t ws_bytes, hipStream_t stream);

/* Reactive-cache step (synchronizes `stream`): copies offsets to the host and lists the
 * experts with a non-empty segment in ascending order. ids_host must hold E ints. */
int exmoe_active_experts(const int32_t* expert_offsets, int E, int32_t* ids_host, int* n_host,
                         hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Expert layer (device, asynchronous). Abstract and Fig. 1: every selected expert runs,
 * grouped, with int4 weights dequantized on the fly (no 16-bit copy of an expert).
 * For every routed pair (t, j) with e = topk_ids[t,j]:
 *   g = W_gate x_t, u = W_up x_t, a = silu(g) * u (stored as bf16), o = W_down a,
 * with W = q*s from expert e's blob, products of bf16 operands accumulated in fp32; then
 *   y[t] = bf16(sum_{j=0..k-1} w[t,j] * o_{t,j}) summed in that slot order.
 * The expert MLP form (SwiGLU) is not on the pages; it is this layer's stated workload.
 *
 * bank: expert e's blob is at base + stride * slot(e), slot(e) = expert_to_slot[e] when
 * expert_to_slot (device int32 [E]) is given, else e. Every routed expert must map to a
 * valid slot (a -1 slot for a routed expert is a caller error; the kernels then skip it
 * and count it in the debug word). x bf16 [T,H]; y bf16 [T,H]; routing buffers as
 * produced by exmoe_route_topk / exmoe_group_tokens for the same T, k, E.
 * ---------------------------------------------------------------------------------- */
typedef struct exmoe_expert_bank {
  const void* base;
  size_t stride;                 /* bytes between slots, >= packed (or bf16) expert bytes, % 16 == 0 */
  const int32_t* expert_to_slot; /* device int32 [E] or NULL for identity */
} exmoe_expert_bank;

enum {
  EXMOE_PATH_AUTO = 0,       /* choose by rows per active expert */
  EXMOE_PATH_DECODE = 1,     /* split-K GEMV-style kernels, 16-token MFMA tiles */
  EXMOE_PATH_PREFILL = 2,    /* grouped GEMM kernels, 64- or 128-token tiles */
  EXMOE_PATH_SEQUENTIAL = 3, /* per-expert launches in ascending expert order (reference
                                W4 path; synchronizes once to read the offsets) */
  EXMOE_PATH_MASK = 0xff,
  EXMOE_WEIGHTS_BF16 = 0x100, /* flag: the bank holds dense bf16 experts (exmoe_bf16_pack);
                                paths AUTO, DECODE and PREFILL */
  EXMOE_FLAG_DEBUG_COUNTERS = 0x200 /* flag: every expert kernel adds the routed rows it ran
                                to its expert's counter in the workspace header (read with
                                exmoe_workspace_rows); the exactness check of the abstract's
                                claim that every selected expert runs and none is pruned or
                                substituted (Fig. 1: all routed rows, grouped by expert) */
};

size_t exmoe_moe_workspace_bytes(int T, int H, int I, int E, int k, int flags);

int exmoe_moe_forward(const exmoe_bf16* x, const int32_t* topk_ids, const float* topk_weights,
                      const int32_t* expert_offsets, const int32_t* sorted_flat,
                      const int32_t* flat_to_sorted, const exmoe_expert_bank* bank, int T, int H,
                      int I, int E, int k, int flags, exmoe_bf16* y, void* workspace,
                      size_t ws_bytes, hipStream_t stream);

/* Whole layer in one call: route (exmoe_route_topk), group (exmoe_group_tokens) and the
 * expert layer (exmoe_moe_forward), with the routing results written to caller buffers
 * (logits is required here: the selection reads it back). Same arguments and rules as
 * those three calls.
 * Workspace contract (this call only): its first 4096 bytes hold arrival counters that
 * persist between calls. They must be zero before the first call on a workspace (allocate
 * it zero-filled or clear it once); every call leaves them zero, and no other call of the
 * library writes them, so one workspace may serve calls of any shape and path. Calls
 * that share a workspace must not overlap in time (same stream, or synchronized). */
size_t exmoe_moe_layer_workspace_bytes(int T, int H, int I, int E, int k, int flags);

/* Conditions the expert kernels recorded in a workspace of exmoe_moe_forward,
 * exmoe_moe_layer or exmoe_moe_forward_cached, since it was cleared (abstract: no selected
 * expert may be skipped; these report a call where one was). Bit 0
 * (EXMOE_FLAG_EXPERT_WITHOUT_SLOT): a routed expert had no slot (expert_to_slot = -1), or
 * was missing from the active list of a cached forward of several waves; its rows were
 * skipped and the output of the tokens routed to it is undefined. Bit 1
 * (EXMOE_FLAG_ROWS_UNGROUPED): the grouping did not cover every routed row
 * (expert_offsets[E] != T*k, e.g. an id outside [0, E) in exmoe_group_tokens); those
 * rows' outputs are undefined. Reads the word after the work already enqueued on `stream`
 * (host-synchronous: the stream is synchronized) into *flags_out, then clears it when
 * clear != 0. workspace: device, ws_bytes >= 4096. */
enum { EXMOE_FLAG_EXPERT_WITHOUT_SLOT = 1, EXMOE_FLAG_ROWS_UNGROUPED = 2 };
int exmoe_workspace_flags(void* workspace, size_t ws_bytes, int clear, uint32_t* flags_out, hipStream_t stream);

/* Exactness counters (abstract and Fig. 1: every selected expert runs on all of its routed
 * rows). With EXMOE_FLAG_DEBUG_COUNTERS in a call's flags, the kernel that finishes a
 * routed row (the down projection) adds it to its expert's int32 counter in the
 * workspace header; a call that ran every routed row exactly once adds
 * expert_offsets[e+1] - expert_offsets[e] to counter e. The counters accumulate over calls
 * until cleared; a zero-filled workspace starts them at zero. Copies counters 0..E-1 to
 * rows_out (host, E ints) after the work enqueued on `stream` (synchronizes), then zeroes
 * them when clear != 0. workspace: device, ws_bytes >= 4096; 1 <= E <= 256. */
int exmoe_workspace_rows(void* workspace, size_t ws_bytes, int E, int clear, int32_t* rows_out, hipStream_t stream);
int exmoe_moe_layer(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias,
                    const exmoe_expert_bank* bank, int T, int H, int I, int E, int k,
                    int renormalize, int flags, exmoe_bf16* logits, int32_t* topk_ids,
                    float* topk_weights, int32_t* expert_offsets, int32_t* sorted_flat,
                    int32_t* flat_to_sorted, exmoe_bf16* y, void* workspace, size_t ws_bytes,
                    hipStream_t stream);

/* exmoe_moe_layer for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same call without a
 * workspace argument. It allocates nothing: its workspace is a fixed 64 MiB array in the
 * library's device code (one copy per GPU, held until the process ends), which serves
 * every call whose exmoe_moe_layer_workspace_bytes(T, H, I, E, k, flags) is at most 64 MiB
 * (e.g. OLMoE-shaped layers up to about 700 tokens); a larger call fails with
 * EXMOE_ERR_UNSUPPORTED before anything is enqueued. EXMOE_FLAG_DEBUG_COUNTERS is
 * EXMOE_ERR_UNSUPPORTED (no workspace to read the counters from). Results are those of
 * exmoe_moe_layer, bit for bit. The caller still passes every input and output buffer.
 * All calls on one GPU share that GPU's array: calls that overlap in time on one GPU
 * (different streams, or host threads) race and must not be issued. */
int exmoe_moe_layer_noalloc(const exmoe_bf16* x, const exmoe_bf16* w_router, const float* logit_bias,
                            const exmoe_expert_bank* bank, int T, int H, int I, int E, int k,
                            int renormalize, int flags, exmoe_bf16* logits, int32_t* topk_ids,
                            float* topk_weights, int32_t* expert_offsets, int32_t* sorted_flat,
                            int32_t* flat_to_sorted, exmoe_bf16* y, hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Slot cache (host policy + asynchronous host-to-device copies). Abstract, Fig. 1, Fig. 2
 * and Tab. 1: a pinned host pool keeps every packed expert; a GPU cache of a configurable
 * number of slots per layer holds the ones in use; misses copy packed weights and scales.
 * Policy (the pages name none): least-recently-used per layer. A layer-step looks up its
 * distinct active experts in ascending id; a hit refreshes the expert's stamp; a miss
 * takes the lowest free slot, else evicts the resident expert with the oldest stamp that
 * is not in the current active set, and copies the blob on one of the cache's two copy
 * streams (successive misses alternate between them).
 * slots_per_layer == E is full residency: exmoe_slot_cache_preload copies everything and
 * lookups are bypassed (counters stay 0, stats.resident = 1).
 * ---------------------------------------------------------------------------------- */
typedef struct exmoe_slot_cache exmoe_slot_cache;

typedef struct exmoe_cache_stats {
  uint64_t lookups, hits, misses, evictions;
  uint64_t h2d_bytes, h2d_copies;
  uint64_t device_bytes;       /* device slot memory held */
  uint64_t pinned_host_bytes;  /* pinned pool held */
  int resident;                /* 1 when slots_per_layer == E */
} exmoe_cache_stats;

enum { EXMOE_CACHE_DRY_RUN = 1 }; /* policy and counters only: no allocation, no copies */

/* Allocates the pinned pool (layers*E*expert_stride bytes), the device slots
 * (layers*slots*expert_stride), two copy streams and the device expert->slot tables;
 * synchronous. expert_bytes is the packed size; the stride rounds it up to 256 B. */
int exmoe_slot_cache_create(int layers, int E, int slots_per_layer, size_t expert_bytes, int flags,
                            exmoe_slot_cache** out);
/* Host pointer of (layer, expert)'s pinned blob, for the caller to fill once (e.g. with
 * exmoe_quantize_pack). Not available in dry-run mode. */
int exmoe_slot_cache_host_slot(exmoe_slot_cache* cache, int layer, int expert, void** pinned_ptr);
/* Full residency only: copies every blob to its slot and waits. */
int exmoe_slot_cache_preload(exmoe_slot_cache* cache, hipStream_t stream);
/* One layer-step: looks up the active experts (host ids, any order, duplicates ignored),
 * enqueues the copies for the misses on the copy streams after everything enqueued on
 * compute_stream so far, uploads the layer's expert->slot table, and makes compute_stream
 * wait for them; bank_out then describes the layer's slots. More distinct active experts than slots -> EXMOE_ERR_CACHE, state kept.
 * In dry-run mode only the policy and counters run and bank_out is zeroed. */
int exmoe_slot_cache_acquire(exmoe_slot_cache* cache, int layer, const int32_t* active_ids_host,
                             int n_active, hipStream_t compute_stream, exmoe_expert_bank* bank_out);
/* The cache-sized waves (Fig. 1) of one exmoe_moe_forward_cached call on `layer`, as that
 * call's host side forms them: the distinct ids of active_ids_host (host, any order,
 * duplicates ignored) in wave order -- the experts already resident in the layer's slots
 * first, then the others, each part ascending -- into order_out (host, room for n_active
 * ints), their count into *n_distinct and the wave size into *wave_size (the waves are
 * consecutive runs of that many ids, the last one possibly shorter: slots_per_layer when
 * every id fits, else slots_per_layer / 2, or 1 with one slot). run == 0 only plans and
 * changes nothing. run != 0 then looks each wave up in turn, the policy and counters a
 * cached forward applies, and is allowed on a dry-run cache only (EXMOE_ERR_CACHE
 * otherwise: with device slots the cached forward itself runs the waves, with copies). */
int exmoe_slot_cache_waves(exmoe_slot_cache* cache, int layer, const int32_t* active_ids_host, int n_active,
                           int run, int32_t* order_out, int* n_distinct, int* wave_size);
/* Host copy of the layer's expert->slot table (-1 = not resident), int32 [E]. */
int exmoe_slot_cache_table(const exmoe_slot_cache* cache, int layer, int32_t* table_host);
int exmoe_slot_cache_stats(const exmoe_slot_cache* cache, exmoe_cache_stats* out);
int exmoe_slot_cache_reset_stats(exmoe_slot_cache* cache);
/* Waits for outstanding copies, frees everything. NULL is a no-op. */
int exmoe_slot_cache_destroy(exmoe_slot_cache* cache);

/* Expert layer through the slot cache in cache-sized waves (Fig. 1: waves of experts that
 * fit the cache). The distinct active experts (host list; it must hold every routed expert
 * of the call, e.g. from exmoe_active_experts) are ordered with the ones already resident in the layer's slots first, then
 * the others, each part in ascending id. A list that fits slots_per_layer is one wave; a
 * longer one is cut into waves of slots_per_layer / 2 (1 when there is one slot). Each
 * wave is acquired (one layer-step of the cache's policy and counters: misses copied on
 * the cache's copy streams, the compute stream waits for them), then the expert kernels
 * run for that wave's experts only. With half-size waves the copies of wave w+1 land in
 * slots that wave w does not read, so they wait only for wave w-1's kernels and overlap
 * wave w's. The copies of a layer's first waves wait only for the last kernels that read
 * that layer's slots (recorded by the previous cached forward of the layer; after an
 * exmoe_slot_cache_acquire of the layer, for all earlier work), so they overlap the
 * kernels of other layers still in flight. The combine runs once after the last wave, so y equals exmoe_moe_forward's on
 * a resident bank bit for bit. Arguments as exmoe_moe_forward, with the bank replaced by
 * (cache, layer); the cache must hold E experts per layer and not be a dry-run cache;
 * EXMOE_PATH_SEQUENTIAL -> EXMOE_ERR_UNSUPPORTED. The workspace size is
 * exmoe_moe_workspace_bytes (the per-wave expert->slot table lives there). A routed
 * expert missing from the list: in a one-wave call it is computed if it happens to be
 * resident, else flagged (exmoe_workspace_flags) and its rows are left unwritten; in a
 * call of several waves its rows are left unwritten and a check after the last wave
 * flags it (EXMOE_FLAG_EXPERT_WITHOUT_SLOT). The host returns once every wave is
 * enqueued, without waiting for the GPU (a per-wave table travels in the arguments of a
 * one-workgroup kernel). Calls on one cache must come from one host thread. */
int exmoe_moe_forward_cached(const exmoe_bf16* x, const int32_t* topk_ids, const float* topk_weights,
                             const int32_t* expert_offsets, const int32_t* sorted_flat,
                             const int32_t* flat_to_sorted, exmoe_slot_cache* cache, int layer,
                             const int32_t* active_ids_host, int n_active, int T, int H, int I, int E,
                             int k, int flags, exmoe_bf16* y, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* ------------------------------------------------------------------------------------
 * Per-kernel timing for benchmarks (not part of the layer's semantics). While enabled,
 * each kernel of the library is launched with a hipEvent pair that stamps that kernel's
 * own start and end on its launch stream (hipExtLaunchKernelGGL; skipped on a stream that
 * is being captured into a graph). exmoe_profile_read
 * synchronizes the recorded events and returns the accumulated milliseconds and launch
 * count of one kernel by name: "route_logits", "route_token", "route_sel", "topk",
 * "group", "decode_gateup", "decode_down", "decode_fused", "combine", "xsum",
 * "prefill_gateup", "prefill_down". Process-global. The events bracket the launch as the
 * stream processes it, so a launch that waits for the host is counted with that wait.
 * ---------------------------------------------------------------------------------- */
int exmoe_profile_enable(int on);
int exmoe_profile_reset(void);
int exmoe_profile_read(const char* kernel_name, double* total_ms, uint64_t* launches);

/* Launch span stamps (benchmark timing; not part of the layer's semantics). After
 * exmoe_span_enable(n) (n > 0; allocates 1 KiB of device memory per slot, n = 0 frees them),
 * each of the next n launches of the expert-layer kernels ("decode_gateup", "decode_down",
 * "decode_fused", "combine", "prefill_gateup", "prefill_down") takes one slot, also while
 * its stream is captured into a graph: its workgroups stamp the GPU's constant-rate clock
 * at their start (minimum) and after their last memory operation (maximum).
 * exmoe_span_read synchronizes the device and returns, for one kernel name, the summed
 * durations in microseconds and the number of slots that ran since the last
 * exmoe_span_clear (which resets the stamps and keeps the slots' assignment, so that a
 * captured graph can be replayed and measured again). Process-global; not thread-safe
 * against concurrent layer calls that take slots. */
int exmoe_span_enable(int max_launches);
int exmoe_span_clear(void);
int exmoe_span_read(const char* kernel_name, double* total_us, uint64_t* launches);

/* Plain device copy of `bytes` bytes (a multiple of 16; both pointers 16-byte aligned),
 * one pass of 16-byte loads and stores, asynchronous on `stream`. Not part of the layer:
 * it is the kernel of known HBM traffic (bytes read + bytes written) against which the
 * hardware traffic counters are calibrated. Kernel name in traces: exmoe::copy_kernel. */
int exmoe_device_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* EXMOE_H */
