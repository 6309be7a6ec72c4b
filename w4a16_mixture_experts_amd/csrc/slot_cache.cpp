// GPU expert slot cache backed by a pinned host pool (ExactMoE abstract; Fig. 1, Fig. 2,
// Tab. 1): every packed expert stays in pinned host memory; each layer has a fixed
// number of device slots; a miss copies the packed blob (int4 weights + bf16 scales, no
// 16-bit expansion) on the cache's own copy stream, and the compute stream waits on an
// event. Misses are split over two copy streams (two DMA queues move more than one over the
// host link). The eviction policy is least-recently-used per layer with deterministic
// tie-breaking (lowest free slot first; the victim is the oldest resident expert outside
// the current active set), so the counters are reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "common.h"
#include "exmoe.h"

using namespace exmoe;

struct exmoe_slot_cache {
  int layers = 0, E = 0, S = 0, flags = 0;
  bool resident = false, dry = false;
  size_t expert_bytes = 0, stride = 0;
  uint8_t* pinned = nullptr;
  uint8_t* dev = nullptr;
  int32_t* d_tables = nullptr;       // [layers, E]
  hipStream_t copy_stream = nullptr, copy_stream2 = nullptr;
  hipEvent_t ev_compute = nullptr, ev_copy = nullptr, ev_copy2 = nullptr;
  std::vector<int32_t> slot_of;      // [layers, E], -1 = absent
  std::vector<int32_t> owner;        // [layers, S], -1 = free
  std::vector<uint64_t> stamp;       // [layers, E]
  uint64_t clock = 0;
  exmoe_cache_stats st{};
  int device = 0;
  std::vector<hipEvent_t> wave_ev;   // compute-stream marks of a forward in waves (grown on demand)
  // [layers] compute-stream mark after the last kernels that read the layer's slots, valid
  // only while every reader of the layer came from the cached forward (created on demand)
  std::vector<hipEvent_t> layer_ev;
  std::vector<char> layer_ev_ok;
};

static void cache_free(exmoe_slot_cache* c) {
  if (!c) return;
  if (c->copy_stream) (void)hipStreamSynchronize(c->copy_stream);
  if (c->copy_stream2) (void)hipStreamSynchronize(c->copy_stream2);
  if (c->pinned) (void)hipHostFree(c->pinned);
  if (c->dev) (void)hipFree(c->dev);
  if (c->d_tables) (void)hipFree(c->d_tables);
  if (c->ev_compute) (void)hipEventDestroy(c->ev_compute);
  if (c->ev_copy) (void)hipEventDestroy(c->ev_copy);
  if (c->ev_copy2) (void)hipEventDestroy(c->ev_copy2);
  for (hipEvent_t ev : c->wave_ev) (void)hipEventDestroy(ev);
  for (hipEvent_t ev : c->layer_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (c->copy_stream) (void)hipStreamDestroy(c->copy_stream);
  if (c->copy_stream2) (void)hipStreamDestroy(c->copy_stream2);
  delete c;
}

namespace exmoe {
void slot_cache_shape(const exmoe_slot_cache* c, int* E, int* S, int* dry, size_t* expert_bytes) {
  *E = c->E;
  *S = c->S;
  *dry = c->dry ? 1 : 0;
  *expert_bytes = c->expert_bytes;
}

int slot_cache_layers(const exmoe_slot_cache* c) { return c->layers; }

hipError_t slot_cache_event(exmoe_slot_cache* c, int i, hipEvent_t* ev) {
  while ((int)c->wave_ev.size() <= i) {
    hipEvent_t e = nullptr;
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) return r;
    c->wave_ev.push_back(e);
  }
  *ev = c->wave_ev[i];
  return hipSuccess;
}

hipEvent_t slot_cache_layer_mark(exmoe_slot_cache* c, int layer) {
  if (layer < 0 || layer >= (int)c->layer_ev_ok.size() || !c->layer_ev_ok[layer]) return nullptr;
  return c->layer_ev[layer];
}

void slot_cache_forget_layer(exmoe_slot_cache* c, int layer) {
  if (layer >= 0 && layer < (int)c->layer_ev_ok.size()) c->layer_ev_ok[layer] = 0;
}

hipError_t slot_cache_mark_layer(exmoe_slot_cache* c, int layer, hipStream_t s) {
  if (c->resident) return hipSuccess;   // nothing is ever copied into its slots
  if (c->layer_ev.empty()) {
    c->layer_ev.assign(c->layers, nullptr);
    c->layer_ev_ok.assign(c->layers, 0);
  }
  if (!c->layer_ev[layer]) {
    hipError_t r = hipEventCreateWithFlags(&c->layer_ev[layer], hipEventDisableTiming);
    if (r != hipSuccess) { c->layer_ev[layer] = nullptr; return r; }
  }
  hipError_t r = hipEventRecord(c->layer_ev[layer], s);
  c->layer_ev_ok[layer] = r == hipSuccess;
  return r;
}

int slot_cache_plan_waves(const exmoe_slot_cache* c, int layer, std::vector<int32_t>& A) {
  std::sort(A.begin(), A.end());
  A.erase(std::unique(A.begin(), A.end()), A.end());
  const int32_t* slot_of = c->slot_of.data() + (size_t)layer * c->E;
  std::stable_partition(A.begin(), A.end(), [&](int32_t e) { return slot_of[e] >= 0; });
  return ((int)A.size() > c->S && c->S >= 2) ? c->S / 2 : c->S;
}

int slot_cache_acquire_ex(exmoe_slot_cache* c, int layer, const int32_t* active_ids_host, int n_active,
                          hipStream_t compute_stream, hipEvent_t after, const int32_t* protect_slots, int n_protect,
                          exmoe_expert_bank* bank_out) {
  if (!c || !bank_out) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache and bank_out must not be NULL");
  if (layer < 0 || layer >= c->layers) return set_error(EXMOE_ERR_CACHE, "layer %d out of range", layer);
  if (n_active < 0 || (n_active > 0 && !active_ids_host))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bad active list");
  std::vector<int> A(active_ids_host, active_ids_host + n_active);
  for (int e : A)
    if (e < 0 || e >= c->E) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "expert id %d out of range", e);
  std::sort(A.begin(), A.end());
  A.erase(std::unique(A.begin(), A.end()), A.end());
  if ((int)A.size() > c->S)
    return set_error(EXMOE_ERR_CACHE, "%zu active experts exceed %d slots", A.size(), c->S);
  int32_t* slot_of = c->slot_of.data() + (size_t)layer * c->E;
  int32_t* owner = c->owner.data() + (size_t)layer * c->S;
  uint64_t* stamp = c->stamp.data() + (size_t)layer * c->E;
  std::vector<std::pair<int, int>> copies;   // (expert, slot)
  if (!c->resident) {
    std::vector<char> in_A(c->E, 0);
    for (int e : A) in_A[e] = 1;
    for (int e : A) {
      c->st.lookups++;
      c->clock++;
      if (slot_of[e] >= 0) {
        c->st.hits++;
      } else {
        c->st.misses++;
        int s = -1;
        for (int i = 0; i < c->S; i++)
          if (owner[i] < 0) { s = i; break; }
        if (s < 0) {
          int victim = -1;
          for (int x = 0; x < c->E; x++)
            if (slot_of[x] >= 0 && !in_A[x] && (victim < 0 || stamp[x] < stamp[victim])) victim = x;
          s = slot_of[victim];      // exists: |A| <= S and every slot is owned
          slot_of[victim] = -1;
          c->st.evictions++;
        }
        slot_of[e] = s;
        owner[s] = e;
        copies.emplace_back(e, s);
        c->st.h2d_bytes += c->expert_bytes;
        c->st.h2d_copies++;
      }
      stamp[e] = c->clock;
    }
  }
  if (c->dry) {
    memset(bank_out, 0, sizeof(*bank_out));
    return EXMOE_OK;
  }
  uint8_t* layer_dev = c->dev + (size_t)layer * c->S * c->stride;
  if (!copies.empty()) {
    // The copy stream must not overwrite a slot that earlier work on the compute stream
    // may still read: it waits for `after` when no copy lands in a protected slot, else
    // for everything enqueued on the compute stream so far.
    bool early = after != nullptr;
    for (auto& es : copies)
      for (int i = 0; i < n_protect; i++) early = early && es.second != protect_slots[i];
    const bool two = copies.size() > 1;   // alternate the copies over both streams
    hipEvent_t wait_for = after;
    if (!early) {
      EXMOE_HIP(hipEventRecord(c->ev_compute, compute_stream));
      wait_for = c->ev_compute;
    }
    EXMOE_HIP(hipStreamWaitEvent(c->copy_stream, wait_for, 0));
    if (two) EXMOE_HIP(hipStreamWaitEvent(c->copy_stream2, wait_for, 0));
    for (size_t i = 0; i < copies.size(); i++)
      EXMOE_HIP(hipMemcpyAsync(layer_dev + (size_t)copies[i].second * c->stride,
                               c->pinned + ((size_t)layer * c->E + copies[i].first) * c->stride, c->expert_bytes,
                               hipMemcpyHostToDevice, (i & 1) ? c->copy_stream2 : c->copy_stream));
    // the table by value in kernel arguments: the host's copy may change right away
    EXMOE_HIP(table_upload(c->d_tables + (size_t)layer * c->E, slot_of, c->E, c->copy_stream));
    EXMOE_HIP(hipEventRecord(c->ev_copy, c->copy_stream));
    EXMOE_HIP(hipStreamWaitEvent(compute_stream, c->ev_copy, 0));
    if (two) {
      EXMOE_HIP(hipEventRecord(c->ev_copy2, c->copy_stream2));
      EXMOE_HIP(hipStreamWaitEvent(compute_stream, c->ev_copy2, 0));
    }
  }
  bank_out->base = layer_dev;
  bank_out->stride = c->stride;
  bank_out->expert_to_slot = c->d_tables + (size_t)layer * c->E;
  return EXMOE_OK;
}
}  // namespace exmoe

extern "C" {

int exmoe_slot_cache_create(int layers, int E, int slots_per_layer, size_t expert_bytes, int flags,
                            exmoe_slot_cache** out) {
  if (!out) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "out must not be NULL");
  *out = nullptr;
  if (layers < 1 || E < 1 || E > kMaxExperts)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "need layers >= 1 and 1 <= E <= 256");
  if (slots_per_layer < 1 || slots_per_layer > E)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "slots_per_layer must be in [1, E] (got %d)", slots_per_layer);
  if (expert_bytes == 0) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "expert_bytes must be > 0");
  if (flags & ~EXMOE_CACHE_DRY_RUN) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "unknown cache flags 0x%x", flags);
  auto* c = new (std::nothrow) exmoe_slot_cache();
  if (!c) return set_error(EXMOE_ERR_OUT_OF_MEMORY, "host allocation failed");
  c->layers = layers;
  c->E = E;
  c->S = slots_per_layer;
  c->flags = flags;
  c->dry = flags & EXMOE_CACHE_DRY_RUN;
  c->resident = slots_per_layer == E;
  c->expert_bytes = expert_bytes;
  c->stride = (expert_bytes + 255) & ~(size_t)255;
  c->slot_of.assign((size_t)layers * E, -1);
  c->owner.assign((size_t)layers * slots_per_layer, -1);
  c->stamp.assign((size_t)layers * E, 0);
  if (c->resident)
    for (int l = 0; l < layers; l++)
      for (int e = 0; e < E; e++) {
        c->slot_of[(size_t)l * E + e] = e;
        c->owner[(size_t)l * E + e] = e;
      }
  c->st.resident = c->resident ? 1 : 0;
  if (!c->dry) {
    hipError_t e;
    if ((e = hipGetDevice(&c->device)) != hipSuccess) { cache_free(c); return hip_error(e, "hipGetDevice"); }
    const size_t pool = (size_t)layers * E * c->stride;
    const size_t slots = (size_t)layers * slots_per_layer * c->stride;
    if ((e = hipHostMalloc((void**)&c->pinned, pool, hipHostMallocDefault)) != hipSuccess) {
      c->pinned = nullptr; cache_free(c); return hip_error(e, "hipHostMalloc(pinned pool)");
    }
    if ((e = hipMalloc((void**)&c->dev, slots)) != hipSuccess) { c->dev = nullptr; cache_free(c); return hip_error(e, "hipMalloc(slots)"); }
    if ((e = hipMalloc((void**)&c->d_tables, sizeof(int32_t) * layers * E)) != hipSuccess) {
      c->d_tables = nullptr; cache_free(c); return hip_error(e, "hipMalloc(tables)");
    }
    if ((e = hipStreamCreateWithFlags(&c->copy_stream, hipStreamNonBlocking)) != hipSuccess) {
      c->copy_stream = nullptr; cache_free(c); return hip_error(e, "hipStreamCreate");
    }
    if ((e = hipStreamCreateWithFlags(&c->copy_stream2, hipStreamNonBlocking)) != hipSuccess) {
      c->copy_stream2 = nullptr; cache_free(c); return hip_error(e, "hipStreamCreate");
    }
    if ((e = hipEventCreateWithFlags(&c->ev_compute, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_copy, hipEventDisableTiming)) != hipSuccess ||
        (e = hipEventCreateWithFlags(&c->ev_copy2, hipEventDisableTiming)) != hipSuccess) {
      cache_free(c); return hip_error(e, "hipEventCreate");
    }
    std::vector<int32_t> init((size_t)layers * E);
    for (size_t i = 0; i < init.size(); i++) init[i] = c->slot_of[i];
    if ((e = hipMemcpy(c->d_tables, init.data(), sizeof(int32_t) * init.size(), hipMemcpyHostToDevice)) != hipSuccess) {
      cache_free(c); return hip_error(e, "hipMemcpy(tables)");
    }
    c->st.device_bytes = slots + sizeof(int32_t) * layers * E;
    c->st.pinned_host_bytes = pool;
  }
  *out = c;
  return EXMOE_OK;
}

int exmoe_slot_cache_host_slot(exmoe_slot_cache* c, int layer, int expert, void** pinned_ptr) {
  if (!c || !pinned_ptr) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache and pinned_ptr must not be NULL");
  if (c->dry) return set_error(EXMOE_ERR_CACHE, "dry-run cache has no pool");
  if (layer < 0 || layer >= c->layers || expert < 0 || expert >= c->E)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "layer/expert out of range");
  *pinned_ptr = c->pinned + ((size_t)layer * c->E + expert) * c->stride;
  return EXMOE_OK;
}

int exmoe_slot_cache_preload(exmoe_slot_cache* c, hipStream_t stream) {
  if (!c) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache must not be NULL");
  if (!c->resident) return set_error(EXMOE_ERR_CACHE, "preload needs slots_per_layer == E");
  if (c->dry) return EXMOE_OK;
  // One copy: the pool and the slot array share the [layer, expert] order when resident.
  EXMOE_HIP(hipMemcpyAsync(c->dev, c->pinned, (size_t)c->layers * c->E * c->stride, hipMemcpyHostToDevice, stream));
  EXMOE_HIP(hipStreamSynchronize(stream));
  return EXMOE_OK;
}

int exmoe_slot_cache_acquire(exmoe_slot_cache* c, int layer, const int32_t* active_ids_host, int n_active,
                             hipStream_t compute_stream, exmoe_expert_bank* bank_out) {
  // the caller's kernels that will read these slots are unknown here: a later cached
  // forward of this layer waits for everything enqueued before its copies
  if (c) exmoe::slot_cache_forget_layer(c, layer);
  return exmoe::slot_cache_acquire_ex(c, layer, active_ids_host, n_active, compute_stream, nullptr, nullptr, 0,
                                      bank_out);
}

int exmoe_slot_cache_waves(exmoe_slot_cache* c, int layer, const int32_t* active_ids_host, int n_active, int run,
                          int32_t* order_out, int* n_distinct, int* wave_size) {
  if (!c || !order_out || !n_distinct || !wave_size)
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache and outputs must not be NULL");
  if (layer < 0 || layer >= c->layers) return set_error(EXMOE_ERR_CACHE, "layer %d out of range", layer);
  if (n_active < 0 || (n_active > 0 && !active_ids_host))
    return set_error(EXMOE_ERR_INVALID_ARGUMENT, "bad active list");
  if (run && !c->dry) return set_error(EXMOE_ERR_CACHE, "waves run only on a dry-run cache here");
  std::vector<int32_t> A(active_ids_host, active_ids_host + n_active);
  for (int e : A)
    if (e < 0 || e >= c->E) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "expert id %d out of range", e);
  const int W = exmoe::slot_cache_plan_waves(c, layer, A);
  if (run) {
    exmoe_expert_bank bank{};
    for (size_t w0 = 0; w0 < A.size(); w0 += W) {
      const int n = (int)std::min(A.size() - w0, (size_t)W);
      int st = exmoe::slot_cache_acquire_ex(c, layer, A.data() + w0, n, nullptr, nullptr, nullptr, 0, &bank);
      if (st) return st;
    }
  }
  std::copy(A.begin(), A.end(), order_out);
  *n_distinct = (int)A.size();
  *wave_size = W;
  return EXMOE_OK;
}

int exmoe_slot_cache_table(const exmoe_slot_cache* c, int layer, int32_t* table_host) {
  if (!c || !table_host) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache and table_host must not be NULL");
  if (layer < 0 || layer >= c->layers) return set_error(EXMOE_ERR_CACHE, "layer %d out of range", layer);
  memcpy(table_host, c->slot_of.data() + (size_t)layer * c->E, sizeof(int32_t) * c->E);
  return EXMOE_OK;
}

int exmoe_slot_cache_stats(const exmoe_slot_cache* c, exmoe_cache_stats* out) {
  if (!c || !out) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache and out must not be NULL");
  *out = c->st;
  return EXMOE_OK;
}

int exmoe_slot_cache_reset_stats(exmoe_slot_cache* c) {
  if (!c) return set_error(EXMOE_ERR_INVALID_ARGUMENT, "cache must not be NULL");
  c->st.lookups = c->st.hits = c->st.misses = c->st.evictions = 0;
  c->st.h2d_bytes = c->st.h2d_copies = 0;
  return EXMOE_OK;
}

int exmoe_slot_cache_destroy(exmoe_slot_cache* c) {
  cache_free(c);
  return EXMOE_OK;
}

}  // extern "C"
