// C ABI of the HiSparse swap-in path: validation, state memory, launches.
//
// Every swap call enqueues exactly two kernels on the caller's stream (the
// plan kernel, then the miss copy), allocates nothing and never synchronises
// the host; this keeps the pages' stream-ordering lesson (PR #20343 summary,
// "Review highlights": an overlap race fixed by a stream wait) structural --
// there is no side stream to wait for.
#include <cmath>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "internal.h"

using namespace hisparse;

#ifndef HISPARSE_HOST_ALLOC_FLAGS
#define HISPARSE_HOST_ALLOC_FLAGS hipHostMallocMapped
#endif

namespace {

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    int cur = -1;
    if (hipGetDevice(&cur) == hipSuccess && cur != dev && hipSetDevice(dev) == hipSuccess)
      prev = cur;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

using host::Derived;
using host::derive;

size_t align256(size_t x) { return (x + 255) & ~size_t{255}; }

int status_of(hipError_t e) {
  if (e == hipSuccess) return HISPARSE_OK;
  if (e == hipErrorOutOfMemory) return HISPARSE_E_NOMEM;
  return HISPARSE_E_HIP;
}

PlanArgs plan_args(const hisparse_state* st, int32_t layer, int32_t batch, int32_t steps,
                   const int32_t* req, const int32_t* seq, const int32_t* topk, int32_t* out,
                   int32_t* miss_count, int32_t* page_table, int32_t* num_pages,
                   const hisparse_miss_plan_t* plan) {
  PlanArgs a{};
  a.slot_key = st->slot_key;
  a.ts = st->ts;
  a.order = st->order;
  a.refbits = st->refbits;
  a.ctrl = st->ctrl;
  a.err = st->err;
  a.R = st->cfg.max_requests;
  a.H = st->cfg.hot_buffer_size;
  a.Hw = st->hw;
  a.K = st->cfg.top_k;
  a.S = steps;
  a.N = st->cfg.max_seq_len;
  a.P = st->cfg.page_size;
  a.nkeys = st->nkeys;
  a.rows = st->rows;
  a.ext = st->cfg.extra_rows;
  a.ext_base = st->rows - st->cfg.extra_rows;
  a.admission = st->cfg.admission;
  a.layer = layer;
  a.batch = batch;
  a.req = req;
  a.seq = seq;
  a.topk = topk;
  a.out_locs = out;
  a.miss_count = miss_count;
  a.page_table = page_table;
  a.num_pages = num_pages;
  a.copy_src = st->cp_src;
  a.copy_dst = st->cp_dst;
  a.ccap = st->cap;
  a.sort_words = 0;
  if (plan != nullptr) {
    a.miss_src = plan->miss_src;
    a.miss_dst = plan->miss_dst;
    a.victim = plan->victim;
    a.cap = plan->capacity;
  } else {
    a.miss_src = st->ws_src;
    a.miss_dst = st->ws_dst;
    a.victim = st->ws_victim;
    a.cap = st->cap;
  }
  return a;
}

// Accumulated profile of drained event triples.
struct ProfileSums {
  int64_t calls = 0, fused = 0;
  double plan_ms = 0, copy_ms = 0;
};

hipError_t drain_events(hisparse_state* st, ProfileSums* sums) {
  hipError_t err = hipSuccess;
  st->events.drain([&](hipEvent_t e0, hipEvent_t e1, hipEvent_t e2) {
    hipError_t e = hipEventSynchronize(e2);
    float t1 = 0, t2 = 0;
    if (e == hipSuccess) e = hipEventElapsedTime(&t1, e0, e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&t2, e1, e2);
    if (e == hipSuccess) {
      sums->calls += 1;
      sums->plan_ms += t1;
      sums->copy_ms += t2;
    } else {
      err = e;
    }
  });
  return err;
}

hipEvent_t take_event(hisparse_state* st) {
  auto& fl = st->events.free_list;
  if (fl.empty()) {
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDefault) != hipSuccess) return nullptr;
    return e;
  }
  hipEvent_t e = fl.back();
  fl.pop_back();
  return e;
}

struct ProfiledState : hisparse_state {
  ProfileSums sums;
};

void record(hisparse_state* st, hipStream_t s) {
  if (!st->profiling) return;
  hipEvent_t e = take_event(st);
  if (e == nullptr) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    st->events.free_list.push_back(e);
    return;
  }
  st->events.push(e);
}

// Turns on the ascending-host-row copy list when its LDS bitmap fits.
void enable_copy_sort(const hisparse_state* st, PlanArgs* a, size_t (*lds_bytes)(const PlanArgs&)) {
  if (st->nkeys > kMaxSortedKeys) return;
  a->sort_words = (st->nkeys + 31) / 32;
  if (lds_bytes(*a) > st->max_lds) a->sort_words = 0;
}

CopyArgs copy_args(const hisparse_state* st, int layer, int batch, const int32_t* miss_count,
                   const int32_t* src, const int32_t* dst, int cap) {
  CopyArgs c{};
  c.miss_count = miss_count;
  c.src = src;
  c.dst = dst;
  c.batch = batch;
  c.cap = cap;
  c.host = st->host_kv[layer];
  c.dev = st->dev_kv[layer];
  const int64_t unit = static_cast<int64_t>(st->cfg.item_size_bytes) * st->cfg.page_size;
  c.unit_bytes = unit;
  c.unit16 = static_cast<int32_t>(unit / 16);
  c.src_rows = static_cast<int64_t>(st->cfg.max_requests) * st->nkeys;
  c.dst_rows = static_cast<int64_t>(st->cfg.max_requests) * st->rows;
  c.err = st->err;
  return c;
}

bool plan_ok(const hisparse_miss_plan_t* plan, int32_t cap) {
  return plan == nullptr ||
         (plan->miss_src && plan->miss_dst && plan->victim && plan->capacity >= cap &&
          (plan->flags & ~HISPARSE_PLAN_DEFER_COPY) == 0);
}

bool defers_copy(const hisparse_miss_plan_t* plan) {
  return plan != nullptr && (plan->flags & HISPARSE_PLAN_DEFER_COPY) != 0;
}

int run_swap(hisparse_state* st, PlanArgs a, bool multistep, bool defer, hipStream_t s) {
  auto* ps = static_cast<ProfiledState*>(st);
  if (st->profiling && st->events.pending.size() >= 3 * 4096) (void)drain_events(st, &ps->sums);
  // every return path keeps this call's events only as one whole triple
  host::TripleGuard<hipEvent_t> guard(&st->events, st->profiling);
  record(st, s);
  if (!defer && a.batch >= kFuseMinRows && st->cfg.page_size == 1) {
    // token rows: the plan kernel copies its rows' misses itself
    a.fuse_copy = 1;
    a.host = st->host_kv[a.layer];
    a.dev = st->dev_kv[a.layer];
    a.unit_bytes = st->cfg.item_size_bytes;
    a.unit16 = st->cfg.item_size_bytes / 16;
  }
  hipError_t e;
  if (multistep)
    e = launch_clock_plan(a, s);
  else if (st->cfg.page_size > 1)
    e = launch_lru_page_plan(a, s);
  else
    e = launch_lru_token_plan(a, s);
  if (e != hipSuccess) return status_of(e);
  record(st, s);
  if (defer || a.fuse_copy) {  // replayed by the caller, or done by the plan kernel
    record(st, s);
    if (st->profiling && a.fuse_copy) ps->sums.fused += 1;
    return HISPARSE_OK;
  }
  const CopyArgs c = a.sort_words
                         ? copy_args(st, a.layer, a.batch, a.miss_count, a.copy_src, a.copy_dst,
                                     a.ccap)
                         : copy_args(st, a.layer, a.batch, a.miss_count, a.miss_src, a.miss_dst,
                                     a.cap);
  e = launch_miss_copy(c, s);
  if (e != hipSuccess) return status_of(e);
  record(st, s);
  return HISPARSE_OK;
}

}  // namespace

extern "C" {

int64_t hisparse_device_rows_per_request(const hisparse_config_t* cfg) {
  Derived d;
  const int rc = derive(cfg, &d);
  return rc == HISPARSE_OK ? d.rows : rc;
}

int hisparse_state_create(const hisparse_config_t* cfg, void* stream, hisparse_state_t* out) {
  if (out == nullptr) return HISPARSE_E_INVAL;
  *out = nullptr;
  Derived d;
  int rc = derive(cfg, &d);
  if (rc != HISPARSE_OK) return rc;
  if (cfg->host_kv == nullptr || cfg->dev_kv == nullptr) return HISPARSE_E_INVAL;
  const int L = cfg->num_layers, R = cfg->max_requests, H = cfg->hot_buffer_size;
  const bool lru = cfg->policy == HISPARSE_POLICY_LRU;
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return HISPARSE_E_HIP;
  int max_lds = 0, num_cus = 0;
  if (hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, device) !=
          hipSuccess ||
      hipDeviceGetAttribute(&num_cus, hipDeviceAttributeMultiprocessorCount, device) !=
          hipSuccess)
    return HISPARSE_E_HIP;

  auto* st = new (std::nothrow) ProfiledState();
  if (st == nullptr) return HISPARSE_E_NOMEM;
  st->cfg = *cfg;
  st->cfg.host_kv = nullptr;
  st->cfg.dev_kv = nullptr;
  st->device = device;
  st->rows = d.rows;
  st->scratch = d.scratch;
  st->nkeys = d.nkeys;
  st->hw = d.hw;
  st->cap = d.cap;
  st->max_lds = static_cast<size_t>(max_lds);
  st->num_cus = num_cus;
  for (int l = 0; l < L; ++l) {
    hipPointerAttribute_t attr{};
    const void* hp = cfg->host_kv[l];
    void* dp = cfg->dev_kv[l];
    if (hp == nullptr || dp == nullptr ||
        hipPointerGetAttributes(&attr, hp) != hipSuccess || attr.type != hipMemoryTypeHost ||
        attr.devicePointer == nullptr) {
      (void)hipGetLastError();
      delete st;
      return HISPARSE_E_INVAL;
    }
    st->host_kv.push_back(static_cast<const uint8_t*>(attr.devicePointer));
    hipPointerAttribute_t dattr{};
    if (hipPointerGetAttributes(&dattr, dp) != hipSuccess || dattr.type != hipMemoryTypeDevice ||
        dattr.device != device) {
      (void)hipGetLastError();
      delete st;
      return HISPARSE_E_INVAL;
    }
    st->dev_kv.push_back(static_cast<uint8_t*>(dp));
  }

  const size_t inst = static_cast<size_t>(L) * R;
  size_t off = 0;
  const size_t o_slot_key = off; off += align256(inst * H * sizeof(int32_t));
  const size_t o_ts = off;       off += lru ? align256(inst * H * sizeof(int32_t)) : 0;
  const size_t o_order = off;    off += lru ? align256(inst * H * sizeof(int16_t)) : 0;
  const size_t o_ref = off;      off += lru ? 0 : align256(inst * d.hw * sizeof(uint32_t));
  const size_t o_ctrl = off;     off += align256(inst * 2 * sizeof(int32_t));
  const size_t ws = align256(static_cast<size_t>(cfg->max_batch) * d.cap * sizeof(int32_t));
  const size_t o_src = off;      off += ws;
  const size_t o_dst = off;      off += ws;
  const size_t o_vic = off;      off += ws;
  const size_t o_cps = off;      off += ws;
  const size_t o_cpd = off;      off += ws;
  const size_t o_err = off;      off += 256;
  hipError_t e = hipMalloc(&st->arena, off);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    delete st;
    return status_of(e);
  }
  auto* base = static_cast<uint8_t*>(st->arena);
  st->slot_key = reinterpret_cast<int32_t*>(base + o_slot_key);
  st->ts = lru ? reinterpret_cast<int32_t*>(base + o_ts) : nullptr;
  st->order = lru ? reinterpret_cast<int16_t*>(base + o_order) : nullptr;
  st->refbits = lru ? nullptr : reinterpret_cast<uint32_t*>(base + o_ref);
  st->ctrl = reinterpret_cast<int32_t*>(base + o_ctrl);
  st->ws_src = reinterpret_cast<int32_t*>(base + o_src);
  st->ws_dst = reinterpret_cast<int32_t*>(base + o_dst);
  st->ws_victim = reinterpret_cast<int32_t*>(base + o_vic);
  st->cp_src = reinterpret_cast<int32_t*>(base + o_cps);
  st->cp_dst = reinterpret_cast<int32_t*>(base + o_cpd);
  st->err = reinterpret_cast<uint32_t*>(base + o_err);

  auto s = static_cast<hipStream_t>(stream);
  e = hipMemsetAsync(st->err, 0, sizeof(uint32_t), s);
  if (e == hipSuccess) {
    ResetArgs ra{nullptr, st->slot_key, st->ts, st->order, st->refbits, st->ctrl, st->err,
                 R, H, d.hw};
    e = launch_reset(ra, R, L, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(st->arena);
    delete st;
    return status_of(e);
  }
  *out = st;
  return HISPARSE_OK;
}

void hisparse_state_destroy(hisparse_state_t st) {
  if (st == nullptr) return;
  DeviceGuard g(st->device);
  for (hipEvent_t e : st->events.pending) (void)hipEventDestroy(e);
  for (hipEvent_t e : st->events.free_list) (void)hipEventDestroy(e);
  (void)hipFree(st->arena);
  delete static_cast<ProfiledState*>(st);
}

int32_t hisparse_plan_capacity(hisparse_state_t st) { return st ? st->cap : HISPARSE_E_INVAL; }

int hisparse_swap_in_selected(hisparse_state_t st, int32_t layer_id, int32_t batch,
                              const int32_t* req_pool_indices, const int32_t* seq_lens,
                              const int32_t* topk_indices, int32_t* out_locs,
                              int32_t* miss_count, int32_t* page_table, int32_t* num_pages,
                              const hisparse_miss_plan_t* plan, void* stream) {
  if (st == nullptr || st->cfg.policy != HISPARSE_POLICY_LRU) return HISPARSE_E_INVAL;
  if (layer_id < 0 || layer_id >= st->cfg.num_layers) return HISPARSE_E_INVAL;
  if (batch < 0 || batch > st->cfg.max_batch) return HISPARSE_E_INVAL;
  if (batch == 0) return HISPARSE_OK;
  if (!req_pool_indices || !seq_lens || !topk_indices || !out_locs || !miss_count)
    return HISPARSE_E_INVAL;
  const bool page = st->cfg.page_size > 1;
  if (page && (page_table == nullptr || num_pages == nullptr)) return HISPARSE_E_INVAL;
  if (!plan_ok(plan, st->cap)) return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  PlanArgs a = plan_args(st, layer_id, batch, 1, req_pool_indices, seq_lens, topk_indices,
                         out_locs, miss_count, page ? page_table : nullptr,
                         page ? num_pages : nullptr, plan);
  if (!page) {
    // key bitmaps when they fit (direct ranks, no hash); else an LDS hash
    a.hash_size = 0;
    enable_copy_sort(st, &a, lru_token_lds_bytes);
    if (a.sort_words == 0) {
      a.hash_size = hash_size_for(a.K, true);
      if (lru_token_lds_bytes(a) > st->max_lds) a.hash_size = hash_size_for(a.K, false);
    }
  }
  if ((page ? lru_page_lds_bytes(a) : lru_token_lds_bytes(a)) > st->max_lds)
    return HISPARSE_E_UNSUPPORTED;
  return run_swap(st, a, false, defers_copy(plan), static_cast<hipStream_t>(stream));
}

int hisparse_swap_in_spec_multistep(hisparse_state_t st, int32_t layer_id, int32_t batch,
                                    int32_t num_steps, const int32_t* req_pool_indices,
                                    const int32_t* seq_lens, const int32_t* topk_indices,
                                    int32_t* out_locs, int32_t* miss_count,
                                    const hisparse_miss_plan_t* plan, void* stream) {
  if (st == nullptr || st->cfg.policy != HISPARSE_POLICY_CLOCK) return HISPARSE_E_INVAL;
  if (layer_id < 0 || layer_id >= st->cfg.num_layers) return HISPARSE_E_INVAL;
  if (num_steps < HISPARSE_MIN_STEPS || num_steps > st->cfg.max_steps) return HISPARSE_E_INVAL;
  if (batch < 0 || batch > st->cfg.max_batch) return HISPARSE_E_INVAL;
  if (batch == 0) return HISPARSE_OK;
  if (!req_pool_indices || !seq_lens || !topk_indices || !out_locs || !miss_count)
    return HISPARSE_E_INVAL;
  if (!plan_ok(plan, st->cap)) return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  PlanArgs a = plan_args(st, layer_id, batch, num_steps, req_pool_indices, seq_lens,
                         topk_indices, out_locs, miss_count, nullptr, nullptr, plan);
  const int E = num_steps * a.K;
  a.hash_size = std::max(64, ((3 * E / 2 + 64) + 63) / 64 * 64);
  enable_copy_sort(st, &a, clock_lds_bytes);
  if (clock_lds_bytes(a) > st->max_lds) return HISPARSE_E_UNSUPPORTED;
  return run_swap(st, a, true, defers_copy(plan), static_cast<hipStream_t>(stream));
}

int hisparse_copy_planned(hisparse_state_t st, int32_t layer_id, int32_t batch,
                          const int32_t* miss_count, const hisparse_miss_plan_t* plan,
                          void* stream) {
  if (st == nullptr || plan == nullptr || miss_count == nullptr) return HISPARSE_E_INVAL;
  if (layer_id < 0 || layer_id >= st->cfg.num_layers || batch < 0) return HISPARSE_E_INVAL;
  if (!plan->miss_src || !plan->miss_dst || plan->capacity < 1) return HISPARSE_E_INVAL;
  if (batch > host::kMaxBatch) return HISPARSE_E_UNSUPPORTED;
  if (batch == 0) return HISPARSE_OK;
  DeviceGuard g(st->device);
  const CopyArgs c = copy_args(st, layer_id, batch, miss_count, plan->miss_src, plan->miss_dst,
                               plan->capacity);
  return status_of(launch_miss_copy(c, static_cast<hipStream_t>(stream)));
}

size_t hisparse_sparse_mla_workspace_bytes(hisparse_state_t st, int32_t batch, int32_t num_heads,
                                           int32_t n_locs) {
  if (st == nullptr || batch < 1 || num_heads < 1 || n_locs < 1) return 0;
  return mla_workspace_bytes(batch, num_heads, n_locs, st->num_cus);
}

int hisparse_sparse_mla_decode(hisparse_state_t st, int32_t layer_id, int32_t batch,
                               int32_t num_heads, int32_t n_locs, const void* q,
                               const int32_t* locs, const int32_t* page_table,
                               float softmax_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (st == nullptr || layer_id < 0 || layer_id >= st->cfg.num_layers) return HISPARSE_E_INVAL;
  if (batch < 0 || num_heads < 1 || num_heads > 1024 || n_locs < 1) return HISPARSE_E_INVAL;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return HISPARSE_E_INVAL;
  if (batch == 0) return HISPARSE_OK;
  if (q == nullptr || locs == nullptr || out == nullptr) return HISPARSE_E_INVAL;
  const int I = st->cfg.item_size_bytes;
  if (I != 1152 && I != 656) return HISPARSE_E_UNSUPPORTED;
  const bool page = st->cfg.page_size > 1;
  if (page != (page_table != nullptr)) return HISPARSE_E_INVAL;
  if (n_locs > mla_max_locations()) return HISPARSE_E_UNSUPPORTED;
  const int64_t kv_rows = static_cast<int64_t>(st->cfg.max_requests) * st->rows * st->cfg.page_size;
  if (kv_rows * I >= (int64_t{1} << 31)) return HISPARSE_E_UNSUPPORTED;  // 32-bit buffer offsets
  if (workspace_bytes < mla_workspace_bytes(batch, num_heads, n_locs, st->num_cus) ||
      (workspace_bytes > 0 && workspace == nullptr))
    return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  MlaDecodeCall c{};
  c.q = q;
  c.locs = locs;
  c.page_table = page ? page_table : nullptr;
  c.kv = st->dev_kv[layer_id];
  c.kv_rows = kv_rows;
  c.item_bytes = I;
  c.page_size = st->cfg.page_size;
  c.pt_stride = st->cfg.hot_buffer_size;
  c.batch = batch;
  c.heads = num_heads;
  c.n_locs = n_locs;
  c.num_cus = st->num_cus;
  c.scale = softmax_scale;
  c.out = out;
  c.lse = lse;
  c.workspace = workspace;
  c.err = st->err;
  return status_of(launch_mla_decode(c, static_cast<hipStream_t>(stream)));
}

namespace {
bool topk_sizes_ok(int32_t batch, int32_t max_len) {
  return batch >= 1 && batch <= (1 << 20) && max_len >= 1 && max_len <= (1 << 28);
}

// Pointer, plan, mode and (optionally) workspace checks of a top-k call whose
// sizes passed topk_sizes_ok and topk_shape_supported.
int topk_call_check(const hisparse_topk_call_t* c, bool with_workspace) {
  if (!c->logits || !c->seq_lens || !c->plan || !c->indices || !c->error_word)
    return HISPARSE_E_INVAL;
  if (c->plan_ints < hisparse_topk_plan_ints(c->batch, c->max_len)) return HISPARSE_E_INVAL;
  switch (c->mode) {
    case HISPARSE_INDEX_NONE:
      break;
    case HISPARSE_INDEX_PAGED:
      if (!c->locs || !c->page_table || c->pt_stride < 1 || c->page_size < 1) return HISPARSE_E_INVAL;
      break;
    case HISPARSE_INDEX_RAGGED:
      if (!c->locs || !c->row_offsets) return HISPARSE_E_INVAL;
      break;
    default:
      return HISPARSE_E_INVAL;
  }
  if (with_workspace) {
    const size_t need = hisparse_topk_workspace_bytes(c->batch, c->max_len, c->k);
    if (c->workspace_bytes < need || (need > 0 && c->workspace == nullptr)) return HISPARSE_E_INVAL;
  }
  return HISPARSE_OK;
}
}  // namespace

size_t hisparse_topk_plan_ints(int32_t batch, int32_t max_len) {
  if (!topk_sizes_ok(batch, max_len)) return 0;
  return static_cast<size_t>(
      hisparse::topk_plan_layout(batch, hisparse::topk_max_items(batch, max_len)).ints);
}

int hisparse_topk_plan(int32_t batch, int32_t max_len, const int32_t* seq_lens, int32_t* plan,
                       size_t plan_ints, void* stream) {
  if (!topk_sizes_ok(batch, max_len) || seq_lens == nullptr || plan == nullptr)
    return HISPARSE_E_INVAL;
  if (plan_ints < hisparse_topk_plan_ints(batch, max_len)) return HISPARSE_E_INVAL;
  return status_of(
      hisparse::launch_topk_plan(seq_lens, plan, batch, max_len, static_cast<hipStream_t>(stream)));
}

size_t hisparse_topk_workspace_bytes(int32_t batch, int32_t max_len, int32_t k) {
  if (!topk_sizes_ok(batch, max_len) || !hisparse::topk_shape_supported(max_len, k)) return 0;
  return hisparse::topk_workspace_layout(batch, max_len, k).bytes;
}

int hisparse_topk_index_build(const hisparse_topk_call_t* c, void* stream) {
  if (c == nullptr || !topk_sizes_ok(c->batch, c->max_len) || c->k < 1) return HISPARSE_E_INVAL;
  if (!hisparse::topk_shape_supported(c->max_len, c->k)) return HISPARSE_E_UNSUPPORTED;
  const int rc = topk_call_check(c, /*with_workspace=*/true);
  if (rc != HISPARSE_OK) return rc;
  return status_of(hisparse::launch_topk_index_build(*c, static_cast<hipStream_t>(stream)));
}

int hisparse_topk_index_build_noalloc(const hisparse_topk_call_t* c, void* stream) {
  if (c == nullptr || !topk_sizes_ok(c->batch, c->max_len) || c->k < 1) return HISPARSE_E_INVAL;
  if (!hisparse::topk_shape_supported(c->max_len, c->k)) return HISPARSE_E_UNSUPPORTED;
  if (hisparse_topk_workspace_bytes(c->batch, c->max_len, c->k) >
      HISPARSE_TOPK_STATIC_SCRATCH_BYTES)
    return HISPARSE_E_UNSUPPORTED;
  hisparse_topk_call_t d = *c;
  d.workspace = nullptr;  // the fixed array stands in for it
  d.workspace_bytes = 0;
  const int rc = topk_call_check(&d, /*with_workspace=*/false);
  if (rc != HISPARSE_OK) return rc;
  return status_of(
      hisparse::launch_topk_index_build_noalloc(d, static_cast<hipStream_t>(stream)));
}

int hisparse_request_reset(hisparse_state_t st, int32_t n, const int32_t* req_pool_indices,
                           void* stream) {
  if (st == nullptr || n < 0) return HISPARSE_E_INVAL;
  if (n == 0) return HISPARSE_OK;
  if (req_pool_indices == nullptr) return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  ResetArgs ra{req_pool_indices, st->slot_key, st->ts, st->order, st->refbits, st->ctrl,
               st->err, st->cfg.max_requests, st->cfg.hot_buffer_size, st->hw};
  return status_of(launch_reset(ra, n, st->cfg.num_layers, static_cast<hipStream_t>(stream)));
}

int hisparse_state_export(hisparse_state_t st, int32_t req, int32_t layer, int32_t* slot_key_h,
                          int32_t* policy_h, int32_t* ctrl_h, int32_t* key_slot_h,
                          void* stream) {
  if (st == nullptr || !slot_key_h || !policy_h || !ctrl_h) return HISPARSE_E_INVAL;
  if (req < 0 || req >= st->cfg.max_requests || layer < 0 || layer >= st->cfg.num_layers)
    return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  auto s = static_cast<hipStream_t>(stream);
  const size_t q = static_cast<size_t>(layer) * st->cfg.max_requests + req;
  const int H = st->cfg.hot_buffer_size;
  std::vector<uint32_t> bits(st->hw);
  hipError_t e = hipMemcpyAsync(slot_key_h, st->slot_key + q * H, H * sizeof(int32_t),
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) {
    if (st->ts)
      e = hipMemcpyAsync(policy_h, st->ts + q * H, H * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    else
      e = hipMemcpyAsync(bits.data(), st->refbits + q * st->hw, st->hw * sizeof(uint32_t),
                         hipMemcpyDeviceToHost, s);
  }
  if (e == hipSuccess)
    e = hipMemcpyAsync(ctrl_h, st->ctrl + 2 * q, 2 * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return status_of(e);
  if (!st->ts) host::decode_refbits(bits.data(), H, policy_h);
  if (key_slot_h && host::invert_slot_key(slot_key_h, H, st->nkeys, key_slot_h) != HISPARSE_OK)
    return HISPARSE_E_HIP;  // the device state is not a valid map
  return HISPARSE_OK;
}

int hisparse_state_import(hisparse_state_t st, int32_t req, int32_t layer,
                          const int32_t* slot_key_h, const int32_t* policy_h,
                          const int32_t* ctrl_h, void* stream) {
  if (st == nullptr || !slot_key_h || !policy_h || !ctrl_h) return HISPARSE_E_INVAL;
  if (req < 0 || req >= st->cfg.max_requests || layer < 0 || layer >= st->cfg.num_layers)
    return HISPARSE_E_INVAL;
  const int H = st->cfg.hot_buffer_size;
  const bool lru = st->ts != nullptr;
  host::InstanceImage img;
  const int rc = host::encode_import(H, st->nkeys, lru, slot_key_h, policy_h, ctrl_h, &img);
  if (rc != HISPARSE_OK) return rc;
  DeviceGuard g(st->device);
  auto s = static_cast<hipStream_t>(stream);
  const size_t q = static_cast<size_t>(layer) * st->cfg.max_requests + req;
  hipError_t e = hipMemcpyAsync(st->slot_key + q * H, slot_key_h, H * sizeof(int32_t),
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess && lru)
    e = hipMemcpyAsync(st->ts + q * H, policy_h, H * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess && lru)
    e = hipMemcpyAsync(st->order + q * H, img.order.data(), H * sizeof(int16_t),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess && !lru)
    e = hipMemcpyAsync(st->refbits + q * st->hw, img.refbits.data(), st->hw * sizeof(uint32_t),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(st->ctrl + 2 * q, ctrl_h, 2 * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return status_of(e);
}

int hisparse_get_error_flags(hisparse_state_t st, uint32_t* flags_h, int32_t clear,
                             void* stream) {
  if (st == nullptr || flags_h == nullptr) return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  auto s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, st->err, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && clear) e = hipMemsetAsync(st->err, 0, sizeof(uint32_t), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return status_of(e);
  *flags_h = v;
  return HISPARSE_OK;
}

const char* hisparse_strerror(int code) {
  switch (code) {
    case HISPARSE_OK: return "success";
    case HISPARSE_E_INVAL: return "invalid argument";
    case HISPARSE_E_NOMEM: return "out of memory";
    case HISPARSE_E_HIP: return "HIP runtime error";
    case HISPARSE_E_UNSUPPORTED: return "outside the limits of this library";
    default: return "unknown status";
  }
}

int hisparse_host_alloc(size_t bytes, void** out_h) {
  if (out_h == nullptr || bytes == 0) return HISPARSE_E_INVAL;
  *out_h = nullptr;
  hipError_t e = hipHostMalloc(out_h, bytes, HISPARSE_HOST_ALLOC_FLAGS);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    *out_h = nullptr;
    return status_of(e) == HISPARSE_E_HIP ? HISPARSE_E_NOMEM : status_of(e);
  }
  return HISPARSE_OK;
}

int hisparse_host_free(void* p_h) {
  if (p_h == nullptr) return HISPARSE_OK;
  return status_of(hipHostFree(p_h));
}

int hisparse_profile_enable(hisparse_state_t st, int32_t enable) {
  if (st == nullptr) return HISPARSE_E_INVAL;
  st->profiling = enable != 0;
  return HISPARSE_OK;
}

int hisparse_profile_read(hisparse_state_t st, hisparse_profile_t* out_h) {
  if (st == nullptr || out_h == nullptr) return HISPARSE_E_INVAL;
  DeviceGuard g(st->device);
  auto* ps = static_cast<ProfiledState*>(st);
  const hipError_t e = drain_events(st, &ps->sums);
  out_h->calls = ps->sums.calls;
  out_h->plan_ms = ps->sums.plan_ms;
  out_h->copy_ms = ps->sums.copy_ms;
  out_h->fused_calls = ps->sums.fused;
  ps->sums = ProfileSums{};
  return status_of(e);
}

}  // extern "C"
