// Internal declarations shared by the ABI implementation and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "copy.h"
#include "device_common.h"
#include "hisparse.h"
#include "host_logic.h"

namespace hisparse {

constexpr int kPlanThreads = 1024;  // one workgroup (16 waves) per batch row
constexpr int kMaxPageModeHot = host::kMaxPageModeHot;
static_assert((HISPARSE_MAX_HOT + 31) / 32 <= kPlanThreads,
              "one thread per word of an H-bit mask in the plan kernels");

// Top-k selection + index-table build (topk.hip).
constexpr int kTopkThreads = 1024;
constexpr int kTopkChunk = HISPARSE_TOPK_CHUNK;          // rows above this are split
constexpr int kTopkMaxCandidates = HISPARSE_TOPK_MAX_CANDIDATES;
constexpr int kTopkMaxChunks = HISPARSE_TOPK_MAX_CHUNKS;
constexpr int kTopkAlign = 1024;
static_assert(kTopkChunk % kTopkThreads == 0 && kTopkMaxCandidates <= kTopkChunk, "chunk shape");

// Word offsets inside a plan: [0] n_items, [1] max_len, row_info [batch][2],
// items [max_items][4].
struct TopkPlan {
  int row_info, items, ints;
};
__host__ __device__ inline int topk_chunks(int len) {
  const int n = (len + kTopkChunk - 1) / kTopkChunk;
  return n < 1 ? 1 : n;
}
__host__ __device__ inline int topk_max_items(int batch, int max_len) {
  return batch * topk_chunks(max_len);
}
__host__ __device__ inline TopkPlan topk_plan_layout(int batch, int max_items) {
  return TopkPlan{2, 2 + 2 * batch, 2 + 2 * batch + 4 * max_items};
}
// Byte offsets of the candidate arrays in the workspace (none when no row
// can be split).
struct TopkWorkspace {
  size_t key, pos, cnt, bytes;
};
inline TopkWorkspace topk_workspace_layout(int batch, int max_len, int k) {
  if (topk_chunks(max_len) == 1) return TopkWorkspace{0, 0, 0, 0};
  const size_t items = static_cast<size_t>(topk_max_items(batch, max_len));
  const size_t words = items * static_cast<size_t>(k);
  return TopkWorkspace{0, 4 * words, 8 * words, 8 * words + 4 * items};
}
// A split row merges chunks x k candidates: at most 32768, from at most 64
// chunks.
inline bool topk_shape_supported(int max_len, int k) {
  const int n = topk_chunks(max_len);
  if (k < 1 || k > kTopkChunk) return false;
  return n == 1 || (n <= kTopkMaxChunks && static_cast<int64_t>(n) * k <= kTopkMaxCandidates);
}
hipError_t launch_topk_plan(const int32_t* seq_lens, int32_t* plan, int32_t batch, int32_t max_len,
                            hipStream_t st);
hipError_t launch_topk_index_build(const hisparse_topk_call_t& c, hipStream_t st);
hipError_t launch_topk_index_build_noalloc(const hisparse_topk_call_t& c, hipStream_t st);

struct ResetArgs {
  const int32_t* reqs;  // NULL = requests 0..n-1
  int32_t* slot_key;
  int32_t* ts;
  int16_t* order;
  uint32_t* refbits;
  int32_t* ctrl;
  uint32_t* err;
  int32_t R, H, Hw;
};

// One sparse MLA decode-attention call (see hisparse_sparse_mla_decode).
struct MlaDecodeCall {
  const void* q;
  const int32_t* locs;
  const int32_t* page_table;
  const uint8_t* kv;
  int64_t kv_rows;
  int32_t item_bytes, page_size, pt_stride;
  int32_t batch, heads, n_locs, num_cus;
  float scale;
  float* out;
  float* lse;
  void* workspace;
  uint32_t* err;
};
int mla_splits(int batch, int heads, int n_locs, int num_cus);
int mla_max_locations();
size_t mla_workspace_bytes(int batch, int heads, int n_locs, int num_cus);
hipError_t launch_mla_decode(const MlaDecodeCall& c, hipStream_t s);

int hash_size_for(int entries, bool pow2);
constexpr int kMaxSortedKeys = 1 << 18;  // keys per request with a sorted copy list
size_t lru_token_lds_bytes(const PlanArgs& a);
size_t lru_page_lds_bytes(const PlanArgs& a);
size_t clock_lds_bytes(const PlanArgs& a);

hipError_t launch_lru_token_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_lru_page_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_clock_plan(const PlanArgs& a, hipStream_t s);
hipError_t launch_reset(const ResetArgs& a, int n, int layers, hipStream_t s);

}  // namespace hisparse

struct hisparse_state {
  hisparse_config_t cfg{};
  std::vector<const uint8_t*> host_kv;  // device-visible addresses
  std::vector<uint8_t*> dev_kv;
  int device = 0;
  int32_t rows = 0;     // device rows per request
  int32_t scratch = 0;  // CLOCK scratch rows per request
  int32_t nkeys = 0;    // keys per request (tokens or pages)
  int32_t hw = 0;       // 32-bit words of an H-bit mask
  int32_t cap = 0;      // plan capacity per row
  // device memory, one allocation
  void* arena = nullptr;
  int32_t* slot_key = nullptr;
  int32_t* ts = nullptr;
  int16_t* order = nullptr;
  uint32_t* refbits = nullptr;
  int32_t* ctrl = nullptr;
  int32_t* ws_src = nullptr;
  int32_t* ws_dst = nullptr;
  int32_t* ws_victim = nullptr;
  int32_t* cp_src = nullptr;  // copy list in ascending host-row order
  int32_t* cp_dst = nullptr;
  uint32_t* err = nullptr;
  size_t max_lds = 0;         // dynamic LDS a workgroup may use
  int num_cus = 0;
  // profiling: triples of events (before plan, after plan, after copy)
  bool profiling = false;
  hisparse::host::EventLedger<hipEvent_t> events;
};
