// Top-k selection fused with the index-table build ("SGLang HiSparse" blog,
// section 2.2: a plan computed from the sequence lengths alone and reused by
// every layer of a step; one kernel that selects the top-k from the indexer
// scores and writes the index table without a global round trip; section
// 2.3: PAGED and RAGGED index tables).
//
// Selection rule: the min(k, seq_len) positions of [0, seq_len) with the
// largest scores, ties to the lower position, NaN below every number; output
// in ascending position order, -1 padded.  Scores map to order-preserving
// 32-bit keys (+0/-0 merged, NaN lowest, 0 reserved for "absent"), so the
// selection is: find the exact threshold key T by radix select, then keep
// keys > T and the first `need` keys == T in position order.  The radix
// select takes a 12-bit digit over all keys (a 4096-bin LDS histogram; sign,
// exponent and 3 mantissa bits, so a binade of scores spreads over 8 bins),
// then gathers the keys of the threshold bin into an LDS list (typically a
// few percent) and finishes with 12- and 8-bit digits over that list.
//
// Work split (the plan): a workgroup of 1024 threads takes one chunk of up
// to 32768 positions, 32 scores per thread in registers (8 coalesced
// 16-byte loads); longer rows are split into equal chunks.  A row of one chunk
// is selected and its index table written by that workgroup alone.  The
// chunks of a longer row each select their own top-k (exact: the row's
// top-k is the top-k of the union of its chunks' top-k) and write them as
// candidates; a second kernel on the same stream (its launch is the only
// synchronisation needed) selects each such row's top-k from its
// candidates and writes its index table.  The logits are read from HBM once.
//
// Position order is kept in LDS bitmaps (one bit per position of the
// chunk): the kept positions and the ties at the threshold are marked, and
// one workgroup scan over the bitmap words gives every kept position its
// output index.  Prefix sums use wave64 DPP scans (row shifts and row
// broadcasts, VALU only) and one LDS exchange per workgroup scan.
#include <mutex>
#include <unordered_map>

#include "internal.h"

// Opt-in instrumentation, a separate build (-DHISPARSE_PHASE_CLOCKS=1, see
// phase_clocks.py): each chunk workgroup records the 100 MHz wall clock at
// its phase boundaries (stamps 0-5) and inside the threshold step (6: first
// bin picked, 7: threshold-bin keys listed, 8: first list pass done), each
// merge workgroup at its own (0: start, 1: offsets published, 2: keys and
// histogram, 3: threshold, 4: selection, 5: staging, 6: end);
// hisparse_topk_phase_clocks() and hisparse_topk_merge_phase_clocks() copy
// out the last launch's stamps.  The default build records nothing.
#ifndef HISPARSE_PHASE_CLOCKS
#define HISPARSE_PHASE_CLOCKS 0
#endif
#if HISPARSE_PHASE_CLOCKS
constexpr int kTopkClockRows = 4096;
constexpr int kTopkStamps = 9;
constexpr int kMergeStamps = 7;
__device__ long long g_topk_clock[kTopkClockRows * kTopkStamps];
__device__ long long g_merge_clock[kTopkClockRows * kMergeStamps];
#define TOPK_CLOCK(i)                                                            \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTopkClockRows)                        \
      g_topk_clock[blockIdx.x * kTopkStamps + (i)] = wall_clock64();            \
  } while (0)
#define MERGE_CLOCK(i)                                                           \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kTopkClockRows)                        \
      g_merge_clock[blockIdx.x * kMergeStamps + (i)] = wall_clock64();          \
  } while (0)
extern "C" int hisparse_topk_phase_clocks(long long* out_h, int n) {
  if (n < 0 || n > kTopkClockRows * kTopkStamps) return -1;
  return hipMemcpyFromSymbol(out_h, HIP_SYMBOL(g_topk_clock), n * sizeof(long long)) == hipSuccess
             ? 0 : -1;
}
extern "C" int hisparse_topk_merge_phase_clocks(long long* out_h, int n) {
  if (n < 0 || n > kTopkClockRows * kMergeStamps) return -1;
  return hipMemcpyFromSymbol(out_h, HIP_SYMBOL(g_merge_clock), n * sizeof(long long)) == hipSuccess
             ? 0 : -1;
}
#else
#define TOPK_CLOCK(i) \
  do {                \
  } while (0)
#define MERGE_CLOCK(i) \
  do {                 \
  } while (0)
#endif

namespace hisparse {

namespace {

constexpr int kThreads = kTopkThreads;             // 1024
constexpr int kPer = kTopkChunk / kThreads;        // 32 keys per thread
constexpr int kWaves = kThreads / kWave;           // 16
constexpr int kBins = 4096;                        // 12-bit digits
constexpr int kListCap = 4096;                     // keys of the threshold bin kept in LDS

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct TopkArgs {
  const float* logits;       // [batch][max_len]
  const int32_t* seq_lens;   // [batch]
  const int32_t* plan;       // TopkPlan layout
  int32_t batch, max_len, k, max_items;
  int32_t mode;
  const int32_t* page_table;  // [batch][pt_stride]
  int32_t pt_stride, page_size;
  const int32_t* row_offsets; // [batch]
  int32_t* indices;           // [batch][k]
  int32_t* locs;              // [batch][k] or null
  uint32_t* cand_key;         // [max_items][k]
  int32_t* cand_pos;          // [max_items][k]
  int32_t* cand_cnt;          // [max_items]
  uint32_t* err;
};

// Order-preserving key of a score: larger score -> larger key.  0 is
// reserved for absent positions, NaN is 1 (below -inf), -0 is taken as +0.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  if (x != x) return 1u;
  if (u == 0x80000000u) u = 0u;
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return k + 1u;  // -inf -> 0x00800000; +inf -> 0xFF800001
}

// Exclusive prefix sum over the workgroup (wave_incl_scan per wave); *total gets the sum.  Two
// barriers; `xch` holds kWaves words.  Every thread must call it.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* xch, uint32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) xch[wid] = incl;
  __syncthreads();
  const uint32_t w = lane < kWaves ? xch[lane] : 0u;
  const uint32_t wi = wave_incl_scan(w);
  const uint32_t before = wid > 0 ? __builtin_amdgcn_readlane(wi, wid - 1) : 0u;
  *total = __builtin_amdgcn_readlane(wi, kWaves - 1);
  __syncthreads();
  return before + incl - v;
}

struct Lds {
  uint32_t hist[kBins];               // first digit (and output staging later)
  uint32_t hist1[kBins];              // second digit, over the threshold bin
  uint32_t hist2[256];                // last digit
  uint32_t list[kListCap];
  uint32_t gt_bits[kTopkChunk / 32];  // slot bitmaps: key > T, key == T
  uint32_t eq_bits[kTopkChunk / 32];
  uint32_t xch[kWaves];
  int pick[2];
  int list_count;
  int offs[kTopkMaxChunks + 1];
};

// Slot of element e (= 4v + j) of thread t: slots are positions in the
// chunk (or candidate order in a merge); each thread owns 8 groups of 4
// consecutive slots 4096 apart, so every load of a wave is one coalesced
// 1 KiB block.
__device__ __forceinline__ int slot_of(int e) { return ((e >> 2) * kThreads + threadIdx.x) * 4 + (e & 3); }

// Digit of a key for pass 1 (bits 19..8) and 2 (7..0); pass 0 is bits 31..20.
__device__ __forceinline__ uint32_t digit(uint32_t x, int pass) {
  return pass == 1 ? (x >> 8) & 4095u : x & 255u;
}

// From a pass's histogram `hist`: the bin holding the `remaining`-th
// largest key and the number of keys in higher bins.  Thread j scans
// bins / 1024 bins (at least one), highest first.  Block-wide.
__device__ __forceinline__ void pick_bin(Lds& s, const uint32_t* hist, int bins, int remaining,
                                         uint32_t& bin, int& above_out) {
  const int tid = threadIdx.x;
  const int per = bins >= kThreads ? bins / kThreads : 1;
  const int top = bins - 1 - tid * per;
  uint32_t c = 0u;
  if (top >= 0)
    for (int i = 0; i < per; ++i) c += hist[top - i];
  uint32_t total;
  int above = static_cast<int>(block_scan(c, s.xch, &total));
  if (top >= 0 && c > 0u && above < remaining && remaining <= above + static_cast<int>(c)) {
    for (int i = 0; i < per; ++i) {
      const int h = static_cast<int>(hist[top - i]);
      if (remaining <= above + h) {
        s.pick[0] = top - i;
        s.pick[1] = above;
        break;
      }
      above += h;
    }
  }
  __syncthreads();
  bin = static_cast<uint32_t>(s.pick[0]);
  above_out = s.pick[1];
}

// Exact threshold of the kk largest keys of the workgroup (key 0 = absent;
// kk >= 1, at most the number of present keys): T and the number `need` of
// keys equal to T to keep.  The first-digit histogram is built by the
// caller (hist0) while the keys are loaded.
template <int N, class Stamp>
__device__ __forceinline__ void radix_threshold(const uint32_t (&key)[N], int kk, Lds& s,
                                                uint32_t& T, int& need, Stamp&& stamp) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  uint32_t b0;
  int above;
  pick_bin(s, s.hist, kBins, kk, b0, above);
  stamp(6);
  int remaining = kk - above;
  uint32_t prefix = b0 << 20;

  // keys of bin b0 -> LDS list (any order; typically a few percent of keys):
  // a wave scan of the lanes' counts places them, one LDS atomic per wave
  // reserves the wave's room
  uint32_t cnt = 0u;
#pragma unroll
  for (int e = 0; e < N; ++e) cnt += key[e] != 0u && (key[e] >> 20) == b0;
  const uint32_t incl = wave_incl_scan(cnt);
  const uint32_t wave_total = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (wave_total > 0u) {
    uint32_t base = 0u;
    if (lane == kWave - 1) base = atomicAdd(reinterpret_cast<uint32_t*>(&s.list_count), wave_total);
    int at = static_cast<int>(__builtin_amdgcn_readlane(base, kWave - 1) + incl - cnt);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      if (key[e] != 0u && (key[e] >> 20) == b0) {
        if (at < kListCap) s.list[at] = key[e];
        ++at;
      }
    }
  }
  __syncthreads();
  stamp(7);
  const int m = s.list_count;
  const bool listed = m <= kListCap;
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) {
    const int bins = pass == 1 ? kBins : 256;
    const uint32_t pm = pass == 1 ? 0xFFF00000u : 0xFFFFFF00u;  // bits fixed so far
    // each pass has its own histogram, cleared at kernel start
    uint32_t* hist = pass == 1 ? s.hist1 : s.hist2;
    if (listed) {  // the list holds exactly the keys of bin b0
      for (int i = tid; i < m; i += kThreads) {
        const uint32_t x = s.list[i];
        if ((x & pm) == prefix) atomicAdd(&hist[digit(x, pass)], 1u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e)
        if (key[e] != 0u && (key[e] & pm) == prefix) atomicAdd(&hist[digit(key[e], pass)], 1u);
    }
    __syncthreads();
    uint32_t b;
    pick_bin(s, hist, bins, remaining, b, above);
    remaining -= above;
    prefix |= pass == 1 ? (b << 8) : b;
    if (pass == 1) stamp(8);
  }
  T = prefix;
  need = remaining;
}

// Marks keys > T and keys == T in the slot bitmaps, then thread w takes
// bitmap word w (slots 32w .. 32w + 31): one workgroup scan of the packed
// (count > T, count == T) per word gives, in slot order, the output offset of
// the word's first kept slot; ties are kept while their rank is below
// `need`.  Returns the word's kept bits and its output offset.
template <int N>
__device__ __forceinline__ uint32_t select_word(const uint32_t (&key)[N], uint32_t T, int need,
                                                Lds& s, int& offset) {
  const int tid = threadIdx.x;
  // (the bitmaps were cleared at kernel start)
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (key[e] >= T) {
      const int i = slot_of(e);
      atomicOr(key[e] > T ? &s.gt_bits[i >> 5] : &s.eq_bits[i >> 5], 1u << (i & 31));
    }
  }
  __syncthreads();
  const uint32_t g = s.gt_bits[tid], q = s.eq_bits[tid];
  uint32_t total;
  const uint32_t pre = block_scan((static_cast<uint32_t>(__popc(g)) << 16) | __popc(q), s.xch, &total);
  const int q_pre = static_cast<int>(pre & 0xFFFFu), g_pre = static_cast<int>(pre >> 16);
  int keep_ties = need - q_pre;
  uint32_t qk = 0u;
  for (uint32_t r = q; r != 0u && keep_ties > 0; r &= r - 1u, --keep_ties) qk |= r & (~r + 1u);
  offset = g_pre + min(q_pre, need);
  return g | qk;
}

__device__ __forceinline__ int32_t table_loc(const TopkArgs& a, int row, int32_t p) {
  if (a.mode == HISPARSE_INDEX_RAGGED) return a.row_offsets[row] + p;
  const int j = p / a.page_size;
  const int32_t page =
      p >= 0 && j < a.pt_stride ? a.page_table[static_cast<size_t>(row) * a.pt_stride + j] : -1;
  if (page < 0) {
    raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
    return -1;
  }
  return page * a.page_size + (p - j * a.page_size);
}

// Final outputs of a row: the kept slots of this thread's bitmap word at
// `offset` on (position of slot i: pos_of(i)), then -1 padding from kk on.
template <class PosOf>
__device__ __forceinline__ void emit_final(const TopkArgs& a, int row, PosOf pos_of, uint32_t w,
                                           int offset, int kk) {
  int32_t* idx = a.indices + static_cast<size_t>(row) * a.k;
  int32_t* loc = a.locs ? a.locs + static_cast<size_t>(row) * a.k : nullptr;
  for (uint32_t r = w; r != 0u; r &= r - 1u) {
    const int32_t p = pos_of(32 * static_cast<int>(threadIdx.x) + __builtin_ctz(r));
    idx[offset] = p;
    if (loc) loc[offset] = table_loc(a, row, p);
    ++offset;
  }
  for (int i = kk + threadIdx.x; i < a.k; i += kThreads) {
    idx[i] = -1;
    if (loc) loc[i] = -1;
  }
}

// Largest output count staged through LDS (the list and histogram arrays,
// free once the threshold is known); above it the outputs go word by word.
constexpr int kStageCap = kListCap < kBins ? kListCap : kBins;

// Puts the kept slots in output order into LDS: s.list[o] = slot and
// s.hist[o] = key of the o-th output.  Word w's kept bits and output offset
// (thread w's select_word result) go through the bitmap arrays; each slot's
// owner, which holds its key, places it.  kk <= kStageCap.
template <int N>
__device__ __forceinline__ void stage_kept(const uint32_t (&key)[N], uint32_t kept, int offset,
                                           Lds& s) {
  const int tid = threadIdx.x;
  s.gt_bits[tid] = kept;
  s.eq_bits[tid] = static_cast<uint32_t>(offset);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < N / 4; ++v) {  // slots i0 .. i0 + 3 share a bitmap word
    const int i0 = slot_of(4 * v);
    const uint32_t wv = s.gt_bits[i0 >> 5];
    const uint32_t sh = static_cast<uint32_t>(i0 & 31);
    if ((wv >> sh) & 15u) {
      int o = static_cast<int>(s.eq_bits[i0 >> 5]) + __popc(wv & ((1u << sh) - 1u));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((wv >> (sh + j)) & 1u) {
          s.list[o] = static_cast<uint32_t>(i0 + j);
          s.hist[o] = key[4 * v + j];
          ++o;
        }
      }
    }
  }
  __syncthreads();
}

// Final outputs from the staged slots: thread t writes outputs t, t + 1024,
// ... (contiguous stores; the position and page-table loads of a thread's
// outputs go out together), then -1 padding from kk on.
template <class PosOf>
__device__ __forceinline__ void emit_staged(const TopkArgs& a, int row, PosOf pos_of, const Lds& s,
                                            int kk) {
  constexpr int kBatch = 2;
  int32_t* idx = a.indices + static_cast<size_t>(row) * a.k;
  int32_t* loc = a.locs ? a.locs + static_cast<size_t>(row) * a.k : nullptr;
  for (int o0 = threadIdx.x; o0 < kk; o0 += kBatch * kThreads) {
    int32_t pos[kBatch], lv[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int o = o0 + j * kThreads;
      pos[j] = o < kk ? pos_of(static_cast<int>(s.list[o])) : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) lv[j] = loc && pos[j] >= 0 ? table_loc(a, row, pos[j]) : -1;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int o = o0 + j * kThreads;
      if (o < kk) {
        idx[o] = pos[j];
        if (loc) loc[o] = lv[j];
      }
    }
  }
  for (int i = kk + threadIdx.x; i < a.k; i += kThreads) {
    idx[i] = -1;
    if (loc) loc[i] = -1;
  }
}

__device__ __forceinline__ bool row_rejected(const TopkArgs& a, int row) {
  const int seq = a.seq_lens[row];
  return seq < 0 || seq > a.max_len;
}

__global__ __launch_bounds__(kThreads) void topk_plan_kernel(const int32_t* seq_lens, int32_t* plan,
                                                             int32_t batch, int32_t max_len,
                                                             int32_t max_items) {
  __shared__ uint32_t xch[kWaves];
  const TopkPlan p = topk_plan_layout(batch, max_items);
  int carry = 0;
  for (int b0 = 0; b0 < batch; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    int s = 0, n = 0;
    if (b < batch) {
      s = seq_lens[b];
      if (s < 0 || s > max_len) s = 0;
      n = max(1, (s + kTopkChunk - 1) / kTopkChunk);
    }
    uint32_t total;
    const int first = carry + static_cast<int>(block_scan(static_cast<uint32_t>(n), xch, &total));
    if (b < batch) {
      plan[p.row_info + 2 * b] = first;
      plan[p.row_info + 2 * b + 1] = n;
      const int per = (s + n - 1) / n;
      const int len = (per + kTopkAlign - 1) / kTopkAlign * kTopkAlign;
      for (int c = 0; c < n; ++c) {
        int32_t* it = plan + p.items + 4 * (first + c);
        it[0] = b;
        it[1] = c;
        it[2] = c * len;
        it[3] = max(0, min(len, s - c * len));
      }
    }
    carry += static_cast<int>(total);
  }
  if (threadIdx.x == 0) {
    plan[0] = carry;
    plan[1] = max_len;
  }
}

// One workgroup per plan item (chunk).
// At most 64 VGPRs (8 waves per SIMD): two 1024-thread workgroups share a CU,
// so a 512-chunk call runs in one round instead of two.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void topk_chunk_kernel(TopkArgs a) {
  __shared__ Lds s;
  const TopkPlan p = topk_plan_layout(a.batch, a.max_items);
  const int w = blockIdx.x;  // < max_items: its item slot lies in the plan
  const int tid = threadIdx.x;
  // Two rounds of dependent loads before the scores: the item count and this
  // workgroup's item together, then the row's length and chunk count
  // together with its scores (a rejected row has an empty item, so its
  // score loads read nothing).  The LDS clears go out meanwhile.
  const int n_items = a.plan[0];
  const int32_t* item = a.plan + p.items + 4 * w;
  const int row = item[0], start = item[2], item_len = item[3];
  for (int i = tid; i < kBins; i += kThreads) {
    s.hist[i] = 0u;
    s.hist1[i] = 0u;
  }
  if (tid < 256) s.hist2[tid] = 0u;
  s.gt_bits[tid] = 0u;  // one word per thread
  s.eq_bits[tid] = 0u;
  if (tid == 0) s.list_count = 0;
  if (w >= n_items) return;
  TOPK_CLOCK(0);
  // an item outside these sizes (a plan made for other sizes): nothing read
  if (row < 0 || row >= a.batch || start < 0 || start > a.max_len) {
    if (tid == 0) raise_error(a.err, HISPARSE_ERR_BAD_PLAN);
    return;
  }
  const int len = max(0, min(item_len, a.max_len - start));
  const int seq = a.seq_lens[row];
  const int n_chunks = a.plan[p.row_info + 2 * row + 1];
  // This thread's scores (positions start + slot), read by buffer loads
  // with no per-lane branch, so all of a thread's loads are in flight at
  // once (a lane-dependent branch around each load made every one wait for
  // the previous): the buffer covers the chunk, a dword past it reads as
  // zero, and slots past `len` are masked.  One dword load per slot; the
  // compiler merges each thread's four consecutive slots into one 16-byte
  // load.
  const float* src = a.logits + static_cast<size_t>(row) * a.max_len + start;
  float x[kPer];
  {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src), 0, 4 * len, 0x00020000);
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      x[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, 4 * slot_of(e), 0, 0));
  }
  // a chunk count no plan for these sizes has (a split row needs the
  // candidate workspace)
  if (n_chunks < 1 || n_chunks > kTopkMaxChunks || (n_chunks > 1 && a.cand_key == nullptr)) {
    if (tid == 0) raise_error(a.err, HISPARSE_ERR_BAD_PLAN);
    return;
  }
  // a rejected row keeps no position: its outputs are all -1
  const bool rejected = seq < 0 || seq > a.max_len;
  if (rejected && tid == 0) raise_error(a.err, HISPARSE_ERR_BAD_ROW);
  const int kept_len = rejected ? 0 : len;
  __syncthreads();  // histogram cleared
  // keys and the first-digit histogram as the scores arrive
  uint32_t key[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    key[e] = slot_of(e) < kept_len ? score_key(x[e]) : 0u;
    if (key[e] != 0u) atomicAdd(&s.hist[key[e] >> 20], 1u);
  }
  __syncthreads();
  TOPK_CLOCK(1);
  const int kk = min(a.k, kept_len);
  uint32_t T = 0u, kept = 0u;
  int need = 0, offset = 0;
  if (kk > 0) {
    radix_threshold(key, kk, s, T, need, [](int i) { TOPK_CLOCK(i); });
    TOPK_CLOCK(2);
    kept = select_word(key, T, need, s, offset);
  }
  TOPK_CLOCK(3);
  const bool staged = kk <= kStageCap;
  if (staged) stage_kept(key, kept, offset, s);
  TOPK_CLOCK(4);
  if (n_chunks == 1) {
    if (staged)
      emit_staged(a, row, [&](int i) { return start + i; }, s, kk);
    else
      emit_final(a, row, [&](int i) { return start + i; }, kept, offset, kk);
    TOPK_CLOCK(5);
    return;
  }
  // a chunk of a split row: its candidates (key, position) in slot order,
  // for topk_merge_kernel
  uint32_t* ck = a.cand_key + static_cast<size_t>(blockIdx.x) * a.k;
  int32_t* cp = a.cand_pos + static_cast<size_t>(blockIdx.x) * a.k;
  if (staged) {
    for (int o = tid; o < kk; o += kThreads) {
      ck[o] = s.hist[o];
      cp[o] = start + static_cast<int>(s.list[o]);
    }
  } else {  // the keys of the kept slots are read again (L2)
    for (uint32_t r = kept; r != 0u; r &= r - 1u) {
      const int i = 32 * tid + __builtin_ctz(r);
      ck[offset] = score_key(src[i]);
      cp[offset] = start + i;
      ++offset;
    }
  }
  if (tid == 0) a.cand_cnt[blockIdx.x] = kk;
}

// One workgroup per row: rows of several chunks select their top-k from the
// chunks' candidates, which are in position order (chunk order, ascending
// within a chunk).  N candidate slots per thread: the launch takes the
// smallest N in {8, 16, 32} whose N x 1024 slots hold every candidate a row
// of max_len can have (4 chunks of top-2048: 8192 candidates, N = 8), so the
// per-slot work scales with the candidates rather than a full chunk.
template <int N>
__global__ __launch_bounds__(kThreads) void topk_merge_kernel(TopkArgs a) {
  __shared__ Lds s;
  const TopkPlan p = topk_plan_layout(a.batch, a.max_items);
  const int row = blockIdx.x;
  const int n_chunks = a.plan[p.row_info + 2 * row + 1];
  const int first = a.plan[p.row_info + 2 * row];
  if (n_chunks == 1 || row_rejected(a, row)) return;
  const int tid = threadIdx.x;
  MERGE_CLOCK(0);
  // a row entry outside these sizes (a plan made for other sizes)
  if (n_chunks < 1 || n_chunks > kTopkMaxChunks || n_chunks * a.k > N * kThreads ||
      first < 0 || first > a.max_items - n_chunks) {
    if (tid == 0) raise_error(a.err, HISPARSE_ERR_BAD_PLAN);
    return;
  }
  // one barrier publishes the chunk offsets and the cleared histograms and
  // bitmaps
  if (tid == 0) {
    int acc = 0;
    for (int c = 0; c < n_chunks; ++c) {
      s.offs[c] = acc;
      acc += min(max(a.cand_cnt[first + c], 0), a.k);  // (a count is at most k)
    }
    s.offs[n_chunks] = acc;
  }
  for (int i = tid; i < kBins; i += kThreads) {
    s.hist[i] = 0u;
    s.hist1[i] = 0u;
  }
  if (tid < 256) s.hist2[tid] = 0u;
  s.gt_bits[tid] = 0u;  // one word per thread
  s.eq_bits[tid] = 0u;
  if (tid == 0) s.list_count = 0;
  __syncthreads();
  MERGE_CLOCK(1);
  const int M = s.offs[n_chunks];
  // candidate i sits in chunk c, the last with offs[c] <= i (binary search);
  // its index relative to the row's first chunk
  auto rel_at = [&](int i) {
    int lo = 0, hi = n_chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s.offs[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    return lo * a.k + (i - s.offs[lo]);
  };
  auto cand_at = [&](int i) { return static_cast<size_t>(first) * a.k + rel_at(i); };
  // Every slot's key is loaded before any is used: buffer loads over the
  // row's candidates with no per-lane branch; a slot past M reads past the
  // buffer, i.e. key 0, absent.
  uint32_t key[N];
  {
    const uint32_t range = 4u * static_cast<uint32_t>(n_chunks * a.k);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        a.cand_key + static_cast<size_t>(first) * a.k, 0, static_cast<int>(range), 0x00020000);
    int off[N];
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int i = slot_of(e);
      off[e] = i < M ? 4 * rel_at(i) : static_cast<int>(range);
    }
#pragma unroll
    for (int e = 0; e < N; ++e) key[e] = __builtin_amdgcn_raw_buffer_load_b32(rs, off[e], 0, 0);
  }
#pragma unroll
  for (int e = 0; e < N; ++e)
    if (key[e] != 0u) atomicAdd(&s.hist[key[e] >> 20], 1u);
  __syncthreads();
  MERGE_CLOCK(2);
  const int kf = min(a.k, M);
  uint32_t T = 0u, w = 0u;
  int need = 0, offset = 0;
  if (kf > 0) {
    radix_threshold(key, kf, s, T, need, [](int) {});
    MERGE_CLOCK(3);
    w = select_word(key, T, need, s, offset);
  }
  MERGE_CLOCK(4);
  if (kf <= kStageCap) {
    if (kf > 0) stage_kept(key, w, offset, s);
    MERGE_CLOCK(5);
    emit_staged(a, row, [&](int i) { return a.cand_pos[cand_at(i)]; }, s, kf);
  } else {
    emit_final(a, row, [&](int i) { return a.cand_pos[cand_at(i)]; }, w, offset, kf);
  }
  MERGE_CLOCK(6);
}

}  // namespace

hipError_t launch_topk_plan(const int32_t* seq_lens, int32_t* plan, int32_t batch, int32_t max_len,
                            hipStream_t st) {
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(kThreads), 0, st, seq_lens, plan, batch,
                     max_len, topk_max_items(batch, max_len));
  return hipGetLastError();
}

// Scratch of hisparse_topk_index_build_noalloc: the split rows' candidates
// live in this fixed array instead of a caller workspace.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol); it passes the device address hipGetSymbolAddress returns for
// the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[HISPARSE_TOPK_STATIC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mutex;
std::unordered_map<int, void*> g_scratch_ptr;  // device -> address of `scratch` there

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch_ptr.find(dev);
  if (it != g_scratch_ptr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || ptr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
  g_scratch_ptr.emplace(dev, ptr);
  *out = ptr;
  return hipSuccess;
}
}  // namespace

hipError_t launch_topk_index_build_noalloc(const hisparse_topk_call_t& c, hipStream_t st) {
  hisparse_topk_call_t d = c;
  d.workspace_bytes = topk_workspace_layout(c.batch, c.max_len, c.k).bytes;
  d.workspace = nullptr;
  if (d.workspace_bytes > 0) {
    const hipError_t e = scratch_address(&d.workspace);
    if (e != hipSuccess) return e;
  }
  return launch_topk_index_build(d, st);
}

hipError_t launch_topk_index_build(const hisparse_topk_call_t& c, hipStream_t st) {
  TopkArgs a{};
  a.logits = c.logits;
  a.seq_lens = c.seq_lens;
  a.plan = c.plan;
  a.batch = c.batch;
  a.max_len = c.max_len;
  a.k = c.k;
  a.max_items = topk_max_items(c.batch, c.max_len);
  a.mode = c.mode;
  a.page_table = c.page_table;
  a.pt_stride = c.pt_stride;
  a.page_size = c.page_size;
  a.row_offsets = c.row_offsets;
  a.indices = c.indices;
  a.locs = c.mode == HISPARSE_INDEX_NONE ? nullptr : c.locs;
  const TopkWorkspace ws = topk_workspace_layout(c.batch, c.max_len, c.k);
  uint8_t* base = static_cast<uint8_t*>(c.workspace);
  a.cand_key = ws.bytes ? reinterpret_cast<uint32_t*>(base + ws.key) : nullptr;
  a.cand_pos = ws.bytes ? reinterpret_cast<int32_t*>(base + ws.pos) : nullptr;
  a.cand_cnt = ws.bytes ? reinterpret_cast<int32_t*>(base + ws.cnt) : nullptr;
  a.err = c.error_word;
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(a.max_items), dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_items == a.batch) return e;  // no row can be split
  // candidate slots per merge thread: the most a row of max_len can have
  const int most = topk_chunks(c.max_len) * c.k;
  if (most <= 8 * kThreads)
    hipLaunchKernelGGL(topk_merge_kernel<8>, dim3(a.batch), dim3(kThreads), 0, st, a);
  else if (most <= 16 * kThreads)
    hipLaunchKernelGGL(topk_merge_kernel<16>, dim3(a.batch), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(topk_merge_kernel<32>, dim3(a.batch), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hisparse
