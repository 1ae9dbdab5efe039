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
// selection is: find the exact threshold key T by radix select (four 8-bit
// digits, LDS histograms), then keep keys > T and the first `need` keys == T
// in position order.
//
// Work split (the plan): a row of up to 32768 positions is one workgroup of
// 1024 threads holding 32 consecutive scores per thread in registers; a
// longer row is split into equal chunks of at most 32768.  Each chunk
// selects its own top-k (exact: the row's top-k is the top-k of the union of
// its chunks' top-k), writes it as candidates, and the last chunk of the row
// to finish (a device-scope ticket) selects the final top-k from the
// candidates.  The logits are read from HBM exactly once.
#include "internal.h"

namespace hisparse {

namespace {

constexpr int kThreads = kTopkThreads;       // 1024
constexpr int kPer = kTopkChunk / kThreads;  // 32 scores per thread
constexpr int kWaves = kThreads / kWave;     // 16

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TopkArgs {
  const float* logits;       // [batch][max_len]
  const int32_t* seq_lens;   // [batch]
  int32_t* plan;             // TopkPlan layout (its ticket counters are updated)
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

struct Lds {
  uint32_t hist[kWaves][256];
  int scan[kWaves + 1];
  int pick[2];
  int offs[kTopkMaxChunks + 1];
  int last;
};

// Exact threshold of the kk largest keys (kk >= 1, at most the number of
// present keys): T and the number `need` of keys equal to T to keep.
__device__ __forceinline__ void radix_threshold(const uint32_t (&key)[kPer], int kk, Lds& s,
                                                uint32_t& T, int& need) {
  const int tid = threadIdx.x, wave = tid / kWave;
  uint32_t prefix = 0u, mask = 0u;
  int remaining = kk;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < kWaves * 256; i += kThreads) (&s.hist[0][0])[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t x = key[e];
      if (x != 0u && (x & mask) == prefix) atomicAdd(&s.hist[wave][(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    // thread j < 256 looks at bin 255 - j, so the exclusive scan gives the
    // number of keys in higher bins
    int c = 0;
    if (tid < 256) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) c += static_cast<int>(s.hist[w][255 - tid]);
    }
    int total;
    const int above = block_exclusive_scan<kThreads>(c, s.scan, &total);
    if (tid < 256 && c > 0 && above < remaining && remaining <= above + c) {
      s.pick[0] = 255 - tid;
      s.pick[1] = above;
    }
    __syncthreads();
    const uint32_t digit = static_cast<uint32_t>(s.pick[0]);
    remaining -= s.pick[1];
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
  need = remaining;
}

// Keeps keys > T and the first `need` keys == T (position order = thread
// order, then element order) and returns, per thread, the selection mask and
// the output offset of its first kept element.
__device__ __forceinline__ uint32_t select_mask(const uint32_t (&key)[kPer], uint32_t T, int need,
                                                Lds& s, int& offset) {
  int ties = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) ties += key[e] == T;
  int total;
  int rank = block_exclusive_scan<kThreads>(ties, s.scan, &total);
  uint32_t m = 0u;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    bool keep = key[e] > T;
    if (key[e] == T) keep = rank++ < need;
    m |= static_cast<uint32_t>(keep) << e;
  }
  offset = block_exclusive_scan<kThreads>(__popc(m), s.scan, &total);
  return m;
}

__device__ __forceinline__ int32_t table_loc(const TopkArgs& a, int row, int32_t p) {
  if (a.mode == HISPARSE_INDEX_RAGGED) return a.row_offsets[row] + p;
  const int j = p / a.page_size;
  const int32_t page = j < a.pt_stride ? a.page_table[static_cast<size_t>(row) * a.pt_stride + j] : -1;
  if (page < 0) {
    raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
    return -1;
  }
  return page * a.page_size + (p - j * a.page_size);
}

// Final outputs of a row from the kept elements (position of element e:
// pos_of(e)) and -1 padding from kk on.
template <class PosOf>
__device__ __forceinline__ void emit_final(const TopkArgs& a, int row, PosOf pos_of, uint32_t m,
                                           int offset, int kk) {
  int32_t* idx = a.indices + static_cast<size_t>(row) * a.k;
  int32_t* loc = a.locs ? a.locs + static_cast<size_t>(row) * a.k : nullptr;
  for (uint32_t r = m; r != 0u; r &= r - 1u) {
    const int32_t p = pos_of(__builtin_ctz(r));
    idx[offset] = p;
    if (loc) loc[offset] = table_loc(a, row, p);
    ++offset;
  }
  for (int i = kk + threadIdx.x; i < a.k; i += kThreads) {
    idx[i] = -1;
    if (loc) loc[i] = -1;
  }
}

__global__ __launch_bounds__(kThreads) void topk_plan_kernel(const int32_t* seq_lens, int32_t* plan,
                                                             int32_t batch, int32_t max_len,
                                                             int32_t max_items) {
  __shared__ int scan[kWaves + 1];
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
    int total;
    const int first = carry + block_exclusive_scan<kThreads>(n, scan, &total);
    if (b < batch) {
      plan[p.row_info + 2 * b] = first;
      plan[p.row_info + 2 * b + 1] = n;
      plan[p.tickets + b] = 0;
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
    carry += total;
  }
  if (threadIdx.x == 0) {
    plan[0] = carry;
    plan[1] = max_len;
  }
}

__global__ __launch_bounds__(kThreads) void topk_index_build_kernel(TopkArgs a) {
  __shared__ Lds s;
  const TopkPlan p = topk_plan_layout(a.batch, a.max_items);
  const int w = blockIdx.x;
  if (w >= a.plan[0]) return;
  const int tid = threadIdx.x;
  const int32_t* item = a.plan + p.items + 4 * w;
  const int row = item[0], start = item[2], len = item[3];
  const int n_chunks = a.plan[p.row_info + 2 * row + 1];
  const int seq = a.seq_lens[row];
  if (seq < 0 || seq > a.max_len) {  // rejected row: one empty chunk
    if (tid == 0) raise_error(a.err, HISPARSE_ERR_BAD_ROW);
    for (int i = tid; i < a.k; i += kThreads) {
      a.indices[static_cast<size_t>(row) * a.k + i] = -1;
      if (a.locs) a.locs[static_cast<size_t>(row) * a.k + i] = -1;
    }
    return;
  }

  // this thread's scores: positions start + 32 tid + e
  uint32_t key[kPer];
  const int base = kPer * tid;
  {
    const float* src = a.logits + static_cast<size_t>(row) * a.max_len + start + base;
    if (base + kPer <= len && ((reinterpret_cast<uintptr_t>(src) & 15u) == 0u)) {
#pragma unroll
      for (int v = 0; v < kPer / 4; ++v) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * v);
#pragma unroll
        for (int j = 0; j < 4; ++j) key[4 * v + j] = score_key(x[j]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kPer; ++e) key[e] = base + e < len ? score_key(src[e]) : 0u;
    }
  }
  const int kk = min(a.k, len);
  uint32_t T = 0u;
  int need = 0;
  if (kk > 0) radix_threshold(key, kk, s, T, need);
  int offset;
  const uint32_t m = kk > 0 ? select_mask(key, T, need, s, offset) : (offset = 0, 0u);
  if (n_chunks == 1) {
    emit_final(a, row, [&](int e) { return start + base + e; }, m, offset, kk);
    return;
  }

  // several chunks: publish this chunk's candidates, take a ticket
  {
    uint32_t* ck = a.cand_key + static_cast<size_t>(w) * a.k;
    int32_t* cp = a.cand_pos + static_cast<size_t>(w) * a.k;
    for (uint32_t r = m; r != 0u; r &= r - 1u) {
      const int e = __builtin_ctz(r);
      ck[offset] = key[e];
      cp[offset] = start + base + e;
      ++offset;
    }
    if (tid == 0) a.cand_cnt[w] = kk;
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int old = atomicAdd(a.plan + p.tickets + row, 1);
    s.last = old == n_chunks - 1;
  }
  __syncthreads();
  if (!s.last) return;
  __threadfence();

  // the last chunk of the row: final selection over all candidates, which
  // are in position order (chunk order, ascending within a chunk)
  const int first = a.plan[p.row_info + 2 * row];
  if (tid == 0) {
    int acc = 0;
    for (int c = 0; c < n_chunks; ++c) {
      s.offs[c] = acc;
      acc += a.cand_cnt[first + c];
    }
    s.offs[n_chunks] = acc;
    a.plan[p.tickets + row] = 0;  // ready for the next call
  }
  __syncthreads();
  const int M = s.offs[n_chunks];
  // candidate i of the row sits in chunk c with offs[c] <= i < offs[c + 1]
  auto cand_at = [&](int i) {
    int c = 0;
    while (c + 1 < n_chunks && s.offs[c + 1] <= i) ++c;
    return static_cast<size_t>(first + c) * a.k + (i - s.offs[c]);
  };
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = base + e;
    key[e] = i < M ? a.cand_key[cand_at(i)] : 0u;
  }
  const int kf = min(a.k, M);
  if (kf > 0) radix_threshold(key, kf, s, T, need);
  const uint32_t mf = kf > 0 ? select_mask(key, T, need, s, offset) : (offset = 0, 0u);
  emit_final(a, row, [&](int e) { return a.cand_pos[cand_at(base + e)]; }, mf, offset, kf);
}

}  // namespace

hipError_t launch_topk_plan(const int32_t* seq_lens, int32_t* plan, int32_t batch, int32_t max_len,
                            hipStream_t st) {
  hipLaunchKernelGGL(topk_plan_kernel, dim3(1), dim3(kThreads), 0, st, seq_lens, plan, batch,
                     max_len, topk_max_items(batch, max_len));
  return hipGetLastError();
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
  hipLaunchKernelGGL(topk_index_build_kernel, dim3(a.max_items), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hisparse
