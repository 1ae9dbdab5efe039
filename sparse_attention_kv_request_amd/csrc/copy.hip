// Miss copy: host KV tier (pinned, device-mapped) -> hot rows in HBM.
//
// The pages keep idle KV in CPU memory and load the selected entries into the
// device buffer (PR #20343 summary, "Features and motivation" and
// "Implementation breakdown"; PR #32162 report, item 1: every unique miss is
// copied as a complete entry).  Here the plan kernel has already written, per
// row b, miss_count[b] pairs (host row, device row); this kernel moves them.
//
// The work is flattened over every 16-byte chunk of every miss of the call:
// each workgroup takes a contiguous range of chunks so a wave reads whole
// rows, each lane keeps kCopyUnroll 16-byte host loads in flight (the host
// link needs many outstanding reads), and rows land in HBM with non-temporal
// stores.  The row of a chunk is found by a search over the per-row prefix
// of miss counts held in LDS.
#include "copy.h"
#include "device_common.h"

namespace hisparse {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int NT, int U>
__global__ __launch_bounds__(NT) void miss_copy(CopyArgs a) {
  extern __shared__ int pre[];  // [batch + 1]
  __shared__ int scan[NT / kWave + 1];
  const int tid = threadIdx.x;
  int running = 0;
  for (int base = 0; base < a.batch; base += NT) {
    const int b = base + tid;
    const int v = b < a.batch ? min(max(a.miss_count[b], 0), a.cap) : 0;
    int tot;
    const int x = block_exclusive_scan<NT>(v, scan, &tot);
    if (b < a.batch) pre[b] = running + x;
    running += tot;
  }
  if (tid == 0) pre[a.batch] = running;
  __syncthreads();

  const int64_t total = static_cast<int64_t>(running) * a.unit16;
  const int64_t per = (total + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = per * blockIdx.x;
  const int64_t c1 = c0 + per < total ? c0 + per : total;
  const double inv_unit = 1.0 / static_cast<double>(a.unit16);

  for (int64_t c = c0 + tid; c < c1; c += static_cast<int64_t>(NT) * U) {
    u32x4 v[U];
    u32x4* dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cu = c + static_cast<int64_t>(u) * NT;
      dst[u] = nullptr;
      if (cu >= c1) continue;
      // miss index g and 16-byte offset within the row
      int64_t g = static_cast<int64_t>(static_cast<double>(cu) * inv_unit);
      int64_t off = cu - g * a.unit16;
      if (off < 0) {
        --g;
        off += a.unit16;
      } else if (off >= a.unit16) {
        ++g;
        off -= a.unit16;
      }
      // row b with pre[b] <= g < pre[b + 1]
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= g) lo = mid; else hi = mid - 1;
      }
      const int j = static_cast<int>(g - pre[lo]);
      const size_t slot = static_cast<size_t>(lo) * a.cap + j;
      const int64_t srow = a.src[slot];
      const int64_t drow = a.dst[slot];
      if (srow < 0 || srow >= a.src_rows || drow < 0 || drow >= a.dst_rows) {
        if (off == 0) raise_error(a.err, HISPARSE_ERR_BAD_PLAN);
        continue;
      }
      const u32x4* sp = reinterpret_cast<const u32x4*>(a.host + srow * a.unit_bytes) + off;
      dst[u] = reinterpret_cast<u32x4*>(a.dev + drow * a.unit_bytes) + off;
#if HISPARSE_COPY_NT_LOAD
      v[u] = __builtin_nontemporal_load(sp);
#else
      v[u] = *sp;
#endif
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u] != nullptr) __builtin_nontemporal_store(v[u], dst[u]);
  }
}

}  // namespace

hipError_t launch_miss_copy(const CopyArgs& a, hipStream_t s) {
  static_assert((HISPARSE_MAX_BATCH + 1 + kCopyThreads / kWave + 1) * sizeof(int) <= 64 * 1024,
                "the largest batch's prefix and the scan scratch fit the default LDS");
  const size_t lds = (static_cast<size_t>(a.batch) + 1) * sizeof(int);
  const int blocks = a.unit_bytes >= kCopyPageUnit ? kCopyBlocks : kCopyRowBlocks;
  hipLaunchKernelGGL((miss_copy<kCopyThreads, kCopyUnroll>), dim3(blocks),
                     dim3(kCopyThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace hisparse
