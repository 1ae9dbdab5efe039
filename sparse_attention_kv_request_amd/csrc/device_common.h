// Device helpers shared by the swap-in kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hisparse.h"

namespace hisparse {

constexpr int kWave = 64;
constexpr int32_t kEmpty = -1;

// Key words of the LDS working-set hash: (token + 1) in the low 28 bits, 0 =
// empty bucket; bits 28..31 record which speculative steps named the token.
constexpr uint32_t kKeyBits = 28;
constexpr uint32_t kKeyMask = (1u << kKeyBits) - 1u;

// Everything a plan (lookup / victim / commit) kernel needs.  One workgroup
// handles one batch row = one (request, layer) cache instance.  The
// key -> slot lookup is a join computed per call: the row's keys go into an
// LDS hash, and every resident key of the instance (slot_key, read in full
// anyway for the victims) is looked up in it, so no key -> slot table is kept.
struct PlanArgs {
  // persistent state of the layer's instances, instance q = layer * R + r
  int32_t* slot_key;    // [L*R][H]      slot -> key, -1 = empty
  int32_t* ts;          // [L*R][H]      LRU timestamp (-1 = empty)
  int16_t* order;       // [L*R][H]      LRU order of slots, least recent first
  uint32_t* refbits;    // [L*R][Hw]     CLOCK reference bits
  int32_t* ctrl;        // [L*R][2]      {LRU call counter, CLOCK hand}
  uint32_t* err;        // sticky error word
  int32_t R, H, Hw, K, S, N, P, nkeys, rows, layer;
  int32_t ext, ext_base;  // extra-row ring: E rows from row ext_base of each request
  int32_t admission;      // HISPARSE_ADMIT_* (multi-step overflow)
  // the call
  int32_t batch;
  const int32_t* req;
  const int32_t* seq;
  const int32_t* topk;
  int32_t* out_locs;
  int32_t* miss_count;
  int32_t* page_table;
  int32_t* num_pages;
  int32_t* miss_src;    // [batch][cap]
  int32_t* miss_dst;
  int32_t* victim;
  int32_t cap;
  int32_t hash_size;    // LDS hash buckets
  // copy list: the same misses in ascending host-row order (rows of one
  // request that are adjacent in host memory then share their 128-byte lines)
  int32_t* copy_src;    // [batch][ccap]
  int32_t* copy_dst;
  int32_t ccap;
  int32_t sort_words;   // words of the LDS miss bitmap; 0 = no copy list
  // fused copy: the plan workgroup moves its own row's misses
  const uint8_t* host;  // device-visible address of the layer's host tier
  uint8_t* dev;
  int64_t unit_bytes;
  int32_t unit16;
  int32_t fuse_copy;
};

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four row
// shifts inside each 16-lane row, then row 0's total broadcast into row 1
// (and row 2's into row 3), then the low half's total into the high half.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false); // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false); // row_bcast:31
  return x;
}

// Exclusive prefix sum over the NT threads of a workgroup.  `scratch` holds
// NT/64 ints of LDS.  Returns the exclusive prefix; *total receives the sum.
// Two barriers (the second keeps `scratch` intact until every wave has read
// it): every thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  static_assert(NT % kWave == 0 && NT / kWave <= kWave, "block shape");
  constexpr int kWaves = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(v)));
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  const int w = lane < kWaves ? scratch[lane] : 0;
  const int wi = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(w)));
  const int before = wid > 0 ? __builtin_amdgcn_readlane(wi, wid - 1) : 0;
  *total = __builtin_amdgcn_readlane(wi, kWaves - 1);
  __syncthreads();
  return before + incl - v;
}

// Two independent exclusive prefix sums over the workgroup in one pass (each
// word may pack narrower fields whose sums cannot carry into each other).
// `scratch` holds 2*NT/64 ints of LDS.  Two barriers; every thread must call it.
template <int NT>
__device__ __forceinline__ void block_exclusive_scan2(uint32_t x, uint32_t y, int* scratch,
                                                      uint32_t* x_pre, uint32_t* y_pre,
                                                      uint32_t* x_tot, uint32_t* y_tot) {
  constexpr int kWaves = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t xi = wave_incl_scan(x);
  const uint32_t yi = wave_incl_scan(y);
  uint32_t* sc = reinterpret_cast<uint32_t*>(scratch);
  if (lane == kWave - 1) {
    sc[wid] = xi;
    sc[kWaves + wid] = yi;
  }
  __syncthreads();
  const uint32_t wx = wave_incl_scan(lane < kWaves ? sc[lane] : 0u);
  const uint32_t wy = wave_incl_scan(lane < kWaves ? sc[kWaves + lane] : 0u);
  *x_pre = (wid > 0 ? __builtin_amdgcn_readlane(wx, wid - 1) : 0u) + xi - x;
  *y_pre = (wid > 0 ? __builtin_amdgcn_readlane(wy, wid - 1) : 0u) + yi - y;
  *x_tot = __builtin_amdgcn_readlane(wx, kWaves - 1);
  *y_tot = __builtin_amdgcn_readlane(wy, kWaves - 1);
  __syncthreads();
}

__device__ __forceinline__ bool bit_test(const uint32_t* bm, int i) {
  return (bm[i >> 5] >> (i & 31)) & 1u;
}
__device__ __forceinline__ void bit_set_atomic(uint32_t* bm, int i) {
  atomicOr(&bm[i >> 5], 1u << (i & 31));
}
__device__ __forceinline__ void bit_clear_atomic(uint32_t* bm, int i) {
  atomicAnd(&bm[i >> 5], ~(1u << (i & 31)));
}

// Bucket of a token in an LDS hash of `size` buckets (multiplicative hash
// scaled to the table size, any size).
__device__ __forceinline__ int hash_bucket(int32_t t, int size) {
  const uint32_t h = static_cast<uint32_t>(t) * 2654435761u;
  return static_cast<int>((static_cast<uint64_t>(h) * static_cast<uint32_t>(size)) >> 32);
}

// Next bucket of a probe sequence: a table of a power-of-two size walks the
// triangular offsets 1, 2, 3, ... (bucket h0 + i(i+1)/2, which visits every
// bucket and breaks up the clusters of linear probing, so the longest probe
// -- what a wave waits for -- stays short); any other size walks linearly.
__device__ __forceinline__ int hash_next(int h, int& step, int size) {
  if ((size & (size - 1)) == 0) return (h + ++step) & (size - 1);
  return h + 1 == size ? 0 : h + 1;
}

// Inserts token t (0 <= t < 2^28 - 1) into the open-addressing LDS table
// `keys` (0 = empty, key + 1 in the low 28 bits) and returns its bucket.  The
// table is sized above the number of distinct keys, so the probe terminates.
// (One entry at a time: issuing a thread's probes together measured slower.)
__device__ __forceinline__ int hash_insert(uint32_t* keys, int size, int32_t t) {
  const uint32_t want = static_cast<uint32_t>(t) + 1u;
  int h = hash_bucket(t, size);
  int step = 0;
  while (true) {
    const uint32_t old = atomicCAS(&keys[h], 0u, want);
    if (old == 0u || (old & kKeyMask) == want) return h;
    h = hash_next(h, step, size);
  }
}

// Bucket of token t in the LDS table `keys`, or -1 when t is not in it (key
// bits only; the step bits above them are ignored).  Follows the probe
// sequence of hash_insert; terminates: the table always has empty buckets.
__device__ __forceinline__ int hash_find(const uint32_t* keys, int size, int32_t t) {
  const uint32_t want = static_cast<uint32_t>(t) + 1u;
  int h = hash_bucket(t, size);
  int step = 0;
  while (true) {
    const uint32_t k = keys[h] & kKeyMask;
    if (k == want) return h;
    if (k == 0u) return -1;
    h = hash_next(h, step, size);
  }
}

// Value words of the LDS hash during the lookup: the low 16 bits take the
// first position of the key in the row (atomicMin of kNoHit | position), the
// high 16 bits the slot of a resident key found by the join (atomicAnd), or
// all ones when the key is not resident.  The two halves are written by
// different threads without a barrier between them.
constexpr uint32_t kNoHit = 0xFFFF0000u;
static_assert(HISPARSE_MAX_WORKING_SET < 0xFFFF && HISPARSE_MAX_HOT < 0xFFFF,
              "positions and slots fit the halves of a value word");
__device__ __forceinline__ void mark_hit(uint32_t* vals, int h, int slot) {
  atomicAnd(&vals[h], (static_cast<uint32_t>(slot) << 16) | 0xFFFFu);
}
__device__ __forceinline__ int first_pos(uint32_t v) { return static_cast<int>(v & 0xFFFFu); }
__device__ __forceinline__ int hit_slot(uint32_t v) {  // -1 when not resident
  return (v >> 16) == 0xFFFFu ? -1 : static_cast<int>(v >> 16);
}

// Thread t holds the EPH consecutive slots t*EPH .. t*EPH+EPH-1 and a mask
// of which of them to mark: the 32/EPH lanes that share a bitmap word OR
// their masks together (lane shuffles, no LDS atomics) and the first of them
// stores the word.  Every lane of the wave must call it.  Overwrites words
// [0, words) that the wave's slots cover.
template <int EPH>
__device__ __forceinline__ void store_slot_words(uint32_t* bm, int words, uint32_t mask) {
  static_assert(EPH >= 1 && EPH <= 32 && 32 % EPH == 0, "slots per thread divide a word");
  constexpr int kLanes = 32 / EPH;
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t v = mask << (EPH * (lane % kLanes) % 32);
#pragma unroll
  for (int d = 1; d < kLanes; d <<= 1) v |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), d));
  const int w = static_cast<int>(threadIdx.x) * EPH / 32;
  if (lane % kLanes == 0 && w < words) bm[w] = v;
}

// Exclusive prefix of set bits over a bitmap of `words` words: wpre[w] =
// bits set in words [0, w).  Threads own contiguous words.  Block-wide.
template <int NT>
__device__ __forceinline__ void bitmap_word_prefix(const uint32_t* bits, int32_t* wpre,
                                                   int words, int* scan) {
  const int wpt = (words + NT - 1) / NT;
  const int w0 = threadIdx.x * wpt;
  int cnt = 0;
  for (int w = w0; w < w0 + wpt && w < words; ++w) cnt += __popc(bits[w]);
  int total;
  int pre = block_exclusive_scan<NT>(cnt, scan, &total);
  for (int w = w0; w < w0 + wpt && w < words; ++w) {
    wpre[w] = pre;
    pre += __popc(bits[w]);
  }
}

// Rank of key k among the set bits of `bits` (after bitmap_word_prefix).
__device__ __forceinline__ int bitmap_rank(const uint32_t* bits, const int32_t* wpre, int k) {
  return wpre[k >> 5] + __popc(bits[k >> 5] & ((1u << (k & 31)) - 1u));
}

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bits) {
  atomicOr(err, bits);
}

#ifndef HISPARSE_FUSE_UNROLL
#define HISPARSE_FUSE_UNROLL 8
#endif

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// The fused copy of a swap call: the row's m misses, (host row, device row)
// pairs at src[0..m) / dst[0..m) that this workgroup has just written, moved
// by the whole workgroup in 16-byte chunks with HISPARSE_FUSE_UNROLL loads in
// flight per lane and non-temporal stores.  Every thread must call it after
// a barrier that follows the list's stores.
template <int NT>
__device__ void copy_own_row(const PlanArgs& a, const int32_t* src, const int32_t* dst, int m) {
  constexpr int U = HISPARSE_FUSE_UNROLL;
  const int64_t total = static_cast<int64_t>(m) * a.unit16;
  const double inv = 1.0 / static_cast<double>(a.unit16);
  for (int64_t c = threadIdx.x; c < total; c += static_cast<int64_t>(NT) * U) {
    u32x4 v[U];
    u32x4* d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t cu = c + static_cast<int64_t>(u) * NT;
      d[u] = nullptr;
      if (cu >= total) continue;
      // miss j and 16-byte offset within its row
      int64_t j = static_cast<int64_t>(static_cast<double>(cu) * inv);
      int64_t off = cu - j * a.unit16;
      if (off < 0) {
        --j;
        off += a.unit16;
      } else if (off >= a.unit16) {
        ++j;
        off -= a.unit16;
      }
      const int64_t srow = src[j];
      const int64_t drow = dst[j];
      v[u] = *(reinterpret_cast<const u32x4*>(a.host + srow * a.unit_bytes) + off);
      d[u] = reinterpret_cast<u32x4*>(a.dev + drow * a.unit_bytes) + off;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (d[u] != nullptr) __builtin_nontemporal_store(v[u], d[u]);
  }
}

}  // namespace hisparse
