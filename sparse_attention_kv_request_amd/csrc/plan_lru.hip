// Single-step LRU swap-in: lookup, dedup, victim selection and commit.
//
// One workgroup resolves one batch row, i.e. one (request, layer) cache
// instance (PR #20343 summary, "Implementation breakdown": hash lookup,
// hit/miss handling and LRU update; "SGLang HiSparse" blog, section 2.1).
//
// Layout choices (gfx950):
//  * The token->slot lookup of the pages is a join computed per call: the
//    row's distinct keys go into an LDS hash (which also deduplicates them),
//    and every slot's resident key -- read in full anyway, the victims need
//    it -- is looked up there.  No key->slot table is kept in HBM, so a call
//    makes no random probe reads and no scattered key->slot stores; the
//    slot->key array, read once per call with the order, is the whole map.
//  * The LRU order is an explicit slot list, least recent first, ties in
//    slot order.  A call moves every slot it used to the back in slot order,
//    so the list always equals the (timestamp, slot) order and the victims
//    are its first m unused slots: two block scans, no sort.
//  * Duplicates inside the row are found with an LDS hash (first occurrence
//    wins by atomicMin of the position); misses are ranked in position order
//    with block scans, so the result does not depend on thread timing.
#include "internal.h"

// Opt-in instrumentation, a separate build (-DHISPARSE_PHASE_CLOCKS=1, see
// phase_clocks.py): every workgroup of a token-mode plan launch records the
// 100 MHz wall clock at its phase boundaries, and hisparse_phase_clocks()
// copies the last launch's stamps out.  The default build records nothing.
#ifndef HISPARSE_PHASE_CLOCKS
#define HISPARSE_PHASE_CLOCKS 0
#endif
#if HISPARSE_PHASE_CLOCKS
constexpr int kClockRows = 4096;   // workgroups recorded
constexpr int kClockStamps = 10;   // per workgroup: 9 stamps, then the row's miss count
__device__ long long g_phase_clock[kClockRows * kClockStamps];
#define PHASE_CLOCK(i, v)                                                        \
  do {                                                                          \
    if (threadIdx.x == 0 && blockIdx.x < kClockRows)                            \
      g_phase_clock[blockIdx.x * kClockStamps + (i)] = (v);                     \
  } while (0)
extern "C" int hisparse_phase_clocks(long long* out_h, int n) {
  if (n < 0 || n > kClockRows * kClockStamps) return -1;
  return hipMemcpyFromSymbol(out_h, HIP_SYMBOL(g_phase_clock), n * sizeof(long long)) == hipSuccess
             ? 0 : -1;
}
#else
#define PHASE_CLOCK(i, v) \
  do {                    \
  } while (0)
#endif

namespace hisparse {

namespace {

// Row checks shared by the single-step kernels: returns nonzero (and the
// error bit) when the row must be rejected.  Uniform over the block.
template <int NT>
__device__ __forceinline__ uint32_t row_check(const PlanArgs& a, int b, int r, int sl) {
  if (!(r >= 0 && r < a.R && sl >= 0 && sl <= a.N)) return HISPARSE_ERR_BAD_ROW;
  int dup = 0;
  for (int bb = threadIdx.x; bb < a.batch; bb += NT) dup |= (bb != b && a.req[bb] == r);
  return __syncthreads_or(dup) ? HISPARSE_ERR_DUP_REQUEST : 0u;
}

template <int NT>
__device__ void reject_row(const PlanArgs& a, int b, int entries, uint32_t code, bool page_mode) {
  int32_t* out = a.out_locs + static_cast<size_t>(b) * entries;
  for (int i = threadIdx.x; i < entries; i += NT) out[i] = -1;
  if (page_mode) {
    int32_t* pt = a.page_table + static_cast<size_t>(b) * a.H;
    for (int j = threadIdx.x; j < a.H; j += NT) pt[j] = -1;
  }
  if (threadIdx.x == 0) {
    a.miss_count[b] = 0;
    if (page_mode) a.num_pages[b] = 0;
    raise_error(a.err, code);
  }
}

// Order positions tid*EPH .. tid*EPH+EPH-1 (slots o[e]) that this call did
// not use (`used` holds the hit slots), as a mask over e.  A position's rank
// among all available positions in order is the thread's base rank plus the
// count of mask bits below it.
template <int EPH>
__device__ __forceinline__ uint32_t lru_available(const int (&o)[EPH], const uint32_t* used) {
  static_assert(EPH <= 32, "one mask bit per position");
  uint32_t avail = 0u;
#pragma unroll
  for (int e = 0; e < EPH; ++e)
    if (o[e] >= 0 && !bit_test(used, o[e])) avail |= 1u << e;
  return avail;
}

// Commit of the m misses into the first m available order positions and
// rewrite of the order.  `o` holds order positions tid*EPH .. tid*EPH+EPH-1;
// `avail` comes from lru_available, `rank0` (the rank of this thread's first
// available position) from a scan over its counts.  `used` has the
// bits of the slots hit by this call; victims are added to it.  Miss j (key
// miss_key[j]) goes to vslot[j].
template <int NT, int EPH>
__device__ void lru_commit(const PlanArgs& a, int b, int r, int now, int m,
                           const int (&o)[EPH], uint32_t avail, int rank0,
                           uint32_t* used, const int32_t* miss_key, int32_t* vslot, int* scan,
                           int32_t* sk, int32_t* tsq, int16_t* ord,
                           const uint32_t* mbits, const int32_t* mwpre, const int (&oldk)[EPH]) {
  const int tid = threadIdx.x;
  // commit: the owner of a victim slot replaces its key
  int32_t* msrc = a.miss_src + static_cast<size_t>(b) * a.cap;
  int32_t* mdst = a.miss_dst + static_cast<size_t>(b) * a.cap;
  int32_t* mvic = a.victim + static_cast<size_t>(b) * a.cap;
  int j = rank0;  // rank of the next available position
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    if (!(avail >> e & 1u)) continue;
    if (j < m) {
      const int s = o[e];
      const int32_t key = miss_key[j];
      // slot_key[s] as the call found it (no other thread writes slot s):
      // fetched at kernel start, or here where 32 slots per thread leave no
      // registers for it
      const int32_t old = EPH < 32 ? oldk[e] : sk[s];
      sk[s] = key;
      tsq[s] = now;
      vslot[j] = s;
      bit_set_atomic(used, s);
      msrc[j] = r * a.nkeys + key;
      mdst[j] = r * a.rows + s;
      mvic[j] = old;
      if (mbits != nullptr) {
        const size_t c = static_cast<size_t>(b) * a.ccap + bitmap_rank(mbits, mwpre, key);
        a.copy_src[c] = r * a.nkeys + key;
        a.copy_dst[c] = r * a.rows + s;
      }
    }
    ++j;
  }
  __syncthreads();
  // untouched slots keep their relative order at the front
  j = rank0;
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    if (!(avail >> e & 1u)) continue;
    if (j >= m) ord[j - m] = static_cast<int16_t>(o[e]);
    ++j;
  }
  // slots used by this call (timestamp = now) go to the back in slot order.
  // Thread w owns bitmap word w (Hw <= NT); each wave that owns words takes
  // its prefix from wave scans over all the words (Hw / 64 of them), so no
  // block barrier is needed here.
  static_assert(HISPARSE_MAX_HOT / 32 <= NT, "one bitmap word per thread");
  (void)scan;
  const int lane = tid & (kWave - 1);
  const int wbase = tid - lane;  // first word of this wave
  if (wbase < a.Hw) {            // uniform over the wave
    int before = 0, ntouched = 0;
    for (int c0 = 0; c0 < a.Hw; c0 += kWave) {
      const int w = c0 + lane;
      const uint32_t n = w < a.Hw ? static_cast<uint32_t>(__popc(used[w])) : 0u;
      const uint32_t incl = wave_incl_scan(n);
      if (c0 == wbase) before = ntouched + static_cast<int>(incl - n);
      ntouched += static_cast<int>(__builtin_amdgcn_readlane(incl, kWave - 1));
    }
    if (tid < a.Hw) {
      int pos = a.H - ntouched + before;
      uint32_t bits = used[tid];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1u;
        ord[pos++] = static_cast<int16_t>(tid * 32 + bit);
      }
    }
  }
}

// -------------------------------------------------------------------------
// Token mode
// -------------------------------------------------------------------------
template <int NT, int EPT, int EPH>
__global__ __launch_bounds__(NT) void lru_token_plan(PlanArgs a) {
  extern __shared__ uint32_t lds[];
  // Every distinct key of the row gets one entry of kmin / kres: with key
  // bitmaps (sw > 0, the request's keys fit a bitmap in LDS) the entry is the
  // key's rank among the row's keys -- popcounts over the bitmap, a perfect
  // hash built per call, no probing; otherwise an LDS hash bucket.
  const int sw = a.sort_words;
  const int T = a.hash_size;                                       // hash path only
  const int D = sw ? a.K : T;                                      // entries
  uint32_t* used = lds;                                            // [Hw]
  int32_t* miss_key = reinterpret_cast<int32_t*>(used + a.Hw);     // [K]
  int32_t* vslot = miss_key + a.K;                                 // [K]
  int* scan = vslot + a.K;                                         // [2*NT/64]
  uint32_t* mbits = reinterpret_cast<uint32_t*>(scan + 2 * NT / kWave);  // [sw] miss keys
  int32_t* mwpre = reinterpret_cast<int32_t*>(mbits + sw);              // [sw]
  uint32_t* rbits = reinterpret_cast<uint32_t*>(mwpre + sw);            // [sw] row keys
  int32_t* rwpre = reinterpret_cast<int32_t*>(rbits + sw);              // [sw]
  uint32_t* kmin = reinterpret_cast<uint32_t*>(rwpre + sw);  // [D] first position of the key
  int32_t* kres = reinterpret_cast<int32_t*>(kmin + D);      // [D] hit slot, then -(miss rank+1)
  uint32_t* hkey = reinterpret_cast<uint32_t*>(kres + D);    // [T] hash path: key + 1

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  PHASE_CLOCK(0, wall_clock64());
  const int r = a.req[b];
  const int sl = a.seq[b];
  // Loads that need only the instance go out before the row checks so they
  // share one round trip (a rejected row discards them).
  const size_t q = static_cast<size_t>(a.layer) * a.R + (r >= 0 && r < a.R ? r : 0);
  int32_t* sk = a.slot_key + q * a.H;
  int32_t* tsq = a.ts + q * a.H;
  int16_t* ord = a.order + q * a.H;
  const int now = a.ctrl[2 * q];
  int o[EPH];
  int rkey[EPH];  // resident keys of slots tid*EPH + e: the join's probe side
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    const int k = tid * EPH + e;
    o[e] = k < a.H ? static_cast<int>(ord[k]) : -1;
    rkey[e] = k < a.H ? sk[k] : kEmpty;
  }
  const int32_t* row = a.topk + static_cast<size_t>(b) * a.K;
  int32_t raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    raw[e] = i < a.K ? row[i] : -1;
  }
  // The LDS tables are cleared before the row checks, whose barrier then
  // publishes the cleared state (a rejected row just returns).
  for (int i = tid; i < D; i += NT) {
    kmin[i] = 0xFFFFFFFFu;
    kres[i] = -1;
  }
  if (sw) {
    for (int i = tid; i < sw; i += NT) {
      mbits[i] = 0u;
      rbits[i] = 0u;
    }
  } else {
    for (int i = tid; i < T; i += NT) hkey[i] = 0u;
  }
  const uint32_t code = row_check<NT>(a, b, r, sl);
  if (code) {
    reject_row<NT>(a, b, a.K, code, false);
    return;
  }
  PHASE_CLOCK(1, wall_clock64());
  // 1. validate every entry.  Entries among the newest ext tokens resolve to
  // their ring row instead (the extra-page lookup, before the hash lookup)
  // and stay out of the cache.
  int32_t tok[EPT];
  int idx[EPT];   // the entry's key entry (rank or bucket)
  int ring[EPT];
  bool bad_index = false;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int32_t t = raw[e];
    const bool valid = t >= 0 && t < sl;
    bad_index |= (!valid && t != -1);
    const bool extra = valid && t >= sl - a.ext;
    ring[e] = extra ? a.ext_base + t % a.ext : -1;
    tok[e] = valid && !extra ? t : -1;
    idx[e] = 0;
  }
  // the resident key of every order position: the victims' old keys for the
  // plan (a gather in LRU order, only needed at the commit)
  int oldk[EPH];
  if constexpr (EPH < 32) {
#pragma unroll
    for (int e = 0; e < EPH; ++e) oldk[e] = o[e] >= 0 ? sk[o[e]] : kEmpty;
  }

  PHASE_CLOCK(2, wall_clock64());
  // 2. dedup and the join.  kmin takes each key's first position (atomicMin);
  // the owner of each resident slot whose key the row names writes the slot
  // into the key's kres entry and marks the slot used now.
  uint32_t hitmask = 0u;
  if (sw) {
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (tok[e] >= 0) bit_set_atomic(rbits, tok[e]);
    __syncthreads();
    bitmap_word_prefix<NT>(rbits, rwpre, sw, scan);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (tok[e] < 0) continue;
      idx[e] = bitmap_rank(rbits, rwpre, tok[e]);
      atomicMin(&kmin[idx[e]], static_cast<uint32_t>(tid * EPT + e));
    }
#pragma unroll
    for (int e = 0; e < EPH; ++e) {
      const int32_t k = rkey[e];
      if (k < 0 || !bit_test(rbits, k)) continue;
      const int s = tid * EPH + e;
      kres[bitmap_rank(rbits, rwpre, k)] = s;
      hitmask |= 1u << e;
      tsq[s] = now;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (tok[e] < 0) continue;
      idx[e] = hash_insert(hkey, T, tok[e]);
      atomicMin(&kmin[idx[e]], static_cast<uint32_t>(tid * EPT + e));
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPH; ++e) {
      if (rkey[e] < 0) continue;
      const int h = hash_find(hkey, T, rkey[e]);
      if (h < 0) continue;
      const int s = tid * EPH + e;
      kres[h] = s;
      hitmask |= 1u << e;
      tsq[s] = now;
    }
  }
  // the used set of the hit slots, per word by lane shuffles (this thread's
  // slots are consecutive)
  store_slot_words<EPH>(used, a.Hw, hitmask);
  __syncthreads();

  PHASE_CLOCK(3, wall_clock64());
  // 3. representatives (first occurrences) take their key's result; misses
  // go into the miss-key bitmap.  One scan then ranks the misses (position
  // order), the available order positions (order) and the miss keys' bitmap
  // words (key order): misses and available positions share one word (at
  // most 8192 and 32768).
  bool rep[EPT];
  int slot[EPT];
  int nmiss = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    rep[e] = tok[e] >= 0 && kmin[idx[e]] == static_cast<uint32_t>(tid * EPT + e);
    slot[e] = rep[e] ? kres[idx[e]] : -1;
    if (rep[e] && slot[e] < 0) {
      ++nmiss;
      if (sw) bit_set_atomic(mbits, tok[e]);
    }
  }
  if (sw) __syncthreads();  // the scan below counts the miss bitmap
  const uint32_t avail = lru_available<EPH>(o, used);
  const int navail = __popc(avail);
  const int wpt = (sw + NT - 1) / NT;
  const int w0 = tid * wpt;
  int nbits = 0;
  for (int w = w0; w < w0 + wpt && w < sw; ++w) nbits += __popc(mbits[w]);
  uint32_t x_pre, y_pre, x_tot, y_tot;
  block_exclusive_scan2<NT>(static_cast<uint32_t>(nmiss) | (static_cast<uint32_t>(navail) << 16),
                            static_cast<uint32_t>(nbits), scan, &x_pre, &y_pre, &x_tot, &y_tot);
  const int m = static_cast<int>(x_tot & 0xffffu);
  int j = static_cast<int>(x_pre & 0xffffu);
  const int rank0 = static_cast<int>(x_pre >> 16);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (rep[e] && slot[e] < 0) {
      kres[idx[e]] = -(j + 1);
      miss_key[j] = tok[e];
      ++j;
    }
  }
  int wp = static_cast<int>(y_pre);
  for (int w = w0; w < w0 + wpt && w < sw; ++w) {
    mwpre[w] = wp;
    wp += __popc(mbits[w]);
  }
  __syncthreads();
  PHASE_CLOCK(4, wall_clock64());

  // 4. victims, commit, new order
  lru_commit<NT, EPH>(a, b, r, now, m, o, avail, rank0, used, miss_key, vslot, scan, sk, tsq,
                      ord, sw ? mbits : nullptr, mwpre, oldk);
  __syncthreads();
  PHASE_CLOCK(5, wall_clock64());

  // 5. outputs
  int32_t* out = a.out_locs + static_cast<size_t>(b) * a.K;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    if (i >= a.K) continue;
    int loc = ring[e] >= 0 ? r * a.rows + ring[e] : -1;
    if (tok[e] >= 0) {
      const int v = kres[idx[e]];
      loc = r * a.rows + (v >= 0 ? v : vslot[-v - 1]);
    }
    out[i] = loc;
  }
  if (tid == 0) {
    a.miss_count[b] = m;
    a.ctrl[2 * q] = now + 1;
  }
  if (bad_index) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
  PHASE_CLOCK(6, wall_clock64());
  PHASE_CLOCK(9, m);
  if (a.fuse_copy) {
    __syncthreads();  // the row's copy list, written above by this workgroup
    PHASE_CLOCK(7, wall_clock64());
    const size_t lb = sw ? static_cast<size_t>(b) * a.ccap : static_cast<size_t>(b) * a.cap;
    copy_own_row<NT>(a, (sw ? a.copy_src : a.miss_src) + lb, (sw ? a.copy_dst : a.miss_dst) + lb,
                     m);
#if HISPARSE_PHASE_CLOCKS
    __syncthreads();  // every wave's last loads returned
    PHASE_CLOCK(8, wall_clock64());
#endif
  }
}

// -------------------------------------------------------------------------
// Page mode ("SGLang HiSparse" blog, sections 1.3 and 2.3)
// -------------------------------------------------------------------------
template <int NT, int EPT, int EPH>
__global__ __launch_bounds__(NT) void lru_page_plan(PlanArgs a) {
  extern __shared__ uint32_t lds[];
  const int npw = (a.nkeys + 31) / 32;
  uint32_t* pbits = lds;                                           // [npw] pages named
  int32_t* wpre = reinterpret_cast<int32_t*>(pbits + npw);         // [npw] pages before word
  uint32_t* used = reinterpret_cast<uint32_t*>(wpre + npw);        // [Hw]
  int32_t* pslot = reinterpret_cast<int32_t*>(used + a.Hw);        // [H] page list, then slot
  int32_t* miss_key = pslot + a.H;                                 // [H]
  int32_t* vslot = miss_key + a.H;                                 // [H]
  int* scan = vslot + a.H;                                         // [NT/64+1]

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int r = a.req[b];
  const int sl = a.seq[b];
  const size_t q = static_cast<size_t>(a.layer) * a.R + (r >= 0 && r < a.R ? r : 0);
  int32_t* sk = a.slot_key + q * a.H;
  int32_t* tsq = a.ts + q * a.H;
  int16_t* ord = a.order + q * a.H;
  const int now = a.ctrl[2 * q];
  int o[EPH];
  int rkey[EPH];  // resident pages of slots tid*EPH + e: the join's probe side
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    const int k = tid * EPH + e;
    o[e] = k < a.H ? static_cast<int>(ord[k]) : -1;
    rkey[e] = k < a.H ? sk[k] : kEmpty;
  }
  const int32_t* row = a.topk + static_cast<size_t>(b) * a.K;
  int32_t raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    raw[e] = i < a.K ? row[i] : -1;
  }
  // the page bitmap and used set are cleared before the row checks, whose
  // barrier then publishes them (a rejected row just returns)
  for (int i = tid; i < npw; i += NT) pbits[i] = 0u;
  for (int i = tid; i < a.Hw; i += NT) used[i] = 0u;
  const uint32_t code = row_check<NT>(a, b, r, sl);
  if (code) {
    reject_row<NT>(a, b, a.K, code, true);
    return;
  }
  int oldk[EPH];
#pragma unroll
  for (int e = 0; e < EPH; ++e) oldk[e] = o[e] >= 0 ? sk[o[e]] : kEmpty;

  // 1. tokens -> pages named by the row
  int32_t tok[EPT];
  bool bad_index = false;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int32_t t = raw[e];
    const bool valid = t >= 0 && t < sl;
    bad_index |= (!valid && t != -1);
    tok[e] = valid ? t : -1;
    if (valid) bit_set_atomic(pbits, t / a.P);
  }
  __syncthreads();

  // 2. distinct pages in ascending order
  const int wpt = (npw + NT - 1) / NT;
  const int w0 = tid * wpt;
  int cnt = 0;
  for (int w = w0; w < w0 + wpt && w < npw; ++w) cnt += __popc(pbits[w]);
  int npages;
  int pre = block_exclusive_scan<NT>(cnt, scan, &npages);
  if (npages > a.H) {  // uniform over the block
    if (bad_index) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
    reject_row<NT>(a, b, a.K, HISPARSE_ERR_PAGE_OVERFLOW, true);
    return;
  }
  for (int w = w0; w < w0 + wpt && w < npw; ++w) {
    wpre[w] = pre;
    uint32_t bits = pbits[w];
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1u;
      pslot[pre++] = w * 32 + bit;
    }
  }
  __syncthreads();

  // 3. the join: every resident page the row names is a hit; its entry in
  // the distinct-page list takes the slot (flagged), the slot is used now
  constexpr int32_t kHit = 1 << 30;  // pages < 2^18, slots < 2^12
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    const int p = rkey[e];
    if (p < 0 || !bit_test(pbits, p)) continue;
    const int s = tid * EPH + e;
    pslot[bitmap_rank(pbits, wpre, p)] = kHit | s;
    bit_set_atomic(used, s);
    tsq[s] = now;
  }
  __syncthreads();
  // rank the misses in page order
  int m = 0;
  for (int base = 0; base < npages; base += NT) {
    const int jp = base + tid;
    const bool active = jp < npages;
    const int x = active ? pslot[jp] : 0;
    const int p = x;
    const int s = x & kHit ? x & ~kHit : -1;
    const bool miss = active && s < 0;
    int round_misses;
    int jm = block_exclusive_scan<NT>(miss ? 1 : 0, scan, &round_misses) + m;
    if (active) {
      if (miss) {
        miss_key[jm] = p;
        pslot[jp] = -(jm + 1);
      } else {
        pslot[jp] = s;
      }
    }
    m += round_misses;
  }
  __syncthreads();

  // 4. victims, commit, new order (pages are already in ascending order)
  const uint32_t avail = lru_available<EPH>(o, used);
  int total_avail;
  const int rank0 = block_exclusive_scan<NT>(__popc(avail), scan, &total_avail);
  lru_commit<NT, EPH>(a, b, r, now, m, o, avail, rank0, used, miss_key, vslot, scan, sk, tsq,
                      ord, nullptr, nullptr, oldk);
  __syncthreads();

  // 5. outputs: page table, page count, token locations (page index, offset)
  int32_t* pt = a.page_table + static_cast<size_t>(b) * a.H;
  for (int jp = tid; jp < a.H; jp += NT) {
    int v = -1;
    if (jp < npages) {
      const int x = pslot[jp];
      v = r * a.rows + (x >= 0 ? x : vslot[-x - 1]);
    }
    pt[jp] = v;
  }
  int32_t* out = a.out_locs + static_cast<size_t>(b) * a.K;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    if (i >= a.K) continue;
    int loc = -1;
    if (tok[e] >= 0) {
      const int p = tok[e] / a.P;
      const uint32_t below = pbits[p >> 5] & ((1u << (p & 31)) - 1u);
      const int jp = wpre[p >> 5] + __popc(below);
      loc = jp * a.P + (tok[e] - p * a.P);
    }
    out[i] = loc;
  }
  if (tid == 0) {
    a.miss_count[b] = m;
    a.num_pages[b] = npages;
    a.ctrl[2 * q] = now + 1;
  }
  if (bad_index) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
}

template <typename K>
hipError_t launch_plan(K kernel, const PlanArgs& a, size_t lds, hipStream_t s) {
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, dim3(a.batch), dim3(kPlanThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

int hash_size_for(int entries, bool pow2) {
  // at least 2 buckets per entry: the next power of two (triangular probing)
  // or, where LDS is short, a multiple of 64 (linear probing)
  const int need = 2 * entries < 64 ? 64 : 2 * entries;
  if (!pow2) return ((need + 63) / 64) * 64;
  int t = 64;
  while (t < need) t *= 2;
  return t;
}

size_t lru_token_lds_bytes(const PlanArgs& a) {
  // used, miss_key, vslot, scan, four key bitmaps / prefixes, kmin + kres,
  // and the hash's key words when there are no bitmaps
  const size_t sw = static_cast<size_t>(a.sort_words);
  const size_t d = sw ? static_cast<size_t>(a.K) : static_cast<size_t>(a.hash_size);
  return (a.Hw + 2 * static_cast<size_t>(a.K) + 2 * kPlanThreads / kWave + 4 * sw + 2 * d +
          (sw ? 0 : static_cast<size_t>(a.hash_size))) * 4;
}

size_t lru_page_lds_bytes(const PlanArgs& a) {
  const size_t npw = (a.nkeys + 31) / 32;
  return (2 * npw + a.Hw + 3 * static_cast<size_t>(a.H) + kPlanThreads / kWave + 1) * 4;
}

// Entries per thread (EPT) and order positions per thread (EPH) are compile
// time so the per-thread arrays stay in registers.
#define HS_DISPATCH_EPH(KERNEL, EPTV)                                                 \
  if (a.H <= 4 * kPlanThreads)                                                        \
    return launch_plan(KERNEL<kPlanThreads, EPTV, 4>, a, lds, s);                     \
  if (a.H <= 8 * kPlanThreads)                                                        \
    return launch_plan(KERNEL<kPlanThreads, EPTV, 8>, a, lds, s);                     \
  if (a.H <= 16 * kPlanThreads)                                                       \
    return launch_plan(KERNEL<kPlanThreads, EPTV, 16>, a, lds, s);                    \
  return launch_plan(KERNEL<kPlanThreads, EPTV, 32>, a, lds, s);

hipError_t launch_lru_token_plan(const PlanArgs& a, hipStream_t s) {
  const size_t lds = lru_token_lds_bytes(a);
  if (a.K <= 2 * kPlanThreads) {
    HS_DISPATCH_EPH(lru_token_plan, 2)
  }
  HS_DISPATCH_EPH(lru_token_plan, 8)
}

hipError_t launch_lru_page_plan(const PlanArgs& a, hipStream_t s) {
  // page mode holds at most 4096 hot pages: four order positions per thread
  static_assert(kMaxPageModeHot <= 4 * kPlanThreads, "page-mode caches fit 4 slots per thread");
  const size_t lds = lru_page_lds_bytes(a);
  if (a.K <= 2 * kPlanThreads) return launch_plan(lru_page_plan<kPlanThreads, 2, 4>, a, lds, s);
  return launch_plan(lru_page_plan<kPlanThreads, 8, 4>, a, lds, s);
}

}  // namespace hisparse
