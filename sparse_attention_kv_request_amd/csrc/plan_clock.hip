// Multi-step CLOCK swap-in: one working set over all speculative steps.
//
// PR #32162 report, "Implementation breakdown" item 1: the top-k rows of all
// MTP steps of a request are flattened, looked up once, their misses are
// deduplicated across steps, and one CLOCK update places them; "Risks and
// impact": once the misses exceed the cache, admission favours the recent
// steps while the data of the call stays exact (here: the rest go to
// per-request scratch rows).
//
// One workgroup per batch row.  The sequential CLOCK hand walk becomes two
// prefix selections over the circular slot order starting at the hand:
//   lap 1: unpinned slots with reference bit 0, in hand order;
//   lap 2 (only if lap 1 has too few): unpinned slots whose bit was 1.
// A slot the hand passes with bit 1 loses it; in lap-2 calls every unpinned
// bit is cleared.  This reproduces the textbook sweep exactly.
#include "internal.h"

namespace hisparse {

namespace {

template <int NT>
__device__ __forceinline__ uint32_t multistep_row_check(const PlanArgs& a, int b, int r, int sl) {
  if (!(r >= 0 && r < a.R && sl >= 0 && sl <= a.N)) return HISPARSE_ERR_BAD_ROW;
  int dup = 0;
  for (int bb = threadIdx.x; bb < a.batch; bb += NT) dup |= (bb != b && a.req[bb] == r);
  return __syncthreads_or(dup) ? HISPARSE_ERR_DUP_REQUEST : 0u;
}

template <int NT, int EPT, int EPH>
__global__ __launch_bounds__(NT) void clock_plan(PlanArgs a) {
  extern __shared__ uint32_t lds[];
  // Every distinct key of the working set gets one entry.  With key bitmaps
  // (sw > 0: the request's keys fit a bitmap in LDS) the entry is the key's
  // rank among the working set's keys -- popcounts over the bitmap, a perfect
  // hash built per call -- with kmin (first position, then the key) and kres
  // (hit slot + 1 | step bits << 16, then the key's row).  Otherwise an LDS
  // hash: hkey (key + 1 | step bits << 28) and hval (first position | hit
  // slot << 16, then the row) per bucket.
  const int sw = a.sort_words;
  const int T = a.hash_size;
  const int E = a.S * a.K;
  const int D = sw ? E : T;
  uint32_t* pinned = lds;                                        // [Hw]
  uint32_t* refl = pinned + a.Hw;                                // [Hw] reference bits
  int* scan = reinterpret_cast<int*>(refl + a.Hw);               // [NT/64+1]
  uint32_t* mbits = reinterpret_cast<uint32_t*>(scan + NT / kWave + 1);  // [sw] miss keys
  int32_t* mwpre = reinterpret_cast<int32_t*>(mbits + sw);              // [sw]
  uint32_t* rbits = reinterpret_cast<uint32_t*>(mwpre + sw);            // [sw] working-set keys
  int32_t* rwpre = reinterpret_cast<int32_t*>(rbits + sw);              // [sw]
  uint32_t* kmin = reinterpret_cast<uint32_t*>(rwpre + sw);  // [D] direct: first pos, then key
  uint32_t* val = kmin + D;                                  // [D] kres, or hval
  uint32_t* hkey = kmin;                                     // [T] hash path: key words
  int16_t* miss_i = reinterpret_cast<int16_t*>(val + D);     // [E] entry of admitted miss j
  __shared__ int s_cnt[HISPARSE_MAX_STEPS];
  __shared__ int s_klast;
  __shared__ int s_last_slot;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int r = a.req[b];
  const int sl = a.seq[b];
  // Loads that need only the instance go out before the row checks so they
  // share one round trip (a rejected row discards them).
  const size_t q = static_cast<size_t>(a.layer) * a.R + (r >= 0 && r < a.R ? r : 0);
  int32_t* sk = a.slot_key + q * a.H;
  uint32_t* refq = a.refbits + q * a.Hw;
  const int hand = a.ctrl[2 * q + 1];
  const int32_t* row = a.topk + static_cast<size_t>(b) * E;
  int32_t raw[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    raw[e] = i < E ? row[i] : -1;
  }
  const uint32_t ref_word = tid < a.Hw ? refq[tid] : 0u;  // Hw <= NT
  // The LDS tables, bitmaps and counters are set up before the row checks,
  // whose barrier then publishes them (a rejected row just returns).
  for (int i = tid; i < D; i += NT) {
    kmin[i] = sw ? 0xFFFFFFFFu : 0u;
    val[i] = sw ? 0u : 0xFFFFFFFFu;
  }
  if (tid < a.Hw) {
    pinned[tid] = 0u;
    refl[tid] = ref_word;
  }
  for (int i = tid; i < sw; i += NT) {
    mbits[i] = 0u;
    rbits[i] = 0u;
  }
  if (tid < HISPARSE_MAX_STEPS) s_cnt[tid] = 0;
  const uint32_t code = multistep_row_check<NT>(a, b, r, sl);
  if (code) {
    int32_t* out = a.out_locs + static_cast<size_t>(b) * E;
    for (int i = tid; i < E; i += NT) out[i] = -1;
    if (tid == 0) {
      a.miss_count[b] = 0;
      raise_error(a.err, code);
    }
    return;
  }
  // circular sweep positions of this thread and their slot->key words (in
  // slot order from the hand, so coalesced): the join's probe side, and the
  // victims' old keys for the plan
  // sweep position tid*EPH + e is slot (hand + position) mod H, -1 past H
  const auto sl_of = [&](int e) {
    const int k = tid * EPH + e;
    const int s = hand + k;
    return k < a.H ? (s >= a.H ? s - a.H : s) : -1;
  };
  int oldk[EPH];
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    const int s = sl_of(e);
    oldk[e] = s >= 0 ? sk[s] : kEmpty;
  }

  // 1. flatten [S][K] step-major.  Entries among the newest ext tokens
  // resolve to their ring row (the extra-page lookup) and stay out of the
  // working set.
  int32_t tok[EPT];
  int idx[EPT];  // the entry's key entry (rank or bucket)
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

  // 2. dedup with first positions and step bits, and the join: each resident
  // key the working set names is a hit, pinned and referenced.
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
      const int i = tid * EPT + e;
      idx[e] = bitmap_rank(rbits, rwpre, tok[e]);
      atomicMin(&kmin[idx[e]], static_cast<uint32_t>(i));
      atomicOr(&val[idx[e]], 1u << (16 + i / a.K));
    }
#pragma unroll
    for (int e = 0; e < EPH; ++e) {
      const int32_t k = oldk[e];
      if (k < 0 || !bit_test(rbits, k)) continue;
      atomicOr(&val[bitmap_rank(rbits, rwpre, k)], static_cast<uint32_t>(sl_of(e) + 1));
      bit_set_atomic(pinned, sl_of(e));
      bit_set_atomic(refl, sl_of(e));
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (tok[e] < 0) continue;
      const int i = tid * EPT + e;
      idx[e] = hash_insert(hkey, T, tok[e]);
      atomicMin(&val[idx[e]], kNoHit | static_cast<uint32_t>(i));
      atomicOr(&hkey[idx[e]], 1u << (kKeyBits + i / a.K));
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPH; ++e) {
      if (oldk[e] < 0) continue;
      const int h = hash_find(hkey, T, oldk[e]);
      if (h < 0) continue;
      mark_hit(val, h, sl_of(e));
      bit_set_atomic(pinned, sl_of(e));
      bit_set_atomic(refl, sl_of(e));
    }
  }
  __syncthreads();

  // 3. representatives (first occurrences) take their key's result: a hit's
  // slot becomes its row; a miss's admission priority under overflow comes
  // from the steps that name it (latest step, number of steps, or none).
  bool rep[EPT];
  int slot[EPT];
  int packed = 0;  // misses | hits << 16
  int last[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t pos = static_cast<uint32_t>(tid * EPT + e);
    last[e] = 0;
    slot[e] = -1;
    rep[e] = false;
    if (tok[e] < 0) continue;
    const uint32_t v = val[idx[e]];
    uint32_t steps;
    if (sw) {
      rep[e] = kmin[idx[e]] == pos;
      slot[e] = static_cast<int>(v & 0xFFFFu) - 1;
      steps = v >> 16;
    } else {
      rep[e] = first_pos(v) == static_cast<int>(pos);
      slot[e] = hit_slot(v);
      steps = hkey[idx[e]] >> kKeyBits;
    }
    if (!rep[e]) {
      slot[e] = -1;
      continue;
    }
    if (slot[e] >= 0) {
      packed += 1 << 16;
    } else {
      last[e] = a.admission == HISPARSE_ADMIT_RECENT     ? 31 - __clz(steps)
                : a.admission == HISPARSE_ADMIT_FREQUENT ? __popc(steps) - 1
                                                         : 0;
      atomicAdd(&s_cnt[last[e]], 1);
      if (sw) bit_set_atomic(mbits, tok[e]);
      packed += 1;
    }
  }
  int tot;
  const int pre = block_exclusive_scan<NT>(packed, scan, &tot);
  // the scan's barriers end every read of the dedup words: representatives
  // now store their hit's row, and (direct path) the key in place of the
  // first position
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (!rep[e]) continue;
    if (slot[e] >= 0) val[idx[e]] = static_cast<uint32_t>(slot[e]);
    if (sw) kmin[idx[e]] = static_cast<uint32_t>(tok[e]);
  }
  const int m = tot & 0xffff;
  const int nhits = tot >> 16;
  const int room = a.H - nhits;

  // admitted misses: all, or (overflow) the highest priorities first
  int ma = m;
  int sstar = -1, take_eq = 0;
  if (m > room) {
    int acc = 0;
    for (int s = a.S - 1; s >= 0; --s) {
      if (acc + s_cnt[s] >= room) {
        sstar = s;
        take_eq = room - acc;
        break;
      }
      acc += s_cnt[s];
    }
  }
  bool adm[EPT];
  int ja[EPT];
  int jm[EPT];
  {
    int j = pre & 0xffff;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const bool miss = rep[e] && slot[e] < 0;
      jm[e] = miss ? j : -1;
      j += miss;
    }
  }
  if (m > room) {
    int neq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) neq += (jm[e] >= 0 && last[e] == sstar);
    int eq_tot;
    int req = block_exclusive_scan<NT>(neq, scan, &eq_tot);
    int nadm = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      adm[e] = false;
      if (jm[e] < 0) continue;
      if (last[e] > sstar) {
        adm[e] = true;
      } else if (last[e] == sstar) {
        adm[e] = req < take_eq;
        ++req;
      }
      nadm += adm[e];
    }
    int pa = block_exclusive_scan<NT>(nadm, scan, &ma);
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      ja[e] = pa;
      pa += adm[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      adm[e] = jm[e] >= 0;
      ja[e] = jm[e];
    }
  }
  int32_t* msrc = a.miss_src + static_cast<size_t>(b) * a.cap;
  int32_t* mdst = a.miss_dst + static_cast<size_t>(b) * a.cap;
  int32_t* mvic = a.victim + static_cast<size_t>(b) * a.cap;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (jm[e] < 0) continue;
    if (adm[e]) {
      miss_i[ja[e]] = static_cast<int16_t>(idx[e]);
    } else {  // scratch row H + jo, outside the cache
      const int jo = jm[e] - ja[e];
      val[idx[e]] = static_cast<uint32_t>(a.H + jo);
      msrc[ma + jo] = r * a.nkeys + tok[e];
      mdst[ma + jo] = r * a.rows + a.H + jo;
      mvic[ma + jo] = -1;
    }
  }
  __syncthreads();
  if (sw) {
    bitmap_word_prefix<NT>(mbits, mwpre, sw, scan);
    __syncthreads();
  }

  // 3. CLOCK sweep over circular positions k (slot = (hand + k) mod H).  The
  // first lap takes unpinned slots whose reference bit is clear (mask c1),
  // the second, if the first falls short, unpinned slots whose bit it
  // cleared (c2); a candidate's victim rank is its lap's base plus its rank
  // within the lap, and only ranks below ma are victims.
  static_assert(EPH <= 32, "one mask bit per position");
  constexpr uint32_t kAll = EPH == 32 ? ~0u : (1u << EPH) - 1u;
  uint32_t pin = 0u, rf = 0u;
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    const int s = sl_of(e);
    if (s < 0 || bit_test(pinned, s)) pin |= 1u << e;
    if (s >= 0 && bit_test(refl, s)) rf |= 1u << e;
  }
  const uint32_t c1 = ~pin & ~rf & kAll;
  uint32_t c2 = 0u;
  const int n1 = __popc(c1);
  int e1_tot;
  const int r1 = block_exclusive_scan<NT>(n1, scan, &e1_tot);
  int r2 = 0;  // second-lap rank of this thread's first c2 candidate, after e1_tot
  if (e1_tot >= ma) {
    if (ma > 0 && r1 <= ma - 1 && ma - 1 < r1 + n1) {  // this thread holds victim ma - 1
      int j = r1;
#pragma unroll
      for (int e = 0; e < EPH; ++e) {
        if (!(c1 >> e & 1u)) continue;
        if (j == ma - 1) {
          s_klast = tid * EPH + e;
          s_last_slot = sl_of(e);
        }
        ++j;
      }
    }
    __syncthreads();
    if (ma > 0) {  // the first lap cleared the bits it passed before the last victim
      const int klast = s_klast;
      const uint32_t c = ~pin & rf;
#pragma unroll
      for (int e = 0; e < EPH; ++e)
        if ((c >> e & 1u) && tid * EPH + e < klast) bit_clear_atomic(refl, sl_of(e));
    }
  } else {
    c2 = ~pin & rf;
    int e2_tot;
    r2 = e1_tot + block_exclusive_scan<NT>(__popc(c2), scan, &e2_tot);
    int j = r2;
#pragma unroll
    for (int e = 0; e < EPH; ++e) {
      if (!(c2 >> e & 1u)) continue;
      bit_clear_atomic(refl, sl_of(e));
      if (j == ma - 1) s_last_slot = sl_of(e);
      ++j;
    }
  }
  __syncthreads();

  // 4. commit admitted misses into their victims
  int j1 = r1, j2 = r2;
#pragma unroll
  for (int e = 0; e < EPH; ++e) {
    int j;
    if (c1 >> e & 1u) {
      j = j1++;
    } else if (c2 >> e & 1u) {
      j = j2++;
    } else {
      continue;
    }
    if (j >= ma) continue;
    const int s = sl_of(e);
    const int h = miss_i[j];
    const int32_t key = sw ? static_cast<int32_t>(kmin[h])
                           : static_cast<int32_t>(hkey[h] & kKeyMask) - 1;
    // slot_key[s] as the call found it (only this thread writes slot s):
    // fetched at kernel start, or here where 32 slots per thread leave no
    // registers to keep it
    const int32_t old = EPH < 32 ? oldk[e] : sk[s];
    sk[s] = key;
    bit_set_atomic(refl, s);
    val[h] = static_cast<uint32_t>(s);
    msrc[j] = r * a.nkeys + key;
    mdst[j] = r * a.rows + s;
    mvic[j] = old;
    if (sw) {
      const size_t c = static_cast<size_t>(b) * a.ccap + bitmap_rank(mbits, mwpre, key);
      a.copy_src[c] = r * a.nkeys + key;
      a.copy_dst[c] = r * a.rows + s;
    }
  }
  if (sw) {  // scratch-row misses join the copy list too
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      if (jm[e] < 0 || adm[e]) continue;
      const size_t c = static_cast<size_t>(b) * a.ccap + bitmap_rank(mbits, mwpre, tok[e]);
      a.copy_src[c] = r * a.nkeys + tok[e];
      a.copy_dst[c] = r * a.rows + a.H + (jm[e] - ja[e]);
    }
  }
  __syncthreads();

  if (tid < a.Hw) refq[tid] = refl[tid];
  int32_t* out = a.out_locs + static_cast<size_t>(b) * E;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const int i = tid * EPT + e;
    if (i >= E) continue;
    out[i] = tok[e] >= 0 ? r * a.rows + static_cast<int>(val[idx[e]])
                         : (ring[e] >= 0 ? r * a.rows + ring[e] : -1);
  }
  if (tid == 0) {
    a.miss_count[b] = m;
    if (ma > 0) {
      const int nh = s_last_slot + 1;
      a.ctrl[2 * q + 1] = nh == a.H ? 0 : nh;
    }
  }
  if (bad_index) raise_error(a.err, HISPARSE_ERR_BAD_INDEX);
  if (a.fuse_copy) {
    __syncthreads();  // the row's copy list, written above by this workgroup
    const size_t lb = sw ? static_cast<size_t>(b) * a.ccap : static_cast<size_t>(b) * a.cap;
    copy_own_row<NT>(a, (sw ? a.copy_src : a.miss_src) + lb, (sw ? a.copy_dst : a.miss_dst) + lb,
                     m);
  }
}

}  // namespace

size_t clock_lds_bytes(const PlanArgs& a) {
  // pinned, refl, scan, four key bitmaps / prefixes, two words per entry
  // (rank or bucket) and the admitted misses' entries (int16)
  const size_t sw = static_cast<size_t>(a.sort_words);
  const size_t E = static_cast<size_t>(a.S) * a.K;
  const size_t d = sw ? E : static_cast<size_t>(a.hash_size);
  return (2 * static_cast<size_t>(a.Hw) + kPlanThreads / kWave + 1 + 4 * sw + 2 * d) * 4 + E * 2;
}

hipError_t launch_clock_plan(const PlanArgs& a, hipStream_t s) {
  const size_t lds = clock_lds_bytes(a);
  const int E = a.S * a.K;
  auto go = [&](auto kernel) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(kernel, dim3(a.batch), dim3(kPlanThreads), lds, s, a);
    return hipGetLastError();
  };
  if (E <= 2 * kPlanThreads) {
    if (a.H <= 4 * kPlanThreads) return go(clock_plan<kPlanThreads, 2, 4>);
    if (a.H <= 8 * kPlanThreads) return go(clock_plan<kPlanThreads, 2, 8>);
    if (a.H <= 16 * kPlanThreads) return go(clock_plan<kPlanThreads, 2, 16>);
    return go(clock_plan<kPlanThreads, 2, 32>);
  }
  if (a.H <= 4 * kPlanThreads) return go(clock_plan<kPlanThreads, 8, 4>);
  if (a.H <= 8 * kPlanThreads) return go(clock_plan<kPlanThreads, 8, 8>);
  if (a.H <= 16 * kPlanThreads) return go(clock_plan<kPlanThreads, 8, 16>);
  return go(clock_plan<kPlanThreads, 8, 32>);
}

}  // namespace hisparse
