// Host-only logic of the C ABI: configuration checks, the import and export
// encodings of a cache instance, and the bookkeeping of the timing events.
//
// No HIP header is included here, so the same code also builds with a plain
// host compiler under address and undefined-behaviour sanitizers (the CPU test
// driver does that); hisparse_api.cpp uses it for the real calls.
#pragma once

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <numeric>
#include <vector>

#include "hisparse.h"

namespace hisparse {
namespace host {

constexpr int32_t kEmptyKey = -1;
constexpr int32_t kMaxPageModeHot = 4096;
// The miss copy keeps the per-row prefix of miss counts of a call in LDS,
// (batch + 1) * 4 bytes beside its scan scratch, within the 64 KiB a
// workgroup gets by default.
constexpr int32_t kMaxBatch = HISPARSE_MAX_BATCH;

struct Derived {
  int32_t rows = 0;     // device rows per request
  int32_t scratch = 0;  // CLOCK scratch rows per request
  int32_t nkeys = 0;    // keys per request (tokens, or pages)
  int32_t hw = 0;       // 32-bit words of an H-bit mask
  int32_t cap = 0;      // plan capacity per row
};

// Scalar validation of a configuration (the pointer arrays are checked by
// state creation, which needs the device).
inline int derive(const hisparse_config_t* c, Derived* d) {
  if (c == nullptr || d == nullptr) return HISPARSE_E_INVAL;
  const bool lru = c->policy == HISPARSE_POLICY_LRU;
  const bool clock = c->policy == HISPARSE_POLICY_CLOCK;
  if (!lru && !clock) return HISPARSE_E_INVAL;
  if (c->max_requests < 1 || c->num_layers < 1 || c->top_k < 1 || c->page_size < 1)
    return HISPARSE_E_INVAL;
  if (c->hot_buffer_size < 1 || c->hot_buffer_size > HISPARSE_MAX_HOT) return HISPARSE_E_INVAL;
  if (c->item_size_bytes < 16 || c->item_size_bytes % 16) return HISPARSE_E_INVAL;
  if (c->max_seq_len < 1) return HISPARSE_E_INVAL;
  if (c->max_seq_len > HISPARSE_MAX_SEQ_LEN) return HISPARSE_E_UNSUPPORTED;
  if (c->max_batch < 1 || c->max_batch > c->max_requests) return HISPARSE_E_INVAL;
  if (c->max_batch > kMaxBatch) return HISPARSE_E_UNSUPPORTED;
  if (c->admission < HISPARSE_ADMIT_RECENT || c->admission > HISPARSE_ADMIT_FIRST)
    return HISPARSE_E_INVAL;
  if (c->extra_rows < 0 || c->extra_rows > c->max_seq_len) return HISPARSE_E_INVAL;
  if (c->extra_rows > 0 && c->page_size > 1) return HISPARSE_E_UNSUPPORTED;
  const int64_t H = c->hot_buffer_size, K = c->top_k, P = c->page_size;
  if (lru) {
    if (c->max_steps != 1) return HISPARSE_E_INVAL;
    if (K > HISPARSE_MAX_WORKING_SET) return HISPARSE_E_UNSUPPORTED;
    if (P == 1) {
      if (K > H) return HISPARSE_E_INVAL;  // a row's distinct tokens must fit
    } else {
      if (c->max_seq_len % P) return HISPARSE_E_INVAL;
      if (c->max_seq_len / P > HISPARSE_MAX_PAGES_PER_REQUEST) return HISPARSE_E_UNSUPPORTED;
      if (H > kMaxPageModeHot) return HISPARSE_E_UNSUPPORTED;
    }
  } else {
    if (P != 1) return HISPARSE_E_INVAL;
    if (c->max_steps < HISPARSE_MIN_STEPS || c->max_steps > HISPARSE_MAX_STEPS)
      return HISPARSE_E_INVAL;
    if (c->max_steps * K > HISPARSE_MAX_WORKING_SET) return HISPARSE_E_UNSUPPORTED;
  }
  const int64_t scratch = clock ? std::max<int64_t>(0, c->max_steps * K - H) : 0;
  const int64_t rows = P > 1 ? H : H + scratch + c->extra_rows;
  const int64_t nkeys = P > 1 ? c->max_seq_len / P : c->max_seq_len;
  // host rows, device rows and plan entries are int32
  const int64_t R = c->max_requests;
  if (R * nkeys >= (int64_t{1} << 31) || R * rows >= (int64_t{1} << 31))
    return HISPARSE_E_UNSUPPORTED;
  d->scratch = static_cast<int32_t>(scratch);
  d->rows = static_cast<int32_t>(rows);
  d->nkeys = static_cast<int32_t>(nkeys);
  d->hw = static_cast<int32_t>((H + 31) / 32);
  d->cap = P > 1 ? static_cast<int32_t>(H) : static_cast<int32_t>(c->max_steps * K);
  return HISPARSE_OK;
}

// Device images of one instance built from the host layout of
// hisparse_state_import: the LRU order (slots by (timestamp, slot)) or the
// CLOCK reference bitmap.  (The slot->key array is copied as given; no
// key->slot table is kept on the device.)
struct InstanceImage {
  std::vector<int16_t> order;     // [H]   LRU
  std::vector<uint32_t> refbits;  // [hw]  CLOCK
};

// Validates and encodes an import.  `ctrl` = {LRU call counter, CLOCK hand}.
// HISPARSE_E_INVAL when a key is out of range or resident twice, an LRU
// timestamp is outside [0, counter) for an occupied slot or not -1 for an
// empty one, the counter is negative, a reference bit is not 0/1, or the
// hand is outside [0, H).
inline int encode_import(int32_t H, int32_t nkeys, bool lru, const int32_t* slot_key,
                         const int32_t* policy, const int32_t* ctrl, InstanceImage* img) {
  if (H < 1 || H > HISPARSE_MAX_HOT || nkeys < 1 || !slot_key || !policy || !ctrl || !img)
    return HISPARSE_E_INVAL;
  if (lru && ctrl[0] < 0) return HISPARSE_E_INVAL;
  if (!lru && (ctrl[1] < 0 || ctrl[1] >= H)) return HISPARSE_E_INVAL;
  std::vector<bool> seen(static_cast<size_t>(nkeys), false);
  for (int32_t s = 0; s < H; ++s) {
    const int32_t k = slot_key[s];
    if (k == kEmptyKey) {
      if (lru && policy[s] != -1) return HISPARSE_E_INVAL;
      continue;
    }
    if (k < 0 || k >= nkeys || seen[static_cast<size_t>(k)]) return HISPARSE_E_INVAL;
    seen[static_cast<size_t>(k)] = true;
    if (lru && (policy[s] < 0 || policy[s] >= ctrl[0])) return HISPARSE_E_INVAL;
  }
  img->order.clear();
  img->refbits.clear();
  if (lru) {
    std::vector<int32_t> idx(static_cast<size_t>(H));
    std::iota(idx.begin(), idx.end(), 0);
    // (timestamp, slot): stable on timestamps over slots in ascending order
    std::stable_sort(idx.begin(), idx.end(),
                     [&](int32_t x, int32_t y) { return policy[x] < policy[y]; });
    img->order.assign(idx.begin(), idx.end());
  } else {
    img->refbits.assign(static_cast<size_t>((H + 31) / 32), 0u);
    for (int32_t s = 0; s < H; ++s) {
      if (policy[s] != 0 && policy[s] != 1) return HISPARSE_E_INVAL;
      if (policy[s]) img->refbits[static_cast<size_t>(s) >> 5] |= 1u << (s & 31);
    }
  }
  return HISPARSE_OK;
}

// Export: the CLOCK reference bitmap as one 0/1 word per slot.
inline void decode_refbits(const uint32_t* bits, int32_t H, int32_t* policy) {
  for (int32_t s = 0; s < H; ++s) policy[s] = static_cast<int32_t>((bits[s >> 5] >> (s & 31)) & 1u);
}

// Export: the key->slot map as the inverse of the slot->key array (every key
// -1 except the resident ones).  HISPARSE_E_INVAL if a key is out of range or
// held by two slots (the array is then not a valid map).
inline int invert_slot_key(const int32_t* slot_key, int32_t H, int32_t nkeys, int32_t* key_slot) {
  std::fill(key_slot, key_slot + nkeys, kEmptyKey);
  for (int32_t s = 0; s < H; ++s) {
    const int32_t k = slot_key[s];
    if (k == kEmptyKey) continue;
    if (k < 0 || k >= nkeys || key_slot[k] != kEmptyKey) return HISPARSE_E_INVAL;
    key_slot[k] = s;
  }
  return HISPARSE_OK;
}

// Events of the timed swap calls: every call records a triple (before the
// plan kernel, between the kernels, after the copy).  A call that cannot
// record all three -- an event could not be taken, or a launch failed --
// returns its events to the free list, so pending events always form whole
// triples and each drained triple belongs to one call.
template <class Ev>
class EventLedger {
 public:
  std::vector<Ev> free_list;
  std::vector<Ev> pending;

  size_t mark() const { return pending.size(); }
  void push(Ev e) { pending.push_back(e); }
  // Keeps the events recorded since `m` if they are one whole triple, else
  // returns them to the free list.
  void settle(size_t m) {
    if (pending.size() - m != 3) rollback(m);
  }
  void rollback(size_t m) {
    while (pending.size() > m) {
      free_list.push_back(pending.back());
      pending.pop_back();
    }
  }
  // Calls f(e0, e1, e2) for every pending triple in order, then moves all of
  // them to the free list.  Returns the number of triples.
  template <class F>
  size_t drain(F&& f) {
    const size_t n = pending.size() / 3;
    for (size_t i = 0; i < n; ++i) f(pending[3 * i], pending[3 * i + 1], pending[3 * i + 2]);
    free_list.insert(free_list.end(), pending.begin(), pending.end());
    pending.clear();
    return n;
  }
};

// RAII guard of one call's triple: settles it on every return path.
template <class Ev>
class TripleGuard {
 public:
  TripleGuard(EventLedger<Ev>* l, bool active) : l_(active ? l : nullptr), m_(l->mark()) {}
  ~TripleGuard() {
    if (l_ != nullptr) l_->settle(m_);
  }
  TripleGuard(const TripleGuard&) = delete;
  TripleGuard& operator=(const TripleGuard&) = delete;

 private:
  EventLedger<Ev>* l_;
  size_t m_;
};

}  // namespace host
}  // namespace hisparse
