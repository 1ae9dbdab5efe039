// CPU checks of the library's host-only logic (configuration derivation,
// instance import encoding and export decoding, event-triple bookkeeping),
// built by tests/test_host_sanitized.py with address and undefined-behaviour
// sanitizers.  Exits non-zero on the first failed check; the sanitizers abort
// on any memory error or undefined behaviour.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "host_logic.h"

using namespace hisparse::host;

static int g_checks = 0;
#define CHECK(cond)                                                             \
  do {                                                                          \
    ++g_checks;                                                                 \
    if (!(cond)) {                                                              \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      std::exit(1);                                                             \
    }                                                                           \
  } while (0)

static hisparse_config_t base_config() {
  hisparse_config_t c{};
  c.max_requests = 4;
  c.num_layers = 1;
  c.hot_buffer_size = 100;
  c.top_k = 60;
  c.max_steps = 1;
  c.page_size = 1;
  c.item_size_bytes = 32;
  c.max_seq_len = 500;
  c.policy = HISPARSE_POLICY_LRU;
  c.max_batch = 4;
  return c;
}

static void check_derive_table() {
  Derived d;
  hisparse_config_t c = base_config();
  CHECK(derive(&c, &d) == HISPARSE_OK && d.rows == 100 && d.cap == 60 && d.hw == 4);
  CHECK(derive(nullptr, &d) == HISPARSE_E_INVAL);
  c.top_k = 101;
  CHECK(derive(&c, &d) == HISPARSE_E_INVAL);  // K > H in token LRU
  c = base_config();
  c.policy = HISPARSE_POLICY_CLOCK;
  c.max_steps = 3;
  CHECK(derive(&c, &d) == HISPARSE_OK && d.scratch == 80 && d.rows == 180 && d.cap == 180);
  c.max_steps = 5;
  CHECK(derive(&c, &d) == HISPARSE_E_INVAL);
  c = base_config();
  c.max_requests = c.max_batch = 20000;
  CHECK(derive(&c, &d) == HISPARSE_E_UNSUPPORTED);  // above HISPARSE_MAX_BATCH
  c.max_batch = HISPARSE_MAX_BATCH;
  CHECK(derive(&c, &d) == HISPARSE_OK);
  c = base_config();
  c.page_size = 16;
  c.max_seq_len = 512;
  c.hot_buffer_size = 40;
  c.top_k = 300;
  CHECK(derive(&c, &d) == HISPARSE_OK && d.rows == 40 && d.nkeys == 32 && d.cap == 40);
  c.max_seq_len = 513;
  CHECK(derive(&c, &d) == HISPARSE_E_INVAL);
  c.max_seq_len = 512;
  c.extra_rows = 1;
  CHECK(derive(&c, &d) == HISPARSE_E_UNSUPPORTED);
  c = base_config();
  c.extra_rows = 7;
  CHECK(derive(&c, &d) == HISPARSE_OK && d.rows == 107);
  c = base_config();
  c.max_requests = c.max_batch = 9000;
  c.max_seq_len = 300000;
  c.top_k = 60;
  CHECK(derive(&c, &d) == HISPARSE_E_UNSUPPORTED);  // R * N host rows beyond int32
}

// Random configurations, including extreme field values: derive must never
// overflow, and every accepted configuration must satisfy its invariants.
static void check_derive_fuzz(std::mt19937_64& rng) {
  const int32_t edge[] = {-2147483647 - 1, -5, -1, 0, 1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33,
                          1000, 2048, 4096, 8192, 8193, 16383, 16384, 32767, 32768, 32769,
                          65536, 1 << 20, (1 << 28) - 2, (1 << 28) - 1, 2147483647};
  // mostly in range (so that many configurations are accepted), sometimes
  // an extreme value
  auto pick = [&](int32_t lo, int32_t hi) -> int32_t {
    if (rng() % 10 == 0) return edge[rng() % (sizeof(edge) / sizeof(edge[0]))];
    return lo + static_cast<int32_t>(rng() % static_cast<uint64_t>(hi - lo + 1));
  };
  int accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    hisparse_config_t c{};
    c.max_requests = pick(1, 300);
    c.num_layers = pick(1, 8);
    c.policy = pick(0, 1);
    c.hot_buffer_size = pick(1, 40000);
    c.top_k = c.policy == HISPARSE_POLICY_LRU ? pick(1, c.hot_buffer_size > 0 ? c.hot_buffer_size : 1)
                                              : pick(1, 4096);
    c.max_steps = c.policy == HISPARSE_POLICY_LRU ? pick(1, 1) : pick(2, 4);
    c.page_size = rng() % 2 ? 1 : pick(1, 300);
    c.item_size_bytes = rng() % 10 == 0 ? pick(1, 2000) : 16 * (1 + static_cast<int32_t>(rng() % 100));
    c.max_seq_len = pick(1, 1 << 20);
    if (c.page_size > 1 && c.page_size < 1000 && rng() % 2)
      c.max_seq_len = c.page_size * (1 + static_cast<int32_t>(rng() % 2000));
    c.max_batch = pick(1, c.max_requests > 0 ? c.max_requests : 1);
    c.admission = pick(0, 2);
    c.extra_rows = rng() % 4 ? 0 : pick(0, 100);
    Derived d;
    if (derive(&c, &d) != HISPARSE_OK) continue;
    ++accepted;
    const int64_t H = c.hot_buffer_size, K = c.top_k;
    CHECK(H >= 1 && H <= HISPARSE_MAX_HOT && c.max_batch <= c.max_requests);
    CHECK(c.max_batch <= HISPARSE_MAX_BATCH && c.item_size_bytes % 16 == 0);
    CHECK(d.hw == (H + 31) / 32);
    CHECK(int64_t{c.max_requests} * d.rows < (int64_t{1} << 31));
    CHECK(int64_t{c.max_requests} * d.nkeys < (int64_t{1} << 31));
    if (c.page_size > 1) {
      CHECK(c.policy == HISPARSE_POLICY_LRU && d.rows == H && d.cap == H);
      CHECK(d.nkeys * int64_t{c.page_size} == c.max_seq_len && H <= kMaxPageModeHot);
    } else if (c.policy == HISPARSE_POLICY_LRU) {
      CHECK(K <= H && d.cap == K && d.scratch == 0 && d.rows == H + c.extra_rows);
    } else {
      CHECK(c.max_steps >= 2 && c.max_steps * K <= HISPARSE_MAX_WORKING_SET);
      CHECK(d.scratch == (c.max_steps * K > H ? c.max_steps * K - H : 0));
      CHECK(d.rows == H + d.scratch + c.extra_rows && d.cap == c.max_steps * K);
    }
  }
  CHECK(accepted > 1000);
}

// Random LRU and CLOCK instances: the import encoding is the inverse of the
// host layout, the LRU order is (timestamp, slot), the reference bitmap
// decodes back to the same bits; every malformed layout is rejected.
static void check_import_export(std::mt19937_64& rng) {
  for (int it = 0; it < 3000; ++it) {
    const int32_t H = 1 + static_cast<int32_t>(rng() % (it % 10 == 0 ? 32768 : 300));
    const int32_t nkeys = H + static_cast<int32_t>(rng() % 1000);
    const bool lru = rng() % 2;
    const int32_t now = 1 + static_cast<int32_t>(rng() % 50);
    std::vector<int32_t> keys(static_cast<size_t>(nkeys));
    for (int32_t i = 0; i < nkeys; ++i) keys[i] = i;
    std::shuffle(keys.begin(), keys.end(), rng);
    std::vector<int32_t> slot_key(H), policy(H);
    for (int32_t s = 0; s < H; ++s) {
      const bool occupied = rng() % 4 != 0;
      slot_key[s] = occupied ? keys[s] : kEmptyKey;
      if (lru)
        policy[s] = occupied ? static_cast<int32_t>(rng() % now) : -1;
      else
        policy[s] = static_cast<int32_t>(rng() % 2);
    }
    const int32_t ctrl[2] = {now, static_cast<int32_t>(rng() % H)};
    InstanceImage img;
    CHECK(encode_import(H, nkeys, lru, slot_key.data(), policy.data(), ctrl, &img) == HISPARSE_OK);
    // export's key->slot map: the inverse of the slot->key array
    std::vector<int32_t> wide(static_cast<size_t>(nkeys), 12345);
    CHECK(invert_slot_key(slot_key.data(), H, nkeys, wide.data()) == HISPARSE_OK);
    int32_t resident = 0;
    for (int32_t k = 0; k < nkeys; ++k) {
      if (wide[k] < 0) {
        CHECK(wide[k] == kEmptyKey);
        continue;
      }
      ++resident;
      CHECK(wide[k] < H && slot_key[wide[k]] == k);
    }
    int32_t occupied = 0;
    for (int32_t s = 0; s < H; ++s) occupied += slot_key[s] != kEmptyKey;
    CHECK(resident == occupied);
    if (lru) {
      CHECK(static_cast<int32_t>(img.order.size()) == H && img.refbits.empty());
      std::vector<char> seen(static_cast<size_t>(H), 0);
      for (int32_t i = 0; i < H; ++i) {
        const int32_t s = img.order[i];
        CHECK(s >= 0 && s < H && !seen[s]);
        seen[s] = 1;
        if (i > 0) {
          const int32_t p = img.order[i - 1];
          CHECK(policy[p] < policy[s] || (policy[p] == policy[s] && p < s));
        }
      }
    } else {
      CHECK(static_cast<int32_t>(img.refbits.size()) == (H + 31) / 32 && img.order.empty());
      std::vector<int32_t> back(static_cast<size_t>(H));
      decode_refbits(img.refbits.data(), H, back.data());
      CHECK(back == policy);
      if (H % 32) CHECK((img.refbits.back() >> (H % 32)) == 0u);  // no bits past H
    }
    // malformed layouts
    if (occupied >= 2) {
      std::vector<int32_t> bad = slot_key;
      int32_t a = -1, b = -1;
      for (int32_t s = 0; s < H && b < 0; ++s)
        if (bad[s] != kEmptyKey) (a < 0 ? a : b) = s;
      bad[b] = bad[a];
      CHECK(encode_import(H, nkeys, lru, bad.data(), policy.data(), ctrl, &img) == HISPARSE_E_INVAL);
      std::vector<int32_t> inv(static_cast<size_t>(nkeys));
      CHECK(invert_slot_key(bad.data(), H, nkeys, inv.data()) == HISPARSE_E_INVAL);
    }
    {
      std::vector<int32_t> bad = slot_key;
      bad[rng() % H] = nkeys + static_cast<int32_t>(rng() % 5);
      CHECK(encode_import(H, nkeys, lru, bad.data(), policy.data(), ctrl, &img) == HISPARSE_E_INVAL);
      bad[rng() % H] = -2;
      CHECK(encode_import(H, nkeys, lru, bad.data(), policy.data(), ctrl, &img) == HISPARSE_E_INVAL);
    }
    if (lru) {
      std::vector<int32_t> bad = policy;
      const int32_t s = static_cast<int32_t>(rng() % H);
      bad[s] = slot_key[s] == kEmptyKey ? 0 : now;  // empty with a time, or not before now
      CHECK(encode_import(H, nkeys, lru, slot_key.data(), bad.data(), ctrl, &img) == HISPARSE_E_INVAL);
      const int32_t neg[2] = {-1, 0};
      CHECK(encode_import(H, nkeys, lru, slot_key.data(), policy.data(), neg, &img) ==
            HISPARSE_E_INVAL);
    } else {
      std::vector<int32_t> bad = policy;
      bad[rng() % H] = 2;
      CHECK(encode_import(H, nkeys, lru, slot_key.data(), bad.data(), ctrl, &img) == HISPARSE_E_INVAL);
      const int32_t far[2] = {0, H};
      CHECK(encode_import(H, nkeys, lru, slot_key.data(), policy.data(), far, &img) ==
            HISPARSE_E_INVAL);
      const int32_t neg[2] = {0, -1};
      CHECK(encode_import(H, nkeys, lru, slot_key.data(), policy.data(), neg, &img) ==
            HISPARSE_E_INVAL);
    }
  }
  InstanceImage img;
  const int32_t one[1] = {0};
  CHECK(encode_import(0, 4, true, one, one, one, &img) == HISPARSE_E_INVAL);
  CHECK(encode_import(1, 4, true, nullptr, one, one, &img) == HISPARSE_E_INVAL);
}

// Calls that record 0-3 events (an event could not be taken, a launch failed)
// with the guard on every return path: pending events stay whole triples of
// one call each, and every event is in exactly one list.
static int fake_call(EventLedger<int>* ledger, int* next_event, int record_ok, bool profiling,
                     std::vector<std::vector<int>>* whole) {
  TripleGuard<int> guard(ledger, profiling);
  std::vector<int> mine;
  for (int k = 0; k < 3; ++k) {
    if (!profiling) continue;
    if (k >= record_ok) return -1;  // early return after a failed launch
    int e;
    if (!ledger->free_list.empty()) {
      e = ledger->free_list.back();
      ledger->free_list.pop_back();
    } else {
      e = (*next_event)++;
    }
    ledger->push(e);
    mine.push_back(e);
  }
  if (profiling) whole->push_back(mine);
  return 0;
}

static void check_event_ledger(std::mt19937_64& rng) {
  EventLedger<int> ledger;
  int next_event = 0;
  std::vector<std::vector<int>> whole;  // triples of successful calls, in order
  size_t drained_calls = 0;
  for (int it = 0; it < 100000; ++it) {
    const bool profiling = rng() % 8 != 0;
    const int record_ok = rng() % 5 == 0 ? static_cast<int>(rng() % 3) : 3;
    fake_call(&ledger, &next_event, record_ok, profiling, &whole);
    CHECK(ledger.pending.size() % 3 == 0);
    CHECK(ledger.pending.size() / 3 + drained_calls == whole.size());
    if (rng() % 97 == 0) {
      size_t i = drained_calls;
      const size_t n = ledger.drain([&](int a, int b, int c) {
        CHECK(i < whole.size());
        CHECK(whole[i][0] == a && whole[i][1] == b && whole[i][2] == c);
        ++i;
      });
      drained_calls += n;
      CHECK(ledger.pending.empty() && i == drained_calls);
    }
    if (it % 1000 == 0) {  // every event lives in exactly one list
      std::set<int> all(ledger.free_list.begin(), ledger.free_list.end());
      CHECK(all.size() == ledger.free_list.size());
      for (int e : ledger.pending) CHECK(all.insert(e).second);
      CHECK(static_cast<int>(all.size()) == next_event);
    }
  }
  CHECK(next_event < 5000);  // events are reused, not leaked (100000 calls)
}

int main() {
  std::mt19937_64 rng(20261203);
  check_derive_table();
  check_derive_fuzz(rng);
  check_import_export(rng);
  check_event_ledger(rng);
  std::printf("host logic: all %d checks passed\n", g_checks);
  return 0;
}
