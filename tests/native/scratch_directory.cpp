// The no-allocation entry point's scratch directory (hkv_scratch.hpp) on the
// host: first-fit placement on 256-byte boundaries inside the capacity,
// least-recently-used eviction that never takes a pinned entry, room freed
// by drop, and refusal when pinned entries leave no room.
#include <cstdio>
#include <vector>

#include "hkv_scratch.hpp"

#define FAIL(...) do { std::printf(__VA_ARGS__); std::printf("\n"); return 1; } while (0)

using Dir = hkv::ScratchDirectory;

static int check_disjoint(const Dir& d, uint64_t cap) {
  const auto& e = d.entries();
  for (size_t i = 0; i < e.size(); ++i) {
    if (e[i].off % 256) FAIL("entry %zu at unaligned offset %llu", i, (unsigned long long)e[i].off);
    if (e[i].off + e[i].bytes > cap) FAIL("entry %zu past the capacity", i);
    if (i && e[i].off < e[i - 1].off + e[i - 1].bytes) FAIL("entries %zu and %zu overlap", i - 1, i);
  }
  return 0;
}

int main() {
  const uint64_t cap = 4096;
  Dir d(cap);
  int ev = 0;
  // three layouts fit side by side, each on a 256-byte boundary
  Dir::Entry* a = d.reserve(1, 1000, &ev);
  if (!a || a->off != 0 || ev) FAIL("first entry");
  d.touch(a, false);
  Dir::Entry* b = d.reserve(2, 1000, &ev);
  if (!b || b->off != 1024 || ev) FAIL("second entry at %llu", b ? (unsigned long long)b->off : 0ull);
  d.touch(b, false);
  Dir::Entry* c = d.reserve(3, 1500, &ev);
  if (!c || c->off != 2048 || ev) FAIL("third entry");
  d.touch(c, false);
  if (check_disjoint(d, cap)) return 1;
  if (!d.find(2) || d.find(4)) FAIL("find");
  // using layout 1 again makes layout 2 the least recently used
  d.touch(d.find(1), false);
  Dir::Entry* e4 = d.reserve(4, 1000, &ev);
  if (!e4 || ev != 1 || d.find(2) || e4->off != 1024) FAIL("LRU eviction (evicted %d)", ev);
  d.touch(e4, false);
  if (check_disjoint(d, cap)) return 1;
  // a pinned entry (used under capture) is never evicted
  d.touch(d.find(1), true);
  Dir::Entry* e5 = d.reserve(5, 3000, &ev);   // needs entries 3 and 4 gone
  if (!e5 || !d.find(1) || d.find(3) || d.find(4) || ev != 2) FAIL("eviction around a pin (evicted %d)", ev);
  if (e5->off != 1024) FAIL("fifth entry at %llu", (unsigned long long)e5->off);
  d.touch(e5, true);
  if (check_disjoint(d, cap)) return 1;
  // with only pinned entries left and no gap, a reservation is refused
  if (d.reserve(6, 512, &ev)) FAIL("reserved past pinned entries");
  if (!d.find(1) || !d.find(5)) FAIL("refusal dropped an entry");
  // dropping a layout frees its range
  d.drop(5);
  Dir::Entry* e6 = d.reserve(6, 2048, &ev);
  if (!e6 || ev || e6->off != 1024) FAIL("room after drop");
  if (check_disjoint(d, cap)) return 1;
  // sizes beyond the capacity, and zero, are refused
  if (d.reserve(7, cap + 1, &ev) || d.reserve(8, 0, &ev)) FAIL("bad sizes");
  // a long random run: entries stay aligned, disjoint and inside
  Dir r(1 << 20);
  uint64_t x = 0x9E3779B97F4A7C15ull;
  for (uint64_t s = 1; s <= 20000; ++s) {
    x ^= x << 13; x ^= x >> 7; x ^= x << 17;
    const uint64_t serial = 1 + x % 64, bytes = 1 + (x >> 20) % (300 << 10);
    Dir::Entry* hit = r.find(serial);
    if (!hit) hit = r.reserve(serial, bytes, &ev);
    if (!hit) FAIL("random run: no room with nothing pinned");
    r.touch(hit, false);
    if (check_disjoint(r, 1 << 20)) return 1;
  }
  std::printf("scratch directory ok\n");
  return 0;
}
