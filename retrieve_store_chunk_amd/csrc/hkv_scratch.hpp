// Directory of the no-allocation entry point's static device array: which
// layouts' constant tables sit where in it.  Host-only bookkeeping (no HIP
// calls), one directory per device, guarded by the caller's lock.
//
// Each resident layout owns one 256-byte-aligned range.  A layout that is not
// resident gets the first gap large enough; when none is, the least recently
// used layout that no captured call needs is evicted, until one is.  A layout
// that a captured call has used is pinned: a graph reads its tables when it
// replays, so it stays until the layout is destroyed.
#pragma once

#include <cstdint>
#include <vector>

namespace hkv {

class ScratchDirectory {
 public:
  struct Entry {
    uint64_t serial;  // the layout's serial (never reused in a process)
    uint64_t off;     // byte offset in the array, 256-byte aligned
    uint64_t bytes;   // its tables' size
    uint64_t last;    // use clock of its latest call
    bool pinned;      // used by a captured call
  };

  // (Room for 64 entries up front, so that steady use does not allocate.)
  explicit ScratchDirectory(uint64_t capacity) : cap_(capacity) { entries_.reserve(64); }

  // The entry of `serial`, or nullptr.
  Entry* find(uint64_t serial) {
    for (Entry& e : entries_)
      if (e.serial == serial) return &e;
    return nullptr;
  }

  // Places `bytes` for `serial` (not resident) at the first gap that fits,
  // evicting least recently used unpinned entries as needed.  Returns the new
  // entry, or nullptr if even evicting every unpinned entry leaves no room;
  // *evicted counts the entries dropped (so the caller knows whether another
  // layout's range was taken over).
  Entry* reserve(uint64_t serial, uint64_t bytes, int* evicted) {
    *evicted = 0;
    if (bytes == 0 || bytes > cap_) return nullptr;
    for (;;) {
      uint64_t off = 0;
      if (first_fit(bytes, &off)) {
        Entry e{serial, off, bytes, 0, false};
        size_t at = 0;
        while (at < entries_.size() && entries_[at].off < off) ++at;
        entries_.insert(entries_.begin() + (long)at, e);
        return &entries_[at];
      }
      if (!evict_lru()) return nullptr;
      ++*evicted;
    }
  }

  // Marks a call of the entry's layout: its use clock, and a pin if captured.
  void touch(Entry* e, bool captured) {
    e->last = ++clock_;
    if (captured) e->pinned = true;
  }

  // Forgets `serial` (its layout is destroyed).
  void drop(uint64_t serial) {
    for (size_t i = 0; i < entries_.size(); ++i)
      if (entries_[i].serial == serial) {
        entries_.erase(entries_.begin() + (long)i);
        return;
      }
  }

  const std::vector<Entry>& entries() const { return entries_; }

 private:
  static uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

  bool first_fit(uint64_t bytes, uint64_t* off) const {
    uint64_t at = 0;  // entries_ is sorted by offset
    for (const Entry& e : entries_) {
      if (e.off >= at + bytes) break;
      at = align256(e.off + e.bytes);
    }
    if (at + bytes > cap_) return false;
    *off = at;
    return true;
  }

  bool evict_lru() {
    size_t victim = entries_.size();
    for (size_t i = 0; i < entries_.size(); ++i)
      if (!entries_[i].pinned && (victim == entries_.size() || entries_[i].last < entries_[victim].last))
        victim = i;
    if (victim == entries_.size()) return false;
    entries_.erase(entries_.begin() + (long)victim);
    return true;
  }

  uint64_t cap_;
  uint64_t clock_ = 0;
  std::vector<Entry> entries_;
};

}  // namespace hkv
