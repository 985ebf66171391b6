// Host-only driver for the scratch table's lifecycle rules (built and run by test_scratch_table.py with
// a host compiler; a fake backend stands in for the HIP runtime).
#include "scratch_table.h"

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <thread>
#include <vector>

struct Fake {
  std::mutex mu;
  std::map<void*, size_t> live;                // allocations not yet freed
  std::vector<std::pair<void*, void*>> frees;  // (ptr, stream) in order
  std::map<void*, void*> recorded_on;          // event -> stream of its last record
  std::map<void*, bool> done;                  // event -> completed
  std::vector<std::pair<void*, void*>> waits;  // (stream, event)
  int allocs = 0, events = 0, records = 0;
  int alloc_async(void** p, size_t bytes, void*) {
    std::lock_guard<std::mutex> lk(mu);
    *p = std::malloc(1);
    live[*p] = bytes;
    ++allocs;
    return 0;
  }
  int free_async(void* p, void* s) {
    std::lock_guard<std::mutex> lk(mu);
    if (!live.count(p)) return 1;
    live.erase(p);
    frees.emplace_back(p, s);
    std::free(p);
    return 0;
  }
  int event_create(void** ev) {
    std::lock_guard<std::mutex> lk(mu);
    *ev = reinterpret_cast<void*>(0x900000 + 16 * (++events));
    return 0;
  }
  int event_record(void* ev, void* s) {
    std::lock_guard<std::mutex> lk(mu);
    recorded_on[ev] = s;
    done[ev] = false;  // work queued behind it is still running
    ++records;
    return 0;
  }
  int event_done(void* ev) {
    std::lock_guard<std::mutex> lk(mu);
    return done[ev] ? 1 : 0;
  }
  int stream_wait(void* s, void* ev) {
    std::lock_guard<std::mutex> lk(mu);
    waits.emplace_back(s, ev);
    return 0;
  }
  void complete_all() {
    std::lock_guard<std::mutex> lk(mu);
    for (auto& d : done) d.second = true;
  }
};

using Table = sanala::ScratchTable<Fake>;
static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL line %d: %s\n", __LINE__, #c);             \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static void* S(long i) { return reinterpret_cast<void*>(0x1000 + 16 * i); }

int main() {
  Fake be;
  Table t(be);
  // 1. More than 256 streams, one at a time: the table grows, each stream gets its own buffer.
  std::vector<void*> bufs;
  for (long i = 0; i < 300; ++i) {
    Table::Lease l;
    CHECK(t.acquire(l, 0, S(i), 4096) == Table::kOk);
    CHECK(l.ptr() != nullptr && l.bytes() >= 4096);
    bufs.push_back(l.ptr());
  }
  CHECK(t.live() == 300 && be.allocs == 300 && be.live.size() == 300);
  // 2. Reuse: a smaller request on a known stream keeps its buffer.
  {
    Table::Lease l;
    CHECK(t.acquire(l, 0, S(5), 100) == Table::kOk);
    CHECK(l.ptr() == bufs[5] && be.allocs == 300);
  }
  // Another device with the same handle is another entry.
  {
    Table::Lease l;
    CHECK(t.acquire(l, 1, S(5), 100) == Table::kOk);
    CHECK(l.ptr() != bufs[5] && t.live() == 301);
  }
  // 3. Growth: the old buffer is freed on the same stream, a larger one taken.
  {
    Table::Lease l;
    CHECK(t.acquire(l, 0, S(7), 10 << 20) == Table::kOk);
    CHECK(l.ptr() != bufs[7] && l.bytes() >= (size_t(10) << 20));
    CHECK(!be.frees.empty() && be.frees.back().first == bufs[7] && be.frees.back().second == S(7));
    bufs[7] = l.ptr();
  }
  // 4. Last use: each lease records an event on its stream; the next acquire of that entry waits for it
  // while it is pending (a reused handle naming a new stream is then ordered after the old kernels) and
  // does not wait once it has completed.
  {
    be.complete_all();
    void* ev = nullptr;
    {
      Table::Lease l;
      CHECK(t.acquire(l, 0, S(9), 64) == Table::kOk);
    }
    for (auto& r : be.recorded_on)
      if (r.second == S(9)) ev = r.first;
    CHECK(ev != nullptr);
    const size_t w0 = be.waits.size();
    {
      Table::Lease l;  // the earlier call's work is pending: wait on it
      CHECK(t.acquire(l, 0, S(9), 64) == Table::kOk);
      CHECK(be.waits.size() == w0 + 1 && be.waits.back().first == S(9) && be.waits.back().second == ev);
    }
    be.complete_all();
    {
      Table::Lease l;  // completed: no wait
      CHECK(t.acquire(l, 0, S(9), 64) == Table::kOk);
      CHECK(be.waits.size() == w0 + 1 && l.ptr() == bufs[9]);
    }
  }
  // 4b. Work that signals the event itself (attached): no separate record, and the next acquire still
  // waits for it while it is pending.
  {
    be.complete_all();
    void* ev = nullptr;
    const int records = be.records;
    {
      Table::Lease l;
      CHECK(t.acquire(l, 0, S(13), 64) == Table::kOk);
      ev = l.event();
      CHECK(ev != nullptr);
      l.attached();
      be.done[ev] = false;  // the call's kernels, carrying the event, are still running
    }
    CHECK(be.records == records);  // no separate record for an attached lease
    const size_t w0 = be.waits.size();
    Table::Lease l;
    CHECK(t.acquire(l, 0, S(13), 64) == Table::kOk);
    CHECK(be.waits.size() == w0 + 1 && be.waits.back().second == ev);
  }
  // 5. Release frees on the stream and empties the entry; a new stream reuses the slot.
  {
    const size_t cap = t.capacity();
    CHECK(t.release(0, S(11)) == Table::kOk);
    CHECK(be.frees.back().first == bufs[11] && be.frees.back().second == S(11));
    CHECK(t.live() == 300 && t.capacity() == cap);
    CHECK(t.release(0, S(11)) == Table::kOk);  // twice: nothing to do
    Table::Lease l;
    CHECK(t.acquire(l, 0, S(5000), 64) == Table::kOk);
    CHECK(t.capacity() == cap && t.live() == 301);
  }
  // 6. Threads: leases of one entry never overlap; every buffer is freed exactly once in the end.
  {
    std::vector<std::atomic<int>> holders(16);
    std::atomic<int> overlap{0};
    std::vector<std::thread> th;
    for (int w = 0; w < 8; ++w)
      th.emplace_back([&, w]() {
        unsigned x = 12345u + 77u * w;
        for (int it = 0; it < 2000; ++it) {
          x = x * 1664525u + 1013904223u;
          const long s = (x >> 8) % 16;
          if ((x >> 20) % 50 == 0) {
            t.release(0, S(100000 + s));
            continue;
          }
          Table::Lease l;
          if (t.acquire(l, 0, S(100000 + s), 1 + ((x >> 4) % (3u << 20))) != Table::kOk) {
            overlap.fetch_add(1000);
            continue;
          }
          if (holders[s].fetch_add(1) != 0) overlap.fetch_add(1);
          holders[s].fetch_sub(1);
        }
      });
    for (auto& x : th) x.join();
    CHECK(overlap.load() == 0);
  }
  for (long i = 0; i < 6000; ++i) t.release(0, S(i)), t.release(1, S(i)), t.release(0, S(100000 + i % 16));
  CHECK(be.live.empty());
  CHECK(t.live() == 0);
  std::printf("scratch table checks: %d failures, %d allocations, %zu frees, %zu stream waits\n", failures,
              be.allocs, be.frees.size(), be.waits.size());
  return failures == 0 ? 0 : 1;
}
