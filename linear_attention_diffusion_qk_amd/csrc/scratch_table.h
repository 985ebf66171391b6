// Per-(device, stream) scratch bookkeeping of the C-ABI entry points.  Written against a small backend
// interface instead of HIP so that the table logic also builds with a host compiler and a fake
// backend (the CPU test of the lifecycle rules).
//
// Rules:
//  * A call on stream s reuses the buffer of the previous call on s.  Stream order runs the new call's
//    kernels after the earlier ones, so no synchronisation is needed; a call that needs more frees the
//    buffer stream-ordered on s and takes a larger one.
//  * The table grows with the number of streams in use; there is no fixed cap.
//  * A stream handle can be reused by the runtime for a new stream once the old one is destroyed, while
//    work the old stream queued may still be running on the old stream's buffer.  Each call's work
//    signals an event when it completes (the buffer's last use: the kernels carry it as their stop
//    event, or it is recorded after them); the next call on the entry makes its stream wait for that
//    event unless it has already completed.  On the same stream that wait is
//    implied by stream order anyway; on a new stream behind a reused handle it is what keeps the old
//    kernels and the new ones apart.
//  * release(dev, s) frees s's buffer stream-ordered on s (so s must still exist) and empties the entry
//    for reuse by another stream.  Entries themselves are never destroyed, so a thread waiting for an
//    entry never touches freed memory; it re-checks after locking that the entry is still its stream's.
#pragma once

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <memory>
#include <mutex>
#include <vector>

namespace sanala {

// Backend: int alloc_async(void** p, size_t bytes, void* stream);  0 = ok
//          int free_async(void* p, void* stream);                  0 = ok
//          int event_create(void** ev);                            0 = ok
//          int event_record(void* ev, void* stream);               0 = ok
//          int event_done(void* ev);                               1 = completed, 0 = not yet
//          int stream_wait(void* stream, void* ev);                0 = ok
template <class Backend>
class ScratchTable {
 public:
  struct Entry {
    int dev = -1;
    void* stream = nullptr;
    void* last_use = nullptr;  // event recorded after the last call's work on the buffer
    bool recorded = false;
    bool in_use = false;  // belongs to (dev, stream)
    void* ptr = nullptr;
    size_t bytes = 0;
    std::mutex mu;
  };

  // Holds the entry's lock from acquire() until destruction: the buffer cannot be grown or released
  // under a caller that has taken it but not yet enqueued its work.
  class Lease {
   public:
    Lease() = default;
    Lease(const Lease&) = delete;
    Lease& operator=(const Lease&) = delete;
    ~Lease() {
      if (!e_) return;
      // The buffer's last use: everything the caller enqueued on the stream while holding the lease.
      // Either the caller's work signalled the event itself (attached), or it is recorded here.
      e_->recorded = attached_ || t_->be_.event_record(e_->last_use, e_->stream) == 0;
      e_->mu.unlock();
    }
    void* ptr() const { return e_ ? e_->ptr : nullptr; }
    size_t bytes() const { return e_ ? e_->bytes : 0; }
    // The last-use event, for work that signals it on completion (then call attached()).
    void* event() const { return e_ ? e_->last_use : nullptr; }
    void attached() { attached_ = true; }

   private:
    friend class ScratchTable;
    Entry* e_ = nullptr;
    ScratchTable* t_ = nullptr;
    bool attached_ = false;
  };

  enum Result { kOk = 0, kErrAlloc = 1, kErrFree = 2, kErrSync = 3 };

  explicit ScratchTable(Backend& be) : be_(be) {}

  // Rounds a request up (a quarter of headroom, 2 MiB granules) so that slowly growing calls do not
  // reallocate every time.
  static size_t granule(size_t bytes) {
    const size_t grown = bytes + bytes / 4;
    constexpr size_t g = size_t(2) << 20;
    return (grown + g - 1) / g * g;
  }

  int acquire(Lease& lease, int dev, void* stream, size_t bytes) {
    for (;;) {
      Entry* e = find_or_claim(dev, stream);
      e->mu.lock();
      if (!owned(e, dev, stream)) {  // released (and perhaps claimed by another stream) meanwhile
        e->mu.unlock();
        continue;
      }
      if (!e->last_use && be_.event_create(&e->last_use) != 0) {
        e->last_use = nullptr;
        e->mu.unlock();
        return kErrSync;
      }
      if (e->recorded && !be_.event_done(e->last_use)) {
        // Kernels of the previous call may still use the buffer: if `stream` is not the stream they
        // were queued on (a handle the runtime gave to a new stream), only this wait orders them.
        if (be_.stream_wait(stream, e->last_use) != 0) {
          e->mu.unlock();
          return kErrSync;
        }
        ++waits_;
      }
      if (e->bytes < bytes) {
        if (e->ptr && be_.free_async(e->ptr, stream) != 0) {
          e->mu.unlock();
          return kErrFree;
        }
        e->ptr = nullptr;
        e->bytes = 0;
        void* p = nullptr;
        const size_t nb = granule(bytes);
        if (be_.alloc_async(&p, nb, stream) != 0) {
          e->mu.unlock();
          return kErrAlloc;
        }
        e->ptr = p;
        e->bytes = nb;
      }
      lease.e_ = e;
      lease.t_ = this;
      return kOk;
    }
  }

  // Frees the buffer of (dev, stream) on `stream` and empties its entry.  No entry: nothing to do.
  int release(int dev, void* stream) {
    Entry* e = nullptr;
    {
      std::lock_guard<std::mutex> lk(mu_);
      for (auto& p : entries_)
        if (p->in_use && p->dev == dev && p->stream == stream) e = p.get();
    }
    if (!e) return kOk;
    std::lock_guard<std::mutex> el(e->mu);
    if (!owned(e, dev, stream)) return kOk;
    int rc = kOk;
    if (e->ptr && be_.free_async(e->ptr, stream) != 0) rc = kErrFree;
    std::lock_guard<std::mutex> lk(mu_);
    e->ptr = nullptr;
    e->bytes = 0;
    e->in_use = false;
    e->stream = nullptr;
    e->dev = -1;
    e->recorded = false;  // the free is ordered on the stream; the event stays for the slot's next owner
    return rc;
  }

  // Entries in use (diagnostics and tests).
  size_t live() {
    std::lock_guard<std::mutex> lk(mu_);
    size_t n = 0;
    for (auto& p : entries_) n += p->in_use ? 1 : 0;
    return n;
  }
  size_t capacity() {
    std::lock_guard<std::mutex> lk(mu_);
    return entries_.size();
  }
  size_t waits() const { return waits_.load(); }

 private:
  bool owned(Entry* e, int dev, void* stream) {
    std::lock_guard<std::mutex> lk(mu_);
    return e->in_use && e->dev == dev && e->stream == stream;
  }

  Entry* find_or_claim(int dev, void* stream) {
    std::lock_guard<std::mutex> lk(mu_);
    Entry* free_slot = nullptr;
    for (auto& p : entries_) {
      if (p->in_use && p->dev == dev && p->stream == stream) return p.get();
      if (!p->in_use && !free_slot) free_slot = p.get();
    }
    Entry* e = free_slot;
    if (!e) {
      entries_.emplace_back(new Entry);
      e = entries_.back().get();
    }
    // Claimed under the table lock, so no other thread claims it too; its fields change only under
    // the table lock while it is not in use.
    e->dev = dev;
    e->stream = stream;
    e->in_use = true;
    return e;
  }

  Backend& be_;
  std::mutex mu_;
  std::vector<std::unique_ptr<Entry>> entries_;
  std::atomic<size_t> waits_{0};
};

}  // namespace sanala
