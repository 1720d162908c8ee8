// blob_cache.h - device copies of small host blobs (multi-tensor tables,
// factored-step plans), cached by content.
//
// A training loop passes the same tensor lists every step, also when it steps
// tensor by tensor from gradient hooks (one blob per tensor, hundreds per
// model), so after the first step nothing is uploaded. Blobs live in
// per-device arenas of pinned host staging plus device memory. When an
// arena's limit is reached, the device is synchronized and that device's
// cache is emptied.
//
// Lifetime rule. A caller takes a Lease, asks for its blob, enqueues the
// launches that read it and only then drops the lease. Emptying the cache
// waits until no lease is held (new leases wait behind it), then synchronizes
// the device: every launch that may read a blob has been enqueued before the
// synchronization, so none reads freed memory. A caller that needs several
// blobs enqueues the launches that read one before it asks for the next: a
// request that empties the cache gives up the caller's own lease meanwhile.
//
// The cache logic is a template over its backend (memory, copies, events,
// synchronization) so that the host tests can drive it under a fake device.
#pragma once

#include <condition_variable>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/ps.h"

namespace ps {

// Shared/exclusive gate in which a waiting exclusive holder goes first.
class UseGate {
 public:
  void lock_shared() {
    std::unique_lock<std::mutex> l(mu_);
    cv_.wait(l, [&] { return !writer_ && waiting_ == 0; });
    ++readers_;
  }
  void unlock_shared() {
    std::lock_guard<std::mutex> l(mu_);
    if (--readers_ == 0) cv_.notify_all();
  }
  void lock() {
    std::unique_lock<std::mutex> l(mu_);
    ++waiting_;
    cv_.wait(l, [&] { return !writer_ && readers_ == 0; });
    --waiting_;
    writer_ = true;
  }
  void unlock() {
    std::lock_guard<std::mutex> l(mu_);
    writer_ = false;
    cv_.notify_all();
  }

 private:
  std::mutex mu_;
  std::condition_variable cv_;
  int readers_ = 0, waiting_ = 0;
  bool writer_ = false;
};

struct BlobLimits {
  size_t max_entries;   // blobs per device
  size_t max_bytes;     // arena bytes per device
  size_t chunk_bytes;   // arena growth step
};

// Backend requirements (B::Stream, B::Event and):
//   int alloc_chunk(size_t bytes, char** dev, char** host)   0 or a ps_status
//   void free_chunk(char* dev, char* host)
//   int create_event(Event*); void destroy_event(Event)
//   int upload(char* dev, const char* host, size_t bytes, Stream, Event)  copy, then record Event
//   bool event_done(Event); int stream_wait(Stream, Event)
//   int device_sync(); void sync_stream(Stream)
template <class B>
class BlobCache {
 public:
  using Stream = typename B::Stream;
  using Event = typename B::Event;

  class Lease {
   public:
    explicit Lease(BlobCache& c) : c_(c) { c_.gate_.lock_shared(); }
    ~Lease() {
      if (held_) c_.gate_.unlock_shared();
    }
    Lease(const Lease&) = delete;
    Lease& operator=(const Lease&) = delete;

   private:
    friend class BlobCache;
    BlobCache& c_;
    bool held_ = true;
  };

  BlobCache(B& backend, BlobLimits lim) : be_(backend), lim_(lim) {}

  // Device copy of `bytes` bytes at `data` on `device`, ready for work
  // enqueued on `s` after this call (the stream waits for the upload if it
  // may still run). `lease` must be held by the caller.
  int get(int device, const void* data, size_t bytes, Stream s, const void** dptr, Lease& lease) {
    const uint64_t h = fnv1a(data, bytes);
    {
      std::lock_guard<std::mutex> lk(mu_);
      Dev& dc = devs_[device];
      if (const Entry* e = find(dc, h, data, bytes)) return hand_out(e, s, dptr);
      if (dc.entries < lim_.max_entries && dc.bytes + bytes <= lim_.max_bytes) return insert(dc, h, data, bytes, s, dptr);
    }
    // Full: empty this device's cache once no caller holds a blob pointer
    // that it has not yet launched on (this caller included).
    lease.held_ = false;
    gate_.unlock_shared();
    int st = 0;
    gate_.lock();
    {
      std::lock_guard<std::mutex> lk(mu_);
      Dev& dc = devs_[device];
      if (dc.entries >= lim_.max_entries || dc.bytes + bytes > lim_.max_bytes) {
        st = be_.device_sync();
        if (!st) {
          flush(dc);
          ++flushes_;
        }
      }
    }
    gate_.unlock();
    gate_.lock_shared();
    lease.held_ = true;
    if (st) return st;
    std::lock_guard<std::mutex> lk(mu_);
    Dev& dc = devs_[device];
    if (const Entry* e = find(dc, h, data, bytes)) return hand_out(e, s, dptr);
    return insert(dc, h, data, bytes, s, dptr);
  }

  size_t flushes() {
    std::lock_guard<std::mutex> lk(mu_);
    return flushes_;
  }

 private:
  struct Entry {
    std::vector<unsigned char> key;
    const void* d_mem = nullptr;
    Event ready{};
    bool done = false;   // the upload is known to have completed
  };
  struct Chunk {
    char* d_mem = nullptr;
    char* h_mem = nullptr;   // pinned source of the uploads
    size_t size = 0, used = 0;
  };
  struct Dev {
    std::unordered_multimap<uint64_t, Entry*> by_hash;
    std::vector<Chunk> chunks;
    size_t entries = 0, bytes = 0;
  };
  static constexpr size_t kAlign = 256;

  static uint64_t fnv1a(const void* data, size_t bytes) {
    const unsigned char* p = (const unsigned char*)data;
    uint64_t h = 1469598103934665603ull;
    for (size_t i = 0; i < bytes; ++i) h = (h ^ p[i]) * 1099511628211ull;
    return h;
  }

  static const Entry* find(Dev& dc, uint64_t h, const void* data, size_t bytes) {
    auto range = dc.by_hash.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const Entry* e = it->second;
      if (e->key.size() == bytes && memcmp(e->key.data(), data, bytes) == 0) return e;
    }
    return nullptr;
  }

  int hand_out(const Entry* ce, Stream s, const void** dptr) {
    Entry* e = const_cast<Entry*>(ce);
    if (!e->done) {
      if (be_.event_done(e->ready))
        e->done = true;
      else if (int st = be_.stream_wait(s, e->ready))
        return st;
    }
    *dptr = e->d_mem;
    return 0;
  }

  void flush(Dev& dc) {
    for (auto& kv : dc.by_hash) {
      be_.destroy_event(kv.second->ready);
      delete kv.second;
    }
    dc.by_hash.clear();
    for (Chunk& c : dc.chunks) be_.free_chunk(c.d_mem, c.h_mem);
    dc.chunks.clear();
    dc.entries = dc.bytes = 0;
  }

  int insert(Dev& dc, uint64_t h, const void* data, size_t bytes, Stream s, const void** dptr) {
    const size_t need = (bytes + kAlign - 1) / kAlign * kAlign;
    if (dc.chunks.empty() || dc.chunks.back().size - dc.chunks.back().used < need) {
      Chunk c;
      c.size = need > lim_.chunk_bytes ? need : lim_.chunk_bytes;
      if (int st = be_.alloc_chunk(c.size, &c.d_mem, &c.h_mem)) return st;
      dc.chunks.push_back(c);
      dc.bytes += c.size;
    }
    Chunk& c = dc.chunks.back();
    char* d = c.d_mem + c.used;
    char* hm = c.h_mem + c.used;
    c.used += need;
    Entry* e = new Entry;
    e->key.assign((const unsigned char*)data, (const unsigned char*)data + bytes);
    e->d_mem = d;
    memcpy(hm, data, bytes);
    int st = be_.create_event(&e->ready);
    if (st) {
      delete e;
      return st;
    }
    if ((st = be_.upload(d, hm, bytes, s, e->ready))) {
      // the arena space stays reserved until the next flush
      be_.sync_stream(s);
      be_.destroy_event(e->ready);
      delete e;
      return st;
    }
    dc.by_hash.emplace(h, e);
    ++dc.entries;
    *dptr = d;
    return 0;
  }

  B& be_;
  const BlobLimits lim_;
  UseGate gate_;
  std::mutex mu_;
  std::unordered_map<int, Dev> devs_;
  size_t flushes_ = 0;
};

}  // namespace ps
