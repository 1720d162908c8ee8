// blob_cache_host_test.cpp - drives the library's device blob cache
// (precision_state_amd/csrc/blob_cache.h) on the host under a fake device,
// with tiny limits so that the cache empties itself many times while several
// threads use it.
//
// The fake device runs every enqueued operation (uploads, "kernels") on one
// background thread in enqueue order, as a GPU runs stream work after the
// host call returns. Freed chunks are poisoned and never reused, and each
// "kernel" checks that the blob it reads still lies in a live chunk and holds
// the bytes its caller asked for. A blob freed between the caller getting its
// pointer and its launch running is therefore caught.
//
// Usage: blob_cache_host_test <threads> <iterations per thread>
// Prints "flushes=<n> launches=<n> errors=<n>" and exits 0 when errors == 0
// and the cache was emptied at least threads times.
#include <atomic>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <functional>
#include <map>
#include <mutex>
#include <random>
#include <thread>
#include <vector>

#include "blob_cache.h"

namespace {

struct FakeDevice {
  using Stream = int;
  struct Ev {
    std::atomic<bool> done{false};
  };
  using Event = Ev*;

  std::mutex mu;
  std::condition_variable cv;
  std::deque<std::function<void()>> q;
  uint64_t enqueued = 0, executed = 0;
  bool stop = false;
  std::map<const char*, size_t> live;             // device chunks not yet freed
  std::vector<std::pair<char*, char*>> graveyard;  // freed chunks, poisoned, never reused
  std::atomic<long> errors{0}, launches{0};
  std::thread worker;

  FakeDevice() : worker([this] { run(); }) {}
  ~FakeDevice() {
    {
      std::lock_guard<std::mutex> l(mu);
      stop = true;
    }
    cv.notify_all();
    worker.join();
    for (auto& c : graveyard) {
      delete[] c.first;
      delete[] c.second;
    }
  }

  void run() {
    std::unique_lock<std::mutex> l(mu);
    for (;;) {
      cv.wait(l, [&] { return stop || !q.empty(); });
      if (q.empty()) return;
      std::function<void()> f = std::move(q.front());
      q.pop_front();
      l.unlock();
      f();
      l.lock();
      ++executed;
      cv.notify_all();
    }
  }

  void enqueue(std::function<void()> f) {
    std::lock_guard<std::mutex> l(mu);
    q.push_back(std::move(f));
    ++enqueued;
    cv.notify_all();
  }

  // true when [p, p + n) lies inside one live chunk (call with mu held)
  bool is_live(const char* p, size_t n) {
    auto it = live.upper_bound(p);
    if (it == live.begin()) return false;
    --it;
    return p >= it->first && p + n <= it->first + it->second;
  }

  // Backend interface of BlobCache.
  int alloc_chunk(size_t bytes, char** d, char** h) {
    *d = new char[bytes];
    *h = new char[bytes];
    std::lock_guard<std::mutex> l(mu);
    live[*d] = bytes;
    return 0;
  }
  void free_chunk(char* d, char* h) {
    std::lock_guard<std::mutex> l(mu);
    auto it = live.find(d);
    if (it == live.end()) {
      ++errors;
      return;
    }
    memset(d, 0xDD, it->second);
    live.erase(it);
    graveyard.emplace_back(d, h);
  }
  int create_event(Event* e) {
    *e = new Ev;
    return 0;
  }
  void destroy_event(Event e) { delete e; }
  int upload(char* d, const char* h, size_t bytes, Stream, Event e) {
    enqueue([this, d, h, bytes, e] {
      {
        std::lock_guard<std::mutex> l(mu);
        if (!is_live(d, bytes)) {
          ++errors;
          return;
        }
      }
      memcpy(d, h, bytes);
      e->done = true;
    });
    return 0;
  }
  bool event_done(Event e) { return e->done.load(); }
  int stream_wait(Stream, Event) { return 0; }   // one queue: enqueue order is execution order
  int device_sync() {
    std::unique_lock<std::mutex> l(mu);
    const uint64_t target = enqueued;
    cv.wait(l, [&] { return executed >= target; });
    return 0;
  }
  void sync_stream(Stream) { (void)device_sync(); }

  // A "kernel" that reads the blob at p and expects `want`.
  void launch(const void* p, std::vector<unsigned char> want) {
    enqueue([this, p, want] {
      std::lock_guard<std::mutex> l(mu);
      const char* c = (const char*)p;
      if (!is_live(c, want.size()) || memcmp(c, want.data(), want.size()) != 0) ++errors;
      ++launches;
    });
  }
};

std::vector<unsigned char> blob_of(uint32_t id) {
  std::vector<unsigned char> b(64 + (id * 2654435761u) % 3000);
  uint32_t x = id * 747796405u + 2891336453u;
  for (auto& c : b) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    c = (unsigned char)x;
  }
  return b;
}

}  // namespace

int main(int argc, char** argv) {
  const int threads = argc > 1 ? atoi(argv[1]) : 8;
  const int iters = argc > 2 ? atoi(argv[2]) : 20000;
  FakeDevice dev;
  // 12 blobs or 24 KiB per device, in 4 KiB chunks: the cache empties itself
  // every few calls.
  ps::BlobCache<FakeDevice> cache(dev, ps::BlobLimits{12, 24 << 10, 4 << 10});
  std::atomic<long> get_failures{0};
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t)
    pool.emplace_back([&, t] {
      std::mt19937 rng(1234 + t);
      for (int i = 0; i < iters; ++i) {
        const uint32_t id = rng() % 64;
        const int device = (int)(rng() % 2);
        std::vector<unsigned char> b = blob_of(id);
        ps::BlobCache<FakeDevice>::Lease lease(cache);
        const void* d = nullptr;
        if (cache.get(device, b.data(), b.size(), t, &d, lease) != 0) {
          ++get_failures;
          continue;
        }
        if (i % 3 == 0) std::this_thread::yield();   // widen the window between the pointer and the launch
        dev.launch(d, std::move(b));
      }
    });
  for (auto& th : pool) th.join();
  dev.device_sync();
  const long errors = dev.errors.load() + get_failures.load();
  printf("flushes=%zu launches=%ld errors=%ld\n", cache.flushes(), dev.launches.load(), errors);
  return errors == 0 && (long)cache.flushes() >= threads && dev.launches.load() == (long)threads * iters ? 0 : 1;
}
