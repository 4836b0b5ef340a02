// Persistent host thread pool (see host_pool.h).
#include "host_pool.h"

#include <algorithm>
#include <condition_variable>
#include <mutex>
#include <thread>

namespace staple {
namespace {

struct Pool {
  std::mutex run_mu;                 // one job at a time
  std::mutex mu;                     // guards everything below
  std::condition_variable wake, done;
  void (*body)(void*, int64_t, int64_t) = nullptr;
  void* ctx = nullptr;
  int64_t n = 0;
  int parts = 0;
  int next = 0;                      // next part to take
  int finished = 0;                  // parts done
  uint64_t generation = 0;           // bumped per job
  int started = 0;                   // worker threads running

  // Takes parts of the current job until none is left; every field is read
  // under the lock, so a worker late from an earlier job sees the new one.
  void take_parts(std::unique_lock<std::mutex>& lk) {
    while (next < parts) {
      const int p = next++;
      void (*b)(void*, int64_t, int64_t) = body;
      void* c = ctx;
      const int64_t nn = n;
      const int pp = parts;
      lk.unlock();
      b(c, nn * p / pp, nn * (p + 1) / pp);
      lk.lock();
      if (++finished == pp) done.notify_all();
    }
  }

  void worker() {
    uint64_t seen = 0;
    std::unique_lock<std::mutex> lk(mu);
    for (;;) {
      wake.wait(lk, [&] { return generation != seen; });
      seen = generation;
      take_parts(lk);
    }
  }

  void ensure_workers(int want) {
    // the calling thread is one of the `want`
    // a thread that cannot be started leaves its parts to the others (the
    // calling thread takes parts too, so every job completes)
    while (started < want - 1) {
      try {
        std::thread(&Pool::worker, this).detach();
      } catch (...) {
        return;
      }
      ++started;
    }
  }
};

Pool& pool() {
  static Pool* p = new Pool();   // never destroyed: detached workers use it to the end
  return *p;
}

}  // namespace

int host_pool_parts(int64_t work_bytes, int cap) {
  const int hw = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  const int lim = std::max(1, std::min({cap, kHostPoolMax, hw}));
  const int64_t by_work = work_bytes >> 21;
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(lim, by_work)));
}

void host_pool_run(int64_t n, int threads, void (*body)(void*, int64_t, int64_t), void* ctx) {
  threads = std::max(1, std::min(threads, kHostPoolMax));
  if (n <= 0) return;
  if (threads == 1 || n == 1) {
    body(ctx, 0, n);
    return;
  }
  // several parts per thread, taken in turn: a thread the OS holds back
  // (other work on the host's cores) delays only the part it is on
  const int parts = static_cast<int>(std::min<int64_t>(n, static_cast<int64_t>(threads) * kPartsPerThread));
  Pool& P = pool();
  std::lock_guard<std::mutex> run_lk(P.run_mu);
  std::unique_lock<std::mutex> lk(P.mu);
  P.ensure_workers(threads);
  P.body = body;
  P.ctx = ctx;
  P.n = n;
  P.parts = parts;
  P.next = 0;
  P.finished = 0;
  ++P.generation;
  P.wake.notify_all();
  P.take_parts(lk);
  P.done.wait(lk, [&] { return P.finished == P.parts; });
}

}  // namespace staple
