// Persistent pool of host threads for the library's host-side loops (miss
// row packing, the host AdamW update).  The workers are started on the first
// call that needs them and live until the process ends, so a call spawns no
// thread and allocates nothing: the job is a function pointer and a context
// pointer handed to the waiting workers.
#pragma once

#include <stdint.h>

namespace staple {

// Runs body(ctx, lo, hi) over [0, n) on `threads` threads (at most
// kHostPoolMax, the calling thread one of them): [0, n) is cut into up to
// kPartsPerThread contiguous ranges per thread, which the threads take in
// turn; returns when every range is done.  Calls from several threads take
// turns.
constexpr int kHostPoolMax = 16;
constexpr int kPartsPerThread = 4;
void host_pool_run(int64_t n, int threads, void (*body)(void*, int64_t, int64_t), void* ctx);

// Threads a host loop of `work` bytes should use: one per 2 MB of work, at
// most `cap` (<= kHostPoolMax) and the host's hardware threads, at least one.
int host_pool_parts(int64_t work_bytes, int cap);

template <typename F>
void host_parallel_for(int64_t n, int threads, F& f) {
  host_pool_run(n, threads,
                [](void* c, int64_t lo, int64_t hi) { (*static_cast<F*>(c))(lo, hi); }, &f);
}

}  // namespace staple
