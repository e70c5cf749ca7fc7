// Test driver for SlotRing (csrc/barrier_slots.h), the bookkeeping of the
// persistent launches' barrier slots, on the CPU under ThreadSanitizer.
//
// Several host threads take leases as callers on separate streams would. The
// fake event policy records, for every lease, which earlier lease its stream
// was made to wait for. The driver checks that
//   - no two leases of one slot are ever held at once;
//   - a slot's first lease waits for nothing, and every later lease waits for
//     exactly the lease that used the slot before it (so its zero-fill cannot
//     overtake the previous user's work);
//   - a failure to create the slot's event releases the slot, and the next
//     lease of that slot creates it.
// Prints "slot ring ok" and exits 0 on success.
#include <atomic>
#include <cstdio>
#include <thread>
#include <vector>

#include "barrier_slots.h"

namespace {

constexpr int kSlots = 8;
constexpr int kThreads = 8;
constexpr int kLeasesPerThread = 2000;

struct FakeEvent {
  std::atomic<long> recorded_by{-1};  // the lease whose release recorded it last
};
FakeEvent g_events[64];
std::atomic<int> g_next_event{0};
std::atomic<int> g_create_failures{0};  // creations still to fail

thread_local long t_lease = -1;   // the lease this thread is taking
thread_local long t_waited = -2;  // the lease its stream was made to wait for (-2: none)

struct FakeOps {
  using Event = int;
  using Stream = int;
  static int create(Event* e) {
    if (g_create_failures.fetch_sub(1) > 0) return 7;
    *e = g_next_event.fetch_add(1);
    return 0;
  }
  static int wait(Stream, Event e) {
    t_waited = g_events[e].recorded_by.load();
    return 0;
  }
  static int record(Event e, Stream) {
    g_events[e].recorded_by.store(t_lease);
    return 0;
  }
};

struct Use {
  long lease;
  long waited;
};

ddp::SlotRing<kSlots, FakeOps> g_ring;
std::vector<Use> g_history[kSlots];  // guarded by the slot's lease
std::atomic<int> g_busy[kSlots];
std::atomic<long> g_next_lease{0};
std::atomic<bool> g_ok{true};

void worker(int stream) {
  for (int i = 0; i < kLeasesPerThread; ++i) {
    t_lease = g_next_lease.fetch_add(1);
    t_waited = -2;
    ddp::SlotRing<kSlots, FakeOps>::Lease l;
    const int st = g_ring.acquire(stream, &l);
    if (st != 0) {
      if (st != 7) g_ok = false;  // only the injected failure is expected
      continue;
    }
    if (g_busy[l.slot].fetch_add(1) != 0) {
      std::fprintf(stderr, "driver: slot %d leased twice at once\n", l.slot);
      g_ok = false;
    }
    g_history[l.slot].push_back({t_lease, t_waited});
    g_busy[l.slot].fetch_sub(1);
    if (g_ring.release(&l, stream) != 0 || l.slot != -1) g_ok = false;
  }
}

}  // namespace

int main() {
  g_create_failures = 3;  // the first three event creations fail
  std::vector<std::thread> threads;
  for (int t = 0; t < kThreads; ++t) threads.emplace_back(worker, t);
  for (auto& th : threads) th.join();
  long leases = 0;
  for (int k = 0; k < kSlots; ++k) {
    const auto& h = g_history[k];
    leases += long(h.size());
    if (h.empty() || h[0].waited != -2) {
      std::fprintf(stderr, "driver: slot %d: first lease waited for %ld\n", k, h.empty() ? -3 : h[0].waited);
      g_ok = false;
    }
    for (size_t j = 1; j < h.size(); ++j) {
      if (h[j].waited != h[j - 1].lease) {
        std::fprintf(stderr, "driver: slot %d: lease %ld waited for %ld, not for %ld\n", k, h[j].lease,
                     h[j].waited, h[j - 1].lease);
        g_ok = false;
      }
    }
  }
  if (leases != long(kThreads) * kLeasesPerThread - 3) {
    std::fprintf(stderr, "driver: %ld leases succeeded\n", leases);
    g_ok = false;
  }
  if (g_next_event.load() != kSlots) g_ok = false;  // one event per slot, created once
  std::printf(g_ok ? "slot ring ok\n" : "slot ring FAILED\n");
  return g_ok ? 0 : 1;
}
