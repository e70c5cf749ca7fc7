// Bookkeeping of a device's persistent-barrier slots (host code only).
//
// A persistent launch needs a few words of device memory that start at zero
// and that no other launch touches while it runs: its grid barrier's arrival
// counter and tile tickets. A device has K such slots, handed out round-robin.
// A slot is reused after K further launches, possibly by a launch on another
// stream; that launch must not clear the slot before the previous user's work
// (the persistent kernel, and whatever reads the slot after it) has finished.
//
// SlotRing makes that so:
//   - acquire() takes the next slot, holds the slot's lock for the lease, and
//     enqueues on the caller's stream a wait for the event that the slot's
//     previous lease recorded when it was released (stream order, not a host
//     wait);
//   - release() records the slot's event on the caller's stream, after all the
//     work enqueued under the lease, and unlocks the slot.
// The lock keeps two host threads that reach the same slot from interleaving
// their wait and record; it is held only between acquire and release, i.e.
// while one call enqueues its kernels.
//
// Ops supplies the event type and operations (HIP events in the library, a
// recording fake in the CPU test):
//   typename Ops::Event, typename Ops::Stream;
//   static int create(Event*);                    // 0 on success
//   static int wait(Stream, Event);               // stream waits for event
//   static int record(Event, Stream);             // event marks stream's position
#pragma once

#include <atomic>
#include <mutex>

namespace ddp {

template <int K, class Ops>
class SlotRing {
 public:
  using Event = typename Ops::Event;
  using Stream = typename Ops::Stream;

  struct Lease {
    int slot = -1;
    SlotRing* ring = nullptr;
  };

  // Takes slot (next++ mod K) for the caller; on success the caller must call
  // release() once its work on the slot is enqueued (also after a failure to
  // enqueue it). Returns 0, or the failing operation's status (nothing held).
  int acquire(Stream stream, Lease* lease) {
    const int k = int(next_.fetch_add(1u) % unsigned(K));
    slot_mu_[k].lock();
    int st = 0;
    if (!has_event_[k]) {
      st = Ops::create(&event_[k]);
      if (st == 0) has_event_[k] = true;
    } else if (used_[k]) {
      st = Ops::wait(stream, event_[k]);
    }
    if (st != 0) {
      slot_mu_[k].unlock();
      return st;
    }
    lease->slot = k;
    lease->ring = this;
    return 0;
  }

  // Records the end of the lease's work on `stream` and frees the slot for
  // its next user. Returns the record's status (the slot is freed either way).
  int release(Lease* lease, Stream stream) {
    const int k = lease->slot;
    if (k < 0) return 0;
    const int st = Ops::record(event_[k], stream);
    used_[k] = st == 0;  // a failed record leaves nothing to wait for
    lease->slot = -1;
    slot_mu_[k].unlock();
    return st;
  }

 private:
  std::atomic<unsigned> next_{0};
  std::mutex slot_mu_[K];
  Event event_[K] = {};
  bool has_event_[K] = {};
  bool used_[K] = {};
};

}  // namespace ddp
