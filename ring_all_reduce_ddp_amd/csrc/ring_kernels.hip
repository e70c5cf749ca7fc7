// Step-faithful ring all-reduce over N virtual ranks held in one GPU's HBM.
//
// Method (page "DDP 与 Ring All-Reduce", blog.vllbc.top, section 03; page "DDP 与
// Ring-AllReduce", xuesongtap.github.io, §1.3.1 and the worked example of
// §1.3.2): the buffer is cut into N chunks of L = ceil(count/N) elements.
// Reduce-scatter: N-1 steps; in step s rank r passes chunk (r-1-s) mod N to
// rank r+1, which adds it into its own copy. All-gather: N-1 steps; in step s
// rank r passes chunk (r-s) mod N and rank r+1 overwrites its copy. Chunk c
// thus starts at rank c+1, collects ranks c+2, ..., c, one rounded add per
// hop, and ends complete on rank c, from where it travels on unchanged.
//
// Two forms run the steps as steps (the one-pass form is in fused_kernels.hip):
//   * ring_allreduce_step: one launch per step, covering all N transfers of
//     the step. Within a step the N transfers touch disjoint chunks (rank r
//     writes chunk (r-1-s) of rank r+1 and reads chunk (r-1-s) of rank r, which
//     no other transfer of the step writes), so one launch may run them all.
//   * ring_allreduce_persistent: all steps in one cooperative launch, with a
//     grid-wide barrier between steps (the per-step synchronisation of a real
//     ring).
//
// Both stream 16-byte vectors when the rank buffers are 16-byte aligned, and
// fall back to one element per thread otherwise. A block works on tiles of
// one chunk, on a grid aligned to whole tiles of the buffer; a vector that a
// chunk boundary cuts (chunk lengths that are not whole vectors) is done
// element by element, this chunk's elements only. No LDS and no matrix
// cores: nothing here is reused across threads or shaped like a contraction.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "ring_common.h"

namespace ddp {
namespace {

constexpr int kStepUnroll = 4;    // 16-byte vectors per thread in a step tile
constexpr int64_t kDefaultTimeoutUs = 10 * 1000 * 1000;  // grid barrier patience: 10 s
// Persistent grid, measured on MI355X (14 steps, 8 ranks): 1024-thread blocks.
// Buffers beyond the Infinity Cache, tiles handed out by tickets: seven
// blocks for every eight compute units (224). With the split barrier whose
// waiters poll a release word, 8 x 256 MiB fp32 took 1.62 ms at 224 blocks
// (16 to 256 blocks: 11.8, 6.09, 3.25, 2.36, 2.02, 1.80, 1.67, 1.62, 1.64 ms).
// Buffers inside it (cached accesses, a fixed share per block): five blocks
// for every eight compute units (160), rounded so that every block has the
// same number of tiles per step (a step ends when its slowest block does):
// 8 x 25 MiB took 0.248 ms at 160 blocks (16 to 256: 0.771, 0.433, 0.286,
// 0.257, 0.256, 0.248, 0.268, 0.258, 0.273 ms). Fewer blocks leave bandwidth
// unused; more add barrier arrivals and, with cached stores, write-backs of
// dirty cache lines at every barrier.
constexpr int kPersistentThreads = 1024;   // threads per persistent block
constexpr int kPersistentBlocksPer8CUsStreaming = 7;
constexpr int kPersistentBlocksPer8CUsCached = 5;

// ---------------------------------------------------------------- one step

// The step kernels stream 16-byte vectors whenever every rank buffer starts
// on a 16-byte boundary; a vector cut by a chunk boundary (chunk lengths
// that are not whole vectors) is done element by element.
inline bool step_vec(const RingArgs& a) { return all_aligned16(const_cast<void* const*>(a.P.p), a.n); }

// Chunk that rank r passes on in step s of `phase`.
__device__ __forceinline__ int step_chunk(int r, int s, int n, int phase) {
  int c = (phase == DDP_RS ? r - 1 - s : r - s) % n;
  return c < 0 ? c + n : c;
}

// One tile of one step: transfer r -> r+1 of chunk step_chunk(r, s). A tile
// is T threads x U 16-byte vectors (VEC) or T elements (!VEC); NT selects
// non-temporal loads and stores.
template <int DT, bool VEC, int T, int U, bool NT>
__device__ __forceinline__ void step_tile(const RankPtrs& P, int n, int64_t count, int64_t L,
                                          int64_t tiles_per_chunk, int64_t tile, int s, int phase) {
  using O = Ops<DT>;
  constexpr int V = VEC ? O::V : 1;
  constexpr int64_t kTile = int64_t(T) * (VEC ? U : 1) * V;
  const int r = int(tile / tiles_per_chunk);
  const int c = step_chunk(r, s, n, phase);
  const int64_t lo = int64_t(c) * L;
  const int64_t hi = min(lo + L, count);
  // Tiles sit on a grid aligned to whole tiles (not to chunk starts), so
  // waves touch whole cache lines even when chunks start between lines.
  const int64_t base = (lo / kTile + (tile - int64_t(r) * tiles_per_chunk)) * kTile;
  if (base >= hi) return;
  const void* src = P.p[r];
  void* dst = P.p[wrap(r + 1, n)];
  if constexpr (VEC) {
    u32x4 a[U], b[U];
    int64_t vi[U];
    bool full[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vi[u] = base / V + int64_t(u) * T + threadIdx.x;
      full[u] = vi[u] * V >= lo && (vi[u] + 1) * V <= hi;
      if (full[u]) {
        a[u] = ld16<NT>(static_cast<const u32x4*>(src) + vi[u]);
        if (phase == DDP_RS) b[u] = ld16<NT>(static_cast<const u32x4*>(dst) + vi[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (full[u]) {
        u32x4 y = a[u];
        if (phase == DDP_RS) {
          typename O::Acc acc = O::from(a[u]);
          O::add(acc, b[u]);
          y = O::to(acc);
        }
        st16<NT>(static_cast<u32x4*>(dst) + vi[u], y);
      } else if ((vi[u] + 1) * V > lo && vi[u] * V < hi) {
        // A vector cut by a chunk boundary (chunk lengths that are not whole
        // vectors) or by the end of the buffer: this chunk's elements only.
        const int64_t e0 = vi[u] * V;
        for (int64_t e = max(e0, lo); e < hi && e < e0 + V; ++e) {
          const float x = O::load1(src, e);
          O::store1(dst, e, phase == DDP_RS ? O::add1(x, O::load1(dst, e)) : x);
        }
      }
    }
  } else {
    const int64_t e = base + threadIdx.x;
    if (e >= lo && e < hi) {
      const float x = O::load1(src, e);
      O::store1(dst, e, phase == DDP_RS ? O::add1(x, O::load1(dst, e)) : x);
    }
  }
}

// The vector form of one tile, in two halves, so that a loop over tiles can
// issue the next tile's loads before the current tile's stores: within a step
// no tile reads what another tile of the step writes (transfer r writes chunk
// (r-1-s) of rank r+1, which only transfer r itself reads), so the order of
// one tile's stores and another's loads does not matter.
template <int U>
struct StagedTile {
  u32x4 a[U], b[U];  // sent operand, and the receiver's own (reduce-scatter only)
  int64_t base = 0, lo = 0, hi = 0;  // the tile's first element; the chunk's range
  int r = 0;                          // the sending rank
};

// Where tile `tile` of step s lies: sending rank, chunk range, first element.
template <int DT, int T, int U>
__device__ __forceinline__ void step_tile_place(int n, int64_t count, int64_t L, int64_t tiles_per_chunk,
                                                int64_t tile, int s, int phase, StagedTile<U>& t) {
  constexpr int64_t kTile = int64_t(T) * U * Ops<DT>::V;
  t.r = int(tile / tiles_per_chunk);
  const int c = step_chunk(t.r, s, n, phase);
  t.lo = int64_t(c) * L;
  t.hi = min(t.lo + L, count);
  t.base = (t.lo / kTile + (tile - int64_t(t.r) * tiles_per_chunk)) * kTile;
}

// The sent operand (rank r's copy of the chunk), whole vectors only.
template <int DT, int T, int U, bool NT>
__device__ __forceinline__ void step_tile_load_sent(const RankPtrs& P, StagedTile<U>& t) {
  constexpr int V = Ops<DT>::V;
  if (t.base >= t.hi) return;
  const u32x4* src = static_cast<const u32x4*>(P.p[t.r]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t vi = t.base / V + int64_t(u) * T + threadIdx.x;
    if (vi * V >= t.lo && (vi + 1) * V <= t.hi) t.a[u] = ld16<NT>(src + vi);
  }
}

// The receiver's own copy of the chunk, which a reduce-scatter step adds to.
// In reduce-scatter step s it has not been written by any earlier step (rank
// r+1 receives chunk (r-1-s) in step s and in no other reduce-scatter step),
// so it may be loaded before the barrier that ends step s-1 completes.
template <int DT, int T, int U, bool NT>
__device__ __forceinline__ void step_tile_load_own(const RankPtrs& P, int n, StagedTile<U>& t) {
  constexpr int V = Ops<DT>::V;
  if (t.base >= t.hi) return;
  const u32x4* dst = static_cast<const u32x4*>(P.p[wrap(t.r + 1, n)]);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t vi = t.base / V + int64_t(u) * T + threadIdx.x;
    if (vi * V >= t.lo && (vi + 1) * V <= t.hi) t.b[u] = ld16<NT>(dst + vi);
  }
}

template <int DT, int T, int U, bool NT>
__device__ __forceinline__ void step_tile_load(const RankPtrs& P, int n, int64_t count, int64_t L,
                                               int64_t tiles_per_chunk, int64_t tile, int s, int phase,
                                               StagedTile<U>& t) {
  step_tile_place<DT, T, U>(n, count, L, tiles_per_chunk, tile, s, phase, t);
  step_tile_load_sent<DT, T, U, NT>(P, t);
  if (phase == DDP_RS) step_tile_load_own<DT, T, U, NT>(P, n, t);
}

template <int DT, int T, int U, bool NT>
__device__ __forceinline__ void step_tile_finish(const RankPtrs& P, int n, int phase, const StagedTile<U>& t) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  if (t.base >= t.hi) return;
  const void* src = P.p[t.r];
  void* dst = P.p[wrap(t.r + 1, n)];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t vi = t.base / V + int64_t(u) * T + threadIdx.x;
    if (vi * V >= t.lo && (vi + 1) * V <= t.hi) {
      u32x4 y = t.a[u];
      if (phase == DDP_RS) {
        typename O::Acc acc = O::from(t.a[u]);
        O::add(acc, t.b[u]);
        y = O::to(acc);
      }
      st16<NT>(static_cast<u32x4*>(dst) + vi, y);
    } else if ((vi + 1) * V > t.lo && vi * V < t.hi) {
      // cut by a chunk boundary or the buffer's end: this chunk's elements only
      const int64_t e0 = vi * V;
      for (int64_t e = max(e0, t.lo); e < t.hi && e < e0 + V; ++e) {
        const float x = O::load1(src, e);
        O::store1(dst, e, phase == DDP_RS ? O::add1(x, O::load1(dst, e)) : x);
      }
    }
  }
}

// Launch shape of the step kernels, measured on MI355X at 8 ranks: one wave
// per block, one 16-byte vector per thread, one tile per block. When the N
// buffers together exceed the 256 MB Infinity Cache the loads and stores are
// non-temporal (8 x 1 GiB: 5.66 ms for the 14 steps vs 6.04 ms cached); when
// they fit, cached accesses let step s+1 read what step s wrote from the cache
// (8 x 25 MiB: 0.15 ms vs 0.18 ms non-temporal).
constexpr int kStepThreads = 64;

template <int DT, bool VEC, int PHASE, bool NT>
__global__ __launch_bounds__(kStepThreads) void k_step(RankPtrs P, int n, int64_t count, int64_t L,
                                                       int64_t tiles_per_chunk, int64_t total_tiles, int s) {
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x)
    step_tile<DT, VEC, kStepThreads, 1, NT>(P, n, count, L, tiles_per_chunk, tile, s, PHASE);
}

// ---------------------------------------------------------------- persistent

// A launch's barrier slot (kSlotWords words, zeroed before the launch), one
// 128-byte line per word in use:
//   word 0:              arrivals over the whole launch; top bit: abort flag
//   word kTicketWord:    the tile-ticket counter
//   word kReleaseWord:   barriers completed; top bit: abort flag
// Arriving blocks add to word 0 and only the last one of a barrier writes the
// release word, which the waiting blocks poll: the polls never contend with
// the arrivals' atomics on one line.
constexpr int kTicketWord = 32;
constexpr int kReleaseWord = 64;

// Grid-wide barrier for a cooperative launch, in two halves so that a block
// can issue loads that do not depend on the other blocks' writes (the next
// reduce-scatter step's own operand) between its arrival and its wait.
// Barrier number g (from 1) completes when g * gridDim.x + extra blocks have
// arrived; `extra` is non-zero only when a test forces the time-out path.
__device__ __forceinline__ void barrier_arrive(unsigned int* words, unsigned int target, unsigned int g) {
  __syncthreads();  // every wave of the block has issued its stores of the step
  if (threadIdx.x == 0) {
    // Release at agent scope (an L2 write-back on this part): the block's
    // writes become visible to every XCD before its arrival is counted.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned int prev = __hip_atomic_fetch_add(words, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1u == target) {
      // The last arrival (never after an abort: the abort bit makes prev
      // larger): it has seen every other block's arrival, so after an acquire
      // it can release them all to the waiters. fetch_max keeps an abort bit.
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_fetch_max(words + kReleaseWord, g, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Waits until barrier g is released. A block that has waited longer than
// `deadline` wall-clock ticks sets the abort bit in words 0 and kReleaseWord,
// records what it saw in status[0..2] (timed out, arrivals seen, arrivals
// expected), and every block then leaves. Returns false if the launch must stop.
__device__ __forceinline__ bool barrier_wait(unsigned int* words, unsigned int target, unsigned int g,
                                             unsigned int* status, unsigned long long deadline) {
  __shared__ int ok;
  if (threadIdx.x == 0) {
    unsigned int* release = words + kReleaseWord;
    unsigned int seen = __hip_atomic_load(release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long t0 = wall_clock64();
    while ((seen & kAbortBit) == 0u && seen < g) {
      __builtin_amdgcn_s_sleep(2);
      seen = __hip_atomic_load(release, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((seen & kAbortBit) == 0u && seen < g && wall_clock64() - t0 > deadline) {
        const unsigned int prev =
            __hip_atomic_fetch_or(words, kAbortBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(release, kAbortBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(&status[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(&status[1], prev & ~kAbortBit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(&status[2], target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        seen = kAbortBit;
      }
    }
    // Acquire at agent scope (a cache invalidate): the other blocks' writes
    // are visible to the loads that follow the barrier.
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    ok = (seen & kAbortBit) == 0u;
  }
  __syncthreads();
  return ok != 0;
}

// All n_steps steps, a grid barrier between consecutive ones. `extra` is
// added to every barrier's expected arrival count; it is non-zero only when
// a test forces the time-out path.
template <int DT, bool VEC, bool NT>
__global__ __launch_bounds__(kPersistentThreads) void k_persistent(RankPtrs P, int n, int64_t count, int64_t L,
                                                         int64_t tiles_per_chunk, int n_steps,
                                                         unsigned int* counter, unsigned int* status,
                                                         unsigned long long deadline, unsigned int extra) {
  const int64_t total_tiles = int64_t(n) * tiles_per_chunk;
  if constexpr (NT && VEC) {
    // Tiles handed out by one ticket counter for the whole launch: tickets
    // [i * total, (i + 1) * total) are step i's tiles. A block takes its next
    // ticket while it works on the current tile; the one ticket past its
    // step that every block ends a step holding is a tile of the next step,
    // since the grid never exceeds one step's tiles. Thread 0 draws, and a
    // double-buffered LDS word passes the ticket to the block with one
    // barrier per tile. Between its arrival at a barrier and its wait, a
    // block loads the own operand of that next tile if the next step is a
    // reduce-scatter step.
    unsigned int* tickets = counter + kTicketWord;
    __shared__ unsigned int next_ticket[2];
    if (threadIdx.x == 0)
      next_ticket[0] = __hip_atomic_fetch_add(tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    unsigned int t = next_ticket[0];
    int k = 1;
    StagedTile<kStepUnroll> cur;
    bool own_loaded = false;  // cur holds the own operand of ticket t (loaded across a barrier)
    for (int i = 0; i < n_steps; ++i) {
      const int phase = i < n - 1 ? DDP_RS : DDP_AG;
      const int s = i < n - 1 ? i : i - (n - 1);
      const unsigned int end = unsigned(i + 1) * unsigned(total_tiles);
      while (t < end) {
        unsigned int drawn = 0u;
        if (threadIdx.x == 0)
          drawn = __hip_atomic_fetch_add(tickets, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (own_loaded) {
          step_tile_load_sent<DT, kPersistentThreads, kStepUnroll, NT>(P, cur);
        } else {
          step_tile_load<DT, kPersistentThreads, kStepUnroll, NT>(P, n, count, L, tiles_per_chunk,
                                                                  int64_t(t) - int64_t(i) * total_tiles, s, phase,
                                                                  cur);
        }
        own_loaded = false;
        step_tile_finish<DT, kPersistentThreads, kStepUnroll, NT>(P, n, phase, cur);
        if (threadIdx.x == 0) next_ticket[k & 1] = drawn;
        __syncthreads();
        t = next_ticket[k & 1];
        ++k;
      }
      if (i + 1 < n_steps) {
        const unsigned int target = unsigned(i + 1) * gridDim.x + extra;
        barrier_arrive(counter, target, unsigned(i + 1));
        if (i + 1 < n - 1 && t < end + unsigned(total_tiles)) {  // the next step reduces: its own operand
          step_tile_place<DT, kPersistentThreads, kStepUnroll>(n, count, L, tiles_per_chunk,
                                                               int64_t(t) - int64_t(end), i + 1, DDP_RS, cur);
          step_tile_load_own<DT, kPersistentThreads, kStepUnroll, NT>(P, n, cur);
          own_loaded = true;
        }
        if (!barrier_wait(counter, target, unsigned(i + 1), status, deadline)) return;
      }
    }
  } else {
    // Buffers inside the Infinity Cache: a fixed grid-stride share per block
    // (tickets measured 1-2 % slower here: 8 x 25 MiB 0.299-0.301 against
    // 0.295-0.297 ms at 96 blocks). With whole vectors, the next tile's loads
    // are issued before the current tile's stores, so a block keeps two
    // tiles' loads in flight, and between its arrival at a barrier and its
    // wait it loads its first tile's own operand if the next step reduces.
    bool own_loaded = false;
    StagedTile<kStepUnroll> cur, nxt;
    for (int i = 0; i < n_steps; ++i) {
      const int phase = i < n - 1 ? DDP_RS : DDP_AG;
      const int s = i < n - 1 ? i : i - (n - 1);
      if constexpr (VEC) {
        int64_t tile = blockIdx.x;
        if (tile < total_tiles) {
          if (own_loaded)
            step_tile_load_sent<DT, kPersistentThreads, kStepUnroll, NT>(P, cur);
          else
            step_tile_load<DT, kPersistentThreads, kStepUnroll, NT>(P, n, count, L, tiles_per_chunk, tile, s,
                                                                    phase, cur);
        }
        own_loaded = false;
        while (tile < total_tiles) {
          const int64_t next = tile + gridDim.x;
          if (next < total_tiles)
            step_tile_load<DT, kPersistentThreads, kStepUnroll, NT>(P, n, count, L, tiles_per_chunk, next, s,
                                                                    phase, nxt);
          step_tile_finish<DT, kPersistentThreads, kStepUnroll, NT>(P, n, phase, cur);
          cur = nxt;
          tile = next;
        }
      } else {
        for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x)
          step_tile<DT, VEC, kPersistentThreads, kStepUnroll, NT>(P, n, count, L, tiles_per_chunk, tile, s, phase);
      }
      if (i + 1 < n_steps) {
        const unsigned int target = unsigned(i + 1) * gridDim.x + extra;
        barrier_arrive(counter, target, unsigned(i + 1));
        if constexpr (VEC) {
          if (i + 1 < n - 1 && int64_t(blockIdx.x) < total_tiles) {  // the next step reduces: own operand
            step_tile_place<DT, kPersistentThreads, kStepUnroll>(n, count, L, tiles_per_chunk, blockIdx.x, i + 1,
                                                                 DDP_RS, cur);
            step_tile_load_own<DT, kPersistentThreads, kStepUnroll, NT>(P, n, cur);
            own_loaded = true;
          }
        }
        if (!barrier_wait(counter, target, unsigned(i + 1), status, deadline)) return;
      }
    }
  }
}

// ---------------------------------------------------------------- allocation-free scratch

// Barrier words of ring_allreduce_persistent_noalloc, for callers that cannot
// allocate device memory: words [0, 128) are one launch's barrier slot (the
// layout above), words [128, 131) its sticky status (timed out, arrivals
// seen, arrivals expected). 1 KiB per device, zero when the code object is
// loaded, held until the process ends.
constexpr int kNoAllocSlotWords = kSlotWords;
constexpr int kNoAllocWords = 256;
static __device__ __align__(256) unsigned int scratch[kNoAllocWords];

// The device address of `scratch` on each device. In host code the array's
// name is only a stand-in for the symbol; the address comes from
// hipGetSymbolAddress, fetched once per device with that device current.
std::mutex g_noalloc_mu;
unsigned int* g_noalloc_words[kMaxDevices] = {};

int noalloc_scratch(unsigned int** out) {
  int dev = 0;
  DDP_HIP_TRY(hipGetDevice(&dev), "ring_allreduce_persistent_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DDP_EINVAL, "ring_allreduce_persistent_noalloc: device index beyond 64");
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  if (g_noalloc_words[dev] == nullptr) {
    void* p = nullptr;
    DDP_HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)),
                "ring_allreduce_persistent_noalloc: hipGetSymbolAddress");
    g_noalloc_words[dev] = static_cast<unsigned int*>(p);
  }
  *out = g_noalloc_words[dev];
  return DDP_OK;
}

// ---------------------------------------------------------------- host side

// Tiles per chunk of the persistent kernel: 1024 threads x kStepUnroll
// vectors, or x 1 element (buffers not 16-byte aligned).
template <int DT, bool VEC>
int64_t step_tiles_per_chunk(const RingArgs& a) {
  const int64_t tile = VEC ? int64_t(kPersistentThreads) * kStepUnroll * Ops<DT>::V : int64_t(kPersistentThreads);
  return aligned_tiles_per_chunk(a.L, tile);
}

template <int DT, bool VEC, bool NT>
int launch_step_impl(const RingArgs& a, int step, int phase, hipStream_t s) {
  const int64_t tile = VEC ? int64_t(kStepThreads) * Ops<DT>::V : kStepThreads;
  const int64_t tpc = aligned_tiles_per_chunk(a.L, tile);
  const int64_t total = tpc * a.n;
  const dim3 g(grid_for(total)), b(kStepThreads);
  if (phase == DDP_RS)
    hipLaunchKernelGGL((k_step<DT, VEC, DDP_RS, NT>), g, b, 0, s, a.P, a.n, a.count, a.L, tpc, total, step);
  else
    hipLaunchKernelGGL((k_step<DT, VEC, DDP_AG, NT>), g, b, 0, s, a.P, a.n, a.count, a.L, tpc, total, step);
  DDP_HIP_TRY(hipGetLastError(), "ring_allreduce_step: launch");
  return DDP_OK;
}

template <int DT>
int launch_step(const RingArgs& a, int step, int phase, hipStream_t s) {
  const bool nt = int64_t(a.n) * a.count * elem_bytes(DT) > kInfinityCacheBytes;
  if (step_vec(a))
    return nt ? launch_step_impl<DT, true, true>(a, step, phase, s) : launch_step_impl<DT, true, false>(a, step, phase, s);
  return nt ? launch_step_impl<DT, false, true>(a, step, phase, s) : launch_step_impl<DT, false, false>(a, step, phase, s);
}

// Test hook (ddp_persistent_test_hook): when set, the persistent launches that
// take default options expect this many more arrivals at every barrier and
// give up after this many microseconds, so tests can drive the time-out path
// of ddp_sync and the reducer from the host.
std::atomic<uint32_t> g_hook_extra{0};
std::atomic<int64_t> g_hook_timeout_us{0};

struct PersistentOpts {
  int32_t max_blocks = 0;       // 0: the default grid (see persistent_grid)
  int64_t timeout_us = kDefaultTimeoutUs;
  uint32_t extra_arrivals = 0;  // test hook: forces the time-out path
  bool noalloc = false;         // barrier words in the file-scope scratch, not library allocations
  unsigned int* words = nullptr;   // barrier words leased (and zeroed) by the caller, if not NULL
  unsigned int* status = nullptr;  // with `words`: the status line of the lease

  // Default options, or the test hook's if it is set.
  static PersistentOpts defaults() {
    PersistentOpts o;
    const int64_t t = g_hook_timeout_us.load();
    if (t > 0) {
      o.timeout_us = t;
      o.extra_arrivals = g_hook_extra.load();
    }
    return o;
  }
};

// Grid of the persistent kernel: the default above for the buffers' cache
// regime (or max_blocks if > 0), never more than one block per tile of a step,
// and never more than (occupancy - 1) blocks per compute unit. The headroom
// is measured, not cosmetic: on MI355X the occupancy query reported 8 blocks
// per CU for this kernel with 256-thread blocks, yet a 2048-block cooperative
// grid had only 1792 blocks (7 per CU) running at the first barrier; the
// other 256 could not start until those left, so the barrier could never
// complete. (With 1024-thread blocks the query reports 1 per CU, its
// register limit, and the clamp is then one block per CU.)
template <int DT, bool VEC, bool NT>
int persistent_grid(const RingArgs& a, int32_t max_blocks, unsigned* grid, int* cus) {
  const int64_t total = step_tiles_per_chunk<DT, VEC>(a) * a.n;
  const void* fn = reinterpret_cast<const void*>(&k_persistent<DT, VEC, NT>);
  int dev = 0, per_cu = 0;
  DDP_HIP_TRY(hipGetDevice(&dev), "ring_allreduce_persistent: hipGetDevice");
  DDP_HIP_TRY(hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev),
              "ring_allreduce_persistent: multiprocessor count");
  DDP_HIP_TRY(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kPersistentThreads, 0),
              "ring_allreduce_persistent: occupancy");
  if (per_cu < 1 || *cus < 1)
    return fail(DDP_ENORESOURCE, "ring_allreduce_persistent: no block can be resident");
  const int64_t safe = int64_t(per_cu > 1 ? per_cu - 1 : 1) * (*cus);
  const int per8 = NT ? kPersistentBlocksPer8CUsStreaming : kPersistentBlocksPer8CUsCached;
  const int64_t want = max_blocks > 0 ? int64_t(max_blocks) : std::max<int64_t>(1, int64_t(per8) * (*cus) / 8);
  int64_t g = std::max<int64_t>(1, std::min({total, want, safe}));
  // A fixed share per block: as few blocks as give each block the same
  // number of tiles per step (tickets balance the load by themselves).
  if (!NT && max_blocks == 0) g = (total + (total + g - 1) / g - 1) / ((total + g - 1) / g);
  *grid = unsigned(g);
  return DDP_OK;
}

template <int DT, bool VEC, bool NT>
int launch_persistent_impl(const RingArgs& a, int n_steps, const PersistentOpts& o, hipStream_t s) {
  const int64_t tpc = step_tiles_per_chunk<DT, VEC>(a);
  const void* fn = reinterpret_cast<const void*>(&k_persistent<DT, VEC, NT>);
  int dev = 0, clock_khz = 0, cus = 0;
  unsigned grid = 0;
  int st = persistent_grid<DT, VEC, NT>(a, o.max_blocks, &grid, &cus);
  if (st != DDP_OK) return st;
  // Tickets are 32-bit: every tile of every step, plus one per block.
  if (int64_t(n_steps) * tpc * a.n + grid >= (int64_t(1) << 32))
    return fail(DDP_EINVAL, "ring_allreduce_persistent: too many tiles for one launch");
  DDP_HIP_TRY(hipGetDevice(&dev), "ring_allreduce_persistent: hipGetDevice");
  DDP_HIP_TRY(hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, dev),
              "ring_allreduce_persistent: wall clock rate");
  unsigned int* slot = nullptr;
  unsigned int* status = nullptr;
  BarrierGuard lease(s);  // barrier words leased here, unless the caller holds them
  if (o.words != nullptr) {
    slot = o.words;
    status = o.status;
  } else if (o.noalloc) {
    unsigned int* words = nullptr;
    st = noalloc_scratch(&words);
    if (st != DDP_OK) return st;
    st = zero_words(words, kNoAllocSlotWords, s);  // the status words stay: they are sticky
    if (st != DDP_OK) return st;
    slot = words;
    status = words + kNoAllocSlotWords;
  } else {
    st = lease.acquire();
    if (st != DDP_OK) return st;
    slot = lease.words();
    status = lease.status();
  }
  RankPtrs P = a.P;
  int n = a.n;
  int64_t count = a.count, L = a.L, tiles = tpc;
  int steps = n_steps;
  unsigned long long deadline =
      (unsigned long long)(std::max<int64_t>(clock_khz, 1)) * (unsigned long long)(o.timeout_us) / 1000ull;
  unsigned int extra = o.extra_arrivals;
  void* args[] = {&P, &n, &count, &L, &tiles, &steps, &slot, &status, &deadline, &extra};
  hipError_t e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kPersistentThreads), args, 0, s);
  if (e == hipErrorCooperativeLaunchTooLarge) {
    (void)hipGetLastError();
    return fail(DDP_ENORESOURCE, "ring_allreduce_persistent: grid cannot be co-resident");
  }
  if (e != hipSuccess) return hip_fail(e, "ring_allreduce_persistent: hipLaunchCooperativeKernel");
  return lease.release();
}

int persistent(const char* fn, void* const* bufs, int32_t N, int64_t count, int32_t dtype, int32_t n_steps,
               const PersistentOpts& o, void* stream) {
  if (N >= 1 && N <= DDP_MAX_RANKS && (n_steps < 0 || n_steps > 2 * (N - 1)))
    return fail(DDP_EINVAL, std::string(fn) + ": n_steps must lie in [0, 2(N-1)]");
  if (o.max_blocks < 0) return fail(DDP_EINVAL, std::string(fn) + ": max_blocks < 0");
  if (o.timeout_us <= 0 || o.timeout_us > int64_t(3600) * 1000000)
    return fail(DDP_EINVAL, std::string(fn) + ": timeout_us must lie in (0, 3600 s]");
  RingArgs a;
  int st = prepare(fn, bufs, N, count, dtype, &a);
  if (st != DDP_OK) return st;
  if (count == 0 || n_steps == 0) return DDP_OK;
  hipStream_t s = as_stream(stream);
  const bool nt = int64_t(a.n) * a.count * elem_bytes(dtype) > kInfinityCacheBytes;
  if (dtype == DDP_FP32) {
    if (step_vec(a)) return nt ? launch_persistent_impl<DDP_FP32, true, true>(a, n_steps, o, s)
                         : launch_persistent_impl<DDP_FP32, true, false>(a, n_steps, o, s);
    return launch_persistent_impl<DDP_FP32, false, false>(a, n_steps, o, s);
  }
  if (step_vec(a)) return nt ? launch_persistent_impl<DDP_BF16, true, true>(a, n_steps, o, s)
                       : launch_persistent_impl<DDP_BF16, true, false>(a, n_steps, o, s);
  return launch_persistent_impl<DDP_BF16, false, false>(a, n_steps, o, s);
}

}  // namespace

int persistent_allreduce_leased(void* const* bufs, int32_t N, int64_t count, int32_t dtype, unsigned int* words,
                                unsigned int* status, hipStream_t s) {
  PersistentOpts o = PersistentOpts::defaults();
  o.words = words;
  o.status = status;
  return persistent("ring_allreduce_persistent", bufs, N, count, dtype, N >= 1 ? 2 * (N - 1) : 0, o, s);
}

unsigned int* noalloc_status_words(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  return g_noalloc_words[dev] == nullptr ? nullptr : g_noalloc_words[dev] + kNoAllocSlotWords;
}

}  // namespace ddp

using namespace ddp;

extern "C" int ring_allreduce_step(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                   int32_t step, int32_t phase, void* stream) {
  const char* fn = "ring_allreduce_step";
  if (phase != DDP_RS && phase != DDP_AG) return fail(DDP_EINVAL, std::string(fn) + ": unknown phase");
  if (N >= 1 && N <= DDP_MAX_RANKS && (step < 0 || step > N - 2))
    return fail(DDP_EINVAL, std::string(fn) + ": step must lie in [0, N-2]");
  RingArgs a;
  int st = prepare(fn, bufs, N, count, dtype, &a);
  if (st != DDP_OK) return st;
  if (count == 0) return DDP_OK;
  return dtype == DDP_FP32 ? launch_step<DDP_FP32>(a, step, phase, as_stream(stream))
                           : launch_step<DDP_BF16>(a, step, phase, as_stream(stream));
}

extern "C" int ring_allreduce_persistent(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                         int32_t n_steps, void* stream) {
  return persistent("ring_allreduce_persistent", bufs, N, count, dtype, n_steps, PersistentOpts::defaults(), stream);
}

extern "C" int ddp_persistent_test_hook(uint32_t extra_arrivals, int64_t timeout_us) {
  if (timeout_us < 0 || timeout_us > int64_t(3600) * 1000000)
    return fail(DDP_EINVAL, "ddp_persistent_test_hook: timeout_us must lie in [0, 3600 s]");
  g_hook_extra.store(timeout_us > 0 ? extra_arrivals : 0u);
  g_hook_timeout_us.store(timeout_us);
  return DDP_OK;
}

extern "C" int ring_allreduce_persistent_noalloc(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                                 int32_t n_steps, void* stream) {
  PersistentOpts o = PersistentOpts::defaults();
  o.noalloc = true;
  return persistent("ring_allreduce_persistent_noalloc", bufs, N, count, dtype, n_steps, o, stream);
}

extern "C" int ddp_persistent_grid(int32_t N, int64_t count, int32_t dtype, int32_t* grid,
                                   int32_t* compute_units) {
  const char* fn = "ddp_persistent_grid";
  if (grid == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": grid is NULL");
  if (!valid_dtype(dtype)) return fail(DDP_EINVAL, std::string(fn) + ": unknown dtype");
  if (N < 1 || N > DDP_MAX_RANKS) return fail(DDP_EINVAL, std::string(fn) + ": N must lie in [1, 64]");
  if (count < 1) return fail(DDP_EINVAL, std::string(fn) + ": count < 1");
  RingArgs a;
  a.n = N;
  a.count = count;
  a.L = (count + N - 1) / N;
  a.vec = true;  // the step kernels stream vectors whenever the buffers are 16-byte aligned (assumed here)
  unsigned g = 0;
  int cus = 0;
  // the same choice of kernel as the launch: the default grid depends on the cache regime
  const bool nt = a.vec && int64_t(N) * count * elem_bytes(dtype) > kInfinityCacheBytes;
  int st;
  if (dtype == DDP_FP32)
    st = !a.vec ? persistent_grid<DDP_FP32, false, false>(a, 0, &g, &cus)
                : nt ? persistent_grid<DDP_FP32, true, true>(a, 0, &g, &cus)
                     : persistent_grid<DDP_FP32, true, false>(a, 0, &g, &cus);
  else
    st = !a.vec ? persistent_grid<DDP_BF16, false, false>(a, 0, &g, &cus)
                : nt ? persistent_grid<DDP_BF16, true, true>(a, 0, &g, &cus)
                     : persistent_grid<DDP_BF16, true, false>(a, 0, &g, &cus);
  if (st != DDP_OK) return st;
  *grid = int32_t(g);
  if (compute_units) *compute_units = cus;
  return DDP_OK;
}

extern "C" int ring_allreduce_persistent_ex(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                            int32_t n_steps, int32_t max_blocks, int64_t timeout_us,
                                            uint32_t extra_arrivals, void* stream) {
  PersistentOpts o;
  o.max_blocks = max_blocks;
  o.timeout_us = timeout_us;
  o.extra_arrivals = extra_arrivals;
  return persistent("ring_allreduce_persistent_ex", bufs, N, count, dtype, n_steps, o, stream);
}
