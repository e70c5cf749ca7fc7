// Device-side helpers and host-side launch checks shared by the HIP sources.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "barrier_slots.h"
#include "ddp_internal.h"

namespace ddp {

// A 16-byte vector of four 32-bit words (a clang vector type, so the
// non-temporal load/store builtins accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // threads per block of every streaming kernel (4 waves of 64)

// The N rank base pointers, passed by value in the kernel arguments (512 bytes).
struct RankPtrs {
  void* p[DDP_MAX_RANKS];
};

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// Returns DDP_EHIP with the runtime's message if `e` is an error.
inline int hip_fail(hipError_t e, const char* where) {
  return fail(DDP_EHIP, std::string(where) + ": " + hipGetErrorString(e));
}

#define DDP_HIP_TRY(expr, where)                       \
  do {                                                 \
    hipError_t _e = (expr);                            \
    if (_e != hipSuccess) return ::ddp::hip_fail(_e, where); \
  } while (0)

// Host-side checks (defined in runtime.hip).
// Every byte of [p, p + bytes) must lie inside one device allocation.
int check_range(const void* p, int64_t bytes, const char* fn, const char* what);
// N rank buffers of `bytes` each: non-NULL, aligned to `align`, inside their
// allocations and pairwise disjoint (with bytes == 0 nothing is touched and
// any pointer, NULL included, is accepted).
int check_rank_buffers(void* const* bufs, int32_t n, int64_t bytes, int align, const char* fn,
                       const char* what);
// True if every pointer is 16-byte aligned.
bool all_aligned16(void* const* bufs, int32_t n);

// Per-device persistent-barrier words (defined in runtime.hip). A lease holds
// one of the device's slots of kSlotWords 32-bit words: barrier_acquire makes
// `stream` wait for the slot's previous user's work (see barrier_slots.h),
// then zeroes the words on `stream`; `status` is the device's sticky timeout
// line. barrier_release records the end of the lease's work on `stream` and
// frees the slot; it must follow every successful barrier_acquire, after
// everything that reads the words (a kernel that checks the abort bit
// included) has been enqueued.
struct BarrierLease {
  unsigned int* words = nullptr;
  unsigned int* status = nullptr;
  int slot = -1;
  int dev = -1;
};
int barrier_acquire(hipStream_t stream, BarrierLease* lease);
int barrier_release(BarrierLease* lease, hipStream_t stream);

// Releases a held lease when it goes out of scope (on an early error return).
class BarrierGuard {
 public:
  explicit BarrierGuard(hipStream_t s) : s_(s) {}
  BarrierGuard(const BarrierGuard&) = delete;
  BarrierGuard& operator=(const BarrierGuard&) = delete;
  ~BarrierGuard() { (void)barrier_release(&lease_, s_); }
  int acquire() { return barrier_acquire(s_, &lease_); }
  int release() { return barrier_release(&lease_, s_); }
  unsigned int* words() const { return lease_.words; }
  unsigned int* status() const { return lease_.status; }

 private:
  hipStream_t s_;
  BarrierLease lease_;
};

// The top bit of a persistent launch's arrival word: set when a grid barrier
// gave up waiting (the launch's result is incomplete).
constexpr unsigned int kAbortBit = 0x80000000u;
// 32-bit words in one launch's barrier slot (three 128-byte lines in use; see
// ring_kernels.hip).
constexpr int kSlotWords = 128;

// The whole persistent all-reduce (2(N-1) steps) with barrier words that the
// caller leased and that are zero (ring_kernels.hip).
int persistent_allreduce_leased(void* const* bufs, int32_t N, int64_t count, int32_t dtype, unsigned int* words,
                                unsigned int* status, hipStream_t s);
// bucket_unpack_scale on checked arguments, skipped by every block if
// `abort_word` is not NULL and has kAbortBit set when the kernel runs: the
// copy back of a persistent all-reduce that gave up leaves the gradients as
// they were (pack_kernels.hip).
int unpack_scale_guarded(const ddp_plan* plan, int32_t b, const void* const* bucket_bufs, void* const* grad_arenas,
                         int32_t N, float scale, const unsigned int* abort_word, hipStream_t s);
// pack, persistent all-reduce, guarded unpack of bucket b under one lease
// (pack_kernels.hip; used by ddp_sync and the reducer).
int sync_bucket_persistent(const ddp_plan* plan, int32_t b, void* const* grad_arenas, void* const* bucket_bufs,
                           int32_t N, float scale, hipStream_t s);
// Zeroes n 32-bit words at p on `stream` with a fill kernel (runtime.hip).
int zero_words(unsigned int* p, int n, hipStream_t stream);
// The status words of the allocation-free persistent launches on device
// `dev`, or NULL if none has run there (ring_kernels.hip).
unsigned int* noalloc_status_words(int dev);

// The in-place sync of bucket b on arenas already checked by
// check_view_arenas, with at most max_blocks blocks (0: as many as tiles)
// (view_kernels.hip).
int launch_view_bucket(const ddp_plan* plan, int32_t b, const RankPtrs& P, int32_t N, float scale,
                       int64_t max_blocks, hipStream_t s);
int check_view_arenas(const ddp_plan* plan, void* const* grad_arenas, int32_t N, const char* fn);
// The in-place sync of every bucket at once: one launch over the whole arena.
int launch_view_arena(const ddp_plan* plan, const RankPtrs& P, int32_t N, float scale, hipStream_t s);

// The synthetic backward kernel on already-checked buffers (runtime.hip).
int launch_synthetic_backward(const RankPtrs& S, const RankPtrs& D, int32_t N, int64_t numel, int32_t dtype,
                              int32_t work, int32_t lds_kib, hipStream_t s);

// ---------------------------------------------------------------- device helpers

// fp32 to bf16, round to nearest with ties to even, by gfx950's conversion
// instruction (v_cvt_pk_bf16_f32, two values at once). Subnormals are kept,
// infinities and overflow give infinity, and a NaN stays a NaN with its quiet
// bit set and its upper payload bits kept. On MI355X it gave the same bits
// as the bit-level definition (add 0x7fff plus the lowest kept bit, then
// truncate; NaN: set the quiet bit, truncate) for all 2^32 fp32 inputs.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 and packed: `lo` in bits 0-15, `hi` in 16-31.
__device__ __forceinline__ uint32_t round_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t bf16_pack(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// One fp32 value rounded to bf16, returned as an fp32 value with its low 16
// bits clear.
__device__ __forceinline__ float round_bf16(float f) { return bf16_lo(round_bf16x2(f, 0.0f)); }

// Per-dtype arithmetic on 16-byte vectors and on single elements. An
// accumulator holds values of the buffer dtype (bf16 values are kept as fp32
// numbers with the low 16 bits clear); every add is rounded once to the dtype.
template <int DT>
struct Ops;

template <>
struct Ops<DDP_FP32> {
  static constexpr int V = 4;  // elements per 16-byte vector
  using scalar_t = float;
  struct Acc {
    float v[4];
  };
  static __device__ __forceinline__ Acc from(u32x4 w) {
    return Acc{{__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z),
                __uint_as_float(w.w)}};
  }
  static __device__ __forceinline__ void add(Acc& a, u32x4 w) {
    a.v[0] += __uint_as_float(w.x);
    a.v[1] += __uint_as_float(w.y);
    a.v[2] += __uint_as_float(w.z);
    a.v[3] += __uint_as_float(w.w);
  }
  static __device__ __forceinline__ u32x4 to(const Acc& a) {
    return u32x4{__float_as_uint(a.v[0]), __float_as_uint(a.v[1]), __float_as_uint(a.v[2]),
                 __float_as_uint(a.v[3])};
  }
  static __device__ __forceinline__ u32x4 scale(u32x4 w, float s) {
    return u32x4{__float_as_uint(__uint_as_float(w.x) * s), __float_as_uint(__uint_as_float(w.y) * s),
                 __float_as_uint(__uint_as_float(w.z) * s), __float_as_uint(__uint_as_float(w.w) * s)};
  }
  // single elements
  static __device__ __forceinline__ float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
  }
  static __device__ __forceinline__ float add1(float a, float b) { return a + b; }
  static __device__ __forceinline__ float mul1(float a, float s) { return a * s; }
};

template <>
struct Ops<DDP_BF16> {
  static constexpr int V = 8;
  using scalar_t = float;  // the bf16 value as an fp32 number
  struct Acc {
    float v[8];
  };
  static __device__ __forceinline__ Acc from(u32x4 w) {
    return Acc{{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), bf16_lo(w.z),
                bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)}};
  }
  static __device__ __forceinline__ void add2(float& lo, float& hi, uint32_t w) {
    const uint32_t r = round_bf16x2(lo + bf16_lo(w), hi + bf16_hi(w));
    lo = bf16_lo(r);
    hi = bf16_hi(r);
  }
  static __device__ __forceinline__ void add(Acc& a, u32x4 w) {
    add2(a.v[0], a.v[1], w.x);
    add2(a.v[2], a.v[3], w.y);
    add2(a.v[4], a.v[5], w.z);
    add2(a.v[6], a.v[7], w.w);
  }
  static __device__ __forceinline__ u32x4 to(const Acc& a) {
    return u32x4{bf16_pack(a.v[0], a.v[1]), bf16_pack(a.v[2], a.v[3]), bf16_pack(a.v[4], a.v[5]),
                 bf16_pack(a.v[6], a.v[7])};
  }
  static __device__ __forceinline__ uint32_t scale2(uint32_t w, float s) {
    return round_bf16x2(bf16_lo(w) * s, bf16_hi(w) * s);
  }
  static __device__ __forceinline__ u32x4 scale(u32x4 w, float s) {
    return u32x4{scale2(w.x, s), scale2(w.y, s), scale2(w.z, s), scale2(w.w, s)};
  }
  static __device__ __forceinline__ float load1(const void* p, int64_t i) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  static __device__ __forceinline__ void store1(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = uint16_t(__float_as_uint(v) >> 16);
  }
  static __device__ __forceinline__ float add1(float a, float b) { return round_bf16(a + b); }
  static __device__ __forceinline__ float mul1(float a, float s) { return round_bf16(a * s); }
};

// One 32-bit word of a staged tile (one fp32 element or two bf16 elements):
// the ring-order sum of the ranks' words, one rounding per add, then scaled.
template <int DT>
struct Word;

template <>
struct Word<DDP_FP32> {
  struct Acc {
    float v;
  };
  static __device__ __forceinline__ Acc from(uint32_t w) { return Acc{__uint_as_float(w)}; }
  static __device__ __forceinline__ void add(Acc& a, uint32_t w) { a.v += __uint_as_float(w); }
  static __device__ __forceinline__ uint32_t out(const Acc& a) { return __float_as_uint(a.v); }
  static __device__ __forceinline__ uint32_t out(const Acc& a, float s) { return __float_as_uint(a.v * s); }
  // Element j of a 16-byte vector, as an fp32 value.
  static __device__ __forceinline__ float elem(u32x4 y, int j) { return __uint_as_float(y[j]); }
  // Elements [e0, e0 + cnt) of p (cnt < 4) as a vector, the rest zero.
  static __device__ __forceinline__ u32x4 load_partial(const void* p, int64_t e0, int cnt) {
    u32x4 y = {0u, 0u, 0u, 0u};
    const uint32_t* q = static_cast<const uint32_t*>(p) + e0;
    for (int j = 0; j < cnt; ++j) y[j] = q[j];
    return y;
  }
};

template <>
struct Word<DDP_BF16> {
  struct Acc {
    float lo, hi;
  };
  static __device__ __forceinline__ Acc from(uint32_t w) { return Acc{bf16_lo(w), bf16_hi(w)}; }
  static __device__ __forceinline__ void add(Acc& a, uint32_t w) {
    const uint32_t r = round_bf16x2(a.lo + bf16_lo(w), a.hi + bf16_hi(w));
    a.lo = bf16_lo(r);
    a.hi = bf16_hi(r);
  }
  static __device__ __forceinline__ uint32_t out(const Acc& a) { return bf16_pack(a.lo, a.hi); }
  static __device__ __forceinline__ uint32_t out(const Acc& a, float s) {
    return round_bf16x2(a.lo * s, a.hi * s);
  }
  static __device__ __forceinline__ float elem(u32x4 y, int j) {
    return (j & 1) ? bf16_hi(y[j >> 1]) : bf16_lo(y[j >> 1]);
  }
  static __device__ __forceinline__ u32x4 load_partial(const void* p, int64_t e0, int cnt) {
    u32x4 y = {0u, 0u, 0u, 0u};
    const uint16_t* q = static_cast<const uint16_t*>(p) + e0;
    for (int j = 0; j < cnt; ++j) y[j >> 1] |= uint32_t(q[j]) << ((j & 1) * 16);
    return y;
  }
};

template <bool NT>
__device__ __forceinline__ u32x4 ld16(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

template <bool NT>
__device__ __forceinline__ void st16(u32x4* p, u32x4 v) {
  if constexpr (NT) {
    __builtin_nontemporal_store(v, p);
  } else {
    *p = v;
  }
}

}  // namespace ddp
