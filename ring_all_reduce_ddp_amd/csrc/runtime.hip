// Host-side argument checks, per-device barrier words, and the two helper
// kernels (all-ranks-equal count, copy probe).
#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "hip_common.h"

namespace ddp {

namespace {

// "what" or "what[index]" (index >= 0): built only for a failure message, so a
// successful check allocates no host memory.
std::string name_of(const char* what, int32_t index) {
  return index < 0 ? std::string(what) : std::string(what) + "[" + std::to_string(index) + "]";
}

int check_range_at(const void* p, int64_t bytes, const char* fn, const char* what, int32_t index) {
  if (bytes == 0) return DDP_OK;
  if (p == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, index) + " is NULL");
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  hipError_t e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, index) +
                                " is not inside a device allocation of this process");
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
  const uintptr_t q = reinterpret_cast<uintptr_t>(p);
  if (q < lo || uint64_t(bytes) > size || q - lo > size - uint64_t(bytes))
    return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, index) + " range of " + std::to_string(bytes) +
                                " bytes runs past the end of its allocation");
  return DDP_OK;
}

}  // namespace

int check_range(const void* p, int64_t bytes, const char* fn, const char* what) {
  return check_range_at(p, bytes, fn, what, -1);
}

int check_rank_buffers(void* const* bufs, int32_t n, int64_t bytes, int align, const char* fn,
                       const char* what) {
  if (bufs == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": " + what + " array is NULL");
  if (n < 1 || n > DDP_MAX_RANKS) return fail(DDP_EINVAL, std::string(fn) + ": N must lie in [1, 64]");
  // Zero-length buffers are never touched: any pointer will do, NULL included
  // (torch reports a null data pointer for an empty tensor).
  if (bytes == 0) return DDP_OK;
  for (int32_t r = 0; r < n; ++r) {
    if (bufs[r] == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, r) + " is NULL");
    if (reinterpret_cast<uintptr_t>(bufs[r]) % uintptr_t(align) != 0)
      return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, r) + " is not " + std::to_string(align) +
                                  "-byte aligned");
  }
  std::pair<uintptr_t, int32_t> spans[DDP_MAX_RANKS];
  for (int32_t r = 0; r < n; ++r) {
    int st = check_range_at(bufs[r], bytes, fn, what, r);
    if (st != DDP_OK) return st;
    spans[r] = {reinterpret_cast<uintptr_t>(bufs[r]), r};
  }
  std::sort(spans, spans + n);
  for (int32_t i = 1; i < n; ++i) {
    if (spans[i].first - spans[i - 1].first < uint64_t(bytes))
      return fail(DDP_EINVAL, std::string(fn) + ": " + name_of(what, spans[i - 1].second) + " and " +
                                  name_of(what, spans[i].second) + " overlap");
  }
  return DDP_OK;
}

bool all_aligned16(void* const* bufs, int32_t n) {
  for (int32_t r = 0; r < n; ++r)
    if (reinterpret_cast<uintptr_t>(bufs[r]) % 16 != 0) return false;
  return true;
}

// ---------------------------------------------------------------- barrier words

namespace {

constexpr int kSlots = 64;          // slots handed out round-robin per device
constexpr int kSlotStride = kSlotWords;  // words between slots (512 bytes; the layout is in ring_kernels.hip)
constexpr int kScratchWords = kSlots * kSlotStride + kSlotStride;  // + status line

// HIP events for SlotRing: a slot's next user waits, on its own stream, for
// the event its previous user recorded after its work on the slot.
struct HipSlotOps {
  using Event = hipEvent_t;
  using Stream = hipStream_t;
  static int create(Event* e) {
    const hipError_t err = hipEventCreateWithFlags(e, hipEventDisableTiming);
    return err == hipSuccess ? DDP_OK : hip_fail(err, "barrier words: hipEventCreateWithFlags");
  }
  static int wait(Stream s, Event e) {
    const hipError_t err = hipStreamWaitEvent(s, e, 0);
    return err == hipSuccess ? DDP_OK : hip_fail(err, "barrier words: hipStreamWaitEvent");
  }
  static int record(Event e, Stream s) {
    const hipError_t err = hipEventRecord(e, s);
    return err == hipSuccess ? DDP_OK : hip_fail(err, "barrier words: hipEventRecord");
  }
};

struct DeviceScratch {
  unsigned int* words = nullptr;    // kScratchWords words; the last line holds the status
  SlotRing<kSlots, HipSlotOps> ring;
};

std::mutex g_scratch_mu;
DeviceScratch g_scratch[kMaxDevices];

__global__ void k_zero_words(unsigned int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

int device_scratch(int* dev_out, DeviceScratch** out) {
  int dev = 0;
  DDP_HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DDP_EINVAL, "device index beyond 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  DeviceScratch& s = g_scratch[dev];
  if (s.words == nullptr) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, sizeof(unsigned int) * kScratchWords);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(DDP_ENOMEM, std::string("barrier words: hipMalloc: ") + hipGetErrorString(e));
    }
    e = hipMemset(p, 0, sizeof(unsigned int) * kScratchWords);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "barrier words: hipMemset");
    }
    s.words = static_cast<unsigned int*>(p);
  }
  *dev_out = dev;
  *out = &s;
  return DDP_OK;
}

}  // namespace

int zero_words(unsigned int* p, int n, hipStream_t stream) {
  // A fill kernel rather than a memset node keeps this usable under graph capture.
  hipLaunchKernelGGL(k_zero_words, dim3(1), dim3(64), 0, stream, p, n);
  DDP_HIP_TRY(hipGetLastError(), "barrier words: zero launch");
  return DDP_OK;
}

int barrier_acquire(hipStream_t stream, BarrierLease* lease) {
  DeviceScratch* s = nullptr;
  int dev = 0;
  int st = device_scratch(&dev, &s);
  if (st != DDP_OK) return st;
  SlotRing<kSlots, HipSlotOps>::Lease l;
  st = s->ring.acquire(stream, &l);
  if (st != DDP_OK) return st;
  lease->dev = dev;
  lease->slot = l.slot;
  lease->words = s->words + size_t(l.slot) * kSlotStride;
  lease->status = s->words + size_t(kSlots) * kSlotStride;
  st = zero_words(lease->words, kSlotStride, stream);
  if (st != DDP_OK) (void)barrier_release(lease, stream);
  return st;
}

int barrier_release(BarrierLease* lease, hipStream_t stream) {
  if (lease->slot < 0) return DDP_OK;
  SlotRing<kSlots, HipSlotOps>::Lease l;
  l.slot = lease->slot;
  l.ring = &g_scratch[lease->dev].ring;
  lease->slot = -1;
  return l.ring->release(&l, stream);
}

// ---------------------------------------------------------------- all-ranks-equal count

namespace {

template <int EB>
__global__ __launch_bounds__(kThreads) void k_count_mismatch(RankPtrs P, int n, int64_t count,
                                                             unsigned long long* out) {
  // EB: element bytes (2 or 4). Compares every rank's bits with rank 0's.
  unsigned long long local = 0;
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < count; i += stride) {
    uint32_t ref, x;
    if constexpr (EB == 4) {
      ref = static_cast<const uint32_t*>(P.p[0])[i];
    } else {
      ref = static_cast<const uint16_t*>(P.p[0])[i];
    }
    bool diff = false;
    for (int r = 1; r < n; ++r) {
      if constexpr (EB == 4) {
        x = static_cast<const uint32_t*>(P.p[r])[i];
      } else {
        x = static_cast<const uint16_t*>(P.p[r])[i];
      }
      diff |= (x != ref);
    }
    local += diff ? 1ull : 0ull;
  }
  __shared__ unsigned long long partial[kThreads];
  partial[threadIdx.x] = local;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (int(threadIdx.x) < w) partial[threadIdx.x] += partial[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && partial[0] != 0) atomicAdd(out, partial[0]);
}

__global__ void k_zero_u64(unsigned long long* p) {
  if (threadIdx.x == 0) *p = 0ull;
}

// ---------------------------------------------------------------- copy probe

// Plain streaming copy in the launch shape that measured fastest for
// streaming on MI355X: one wave per block, one 16-byte vector per thread, one
// tile per block, non-temporal loads and stores.
constexpr int kCopyThreads = 64;

__global__ __launch_bounds__(kCopyThreads) void k_copy16(u32x4* __restrict__ dst,
                                                         const u32x4* __restrict__ src, int64_t nvec) {
  const int64_t stride = int64_t(gridDim.x) * kCopyThreads;
  for (int64_t i = int64_t(blockIdx.x) * kCopyThreads + threadIdx.x; i < nvec; i += stride)
    st16<true>(dst + i, ld16<true>(src + i));
}

// ---------------------------------------------------------------- synthetic backward

// Stands in for the backward computation that produces a gradient: dst = src,
// after `work` dependent fused multiply-adds per element on a separate
// accumulator. The accumulator converges to 1 and never becomes NaN for
// finite inputs, so the branch that would store it is never taken; the
// compiler cannot know that, so the arithmetic is kept. The launch may
// reserve dynamic LDS it never touches, to hold the kernel to a chosen
// occupancy (as register- or LDS-hungry backward kernels are held).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_synthetic_backward(RankPtrs src, RankPtrs dst, int64_t numel,
                                                                 int work) {
  using O = Ops<DT>;
  const void* s = src.p[blockIdx.y];
  void* d = dst.p[blockIdx.y];
  const int64_t stride = int64_t(gridDim.x) * kThreads;
  int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  float x = i < numel ? O::load1(s, i) : 0.0f;
  for (; i < numel; i += stride) {
    // The next element's load is issued before this element's arithmetic,
    // as compute-bound kernels hide their operand fetches.
    // (The last iteration reloads its own element: an unconditional load
    // lets the wait for it sit after the arithmetic.)
    const float next = O::load1(s, min(i + stride, numel - 1));
    float acc = x;
    for (int k = 0; k < work; ++k) acc = __builtin_fmaf(acc, 0.999f, 0.001f);
    O::store1(d, i, acc != acc ? acc : x);
    x = next;
  }
}

}  // namespace

}  // namespace ddp

using namespace ddp;

namespace ddp {
// Launches the synthetic backward on already-checked buffers.
int launch_synthetic_backward(const RankPtrs& S, const RankPtrs& D, int32_t N, int64_t numel, int32_t dtype,
                              int32_t work, int32_t lds_kib, hipStream_t s) {
  if (numel == 0) return DDP_OK;
  const int64_t blocks = std::min<int64_t>((numel + kThreads - 1) / kThreads, 4096);
  const dim3 g(static_cast<unsigned>(blocks), static_cast<unsigned>(N));
  const size_t lds = size_t(lds_kib) * 1024;
  if (dtype == DDP_FP32)
    hipLaunchKernelGGL(k_synthetic_backward<DDP_FP32>, g, dim3(kThreads), lds, s, S, D, numel, work);
  else
    hipLaunchKernelGGL(k_synthetic_backward<DDP_BF16>, g, dim3(kThreads), lds, s, S, D, numel, work);
  DDP_HIP_TRY(hipGetLastError(), "ddp_synthetic_backward: launch");
  return DDP_OK;
}
}  // namespace ddp

extern "C" int ddp_synthetic_backward(const void* const* srcs, void* const* dsts, int32_t N, int64_t numel,
                                      int32_t dtype, int32_t work, int32_t lds_kib, void* stream) {
  const char* fn = "ddp_synthetic_backward";
  if (!valid_dtype(dtype)) return fail(DDP_EINVAL, std::string(fn) + ": unknown dtype");
  if (N < 1 || N > DDP_MAX_RANKS) return fail(DDP_EINVAL, std::string(fn) + ": N must lie in [1, 64]");
  if (numel < 0 || work < 0) return fail(DDP_EINVAL, std::string(fn) + ": numel and work must be >= 0");
  if (lds_kib < 0 || lds_kib > 64) return fail(DDP_EINVAL, std::string(fn) + ": lds_kib must lie in [0, 64]");
  const int eb = elem_bytes(dtype);
  int st = check_rank_buffers(const_cast<void* const*>(srcs), N, numel * eb, eb, fn, "srcs");
  if (st != DDP_OK) return st;
  st = check_rank_buffers(dsts, N, numel * eb, eb, fn, "dsts");
  if (st != DDP_OK) return st;
  RankPtrs S{}, D{};
  for (int r = 0; r < N; ++r) {
    S.p[r] = const_cast<void*>(srcs[r]);
    D.p[r] = dsts[r];
  }
  return launch_synthetic_backward(S, D, N, numel, dtype, work, lds_kib, as_stream(stream));
}

extern "C" int ddp_persistent_status(void* stream) {
  int dev = 0;
  DDP_HIP_TRY(hipGetDevice(&dev), "ddp_persistent_status: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DDP_EINVAL, "ddp_persistent_status: device index beyond 64");
  DDP_HIP_TRY(hipStreamSynchronize(as_stream(stream)), "ddp_persistent_status: hipStreamSynchronize");
  // The status words of the launches with library-allocated barrier words
  // (if any was made on this device) and of the allocation-free ones.
  unsigned int* lines[2] = {nullptr, noalloc_status_words(dev)};
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev].words != nullptr) lines[0] = g_scratch[dev].words + size_t(kSlots) * kSlotStride;
  }
  for (unsigned int* status : lines) {
    if (status == nullptr) continue;
    unsigned int host[3] = {0, 0, 0};
    DDP_HIP_TRY(hipMemcpy(host, status, sizeof(host), hipMemcpyDeviceToHost),
                "ddp_persistent_status: hipMemcpy");
    if (host[0] != 0) {
      const unsigned int zero[3] = {0, 0, 0};
      DDP_HIP_TRY(hipMemcpy(status, zero, sizeof(zero), hipMemcpyHostToDevice),
                  "ddp_persistent_status: hipMemcpy");
      return fail(DDP_ETIMEOUT, "ring_allreduce_persistent: a grid barrier timed out with " +
                                    std::to_string(host[1]) + " of " + std::to_string(host[2]) +
                                    " block arrivals; results are incomplete");
    }
  }
  return DDP_OK;
}

extern "C" int ddp_count_mismatches(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                    uint64_t* out_dev, void* stream) {
  const char* fn = "ddp_count_mismatches";
  if (!valid_dtype(dtype)) return fail(DDP_EINVAL, std::string(fn) + ": unknown dtype");
  if (N < 1 || N > DDP_MAX_RANKS) return fail(DDP_EINVAL, std::string(fn) + ": N must lie in [1, 64]");
  if (count < 0) return fail(DDP_EINVAL, std::string(fn) + ": count < 0");
  const int eb = elem_bytes(dtype);
  int st = check_rank_buffers(bufs, N, count * eb, eb, fn, "bufs");
  if (st != DDP_OK) return st;
  st = check_range(out_dev, sizeof(uint64_t), fn, "out_dev");
  if (st != DDP_OK) return st;
  if (reinterpret_cast<uintptr_t>(out_dev) % 8 != 0)
    return fail(DDP_EINVAL, std::string(fn) + ": out_dev is not 8-byte aligned");
  hipStream_t s = as_stream(stream);
  auto* out = reinterpret_cast<unsigned long long*>(out_dev);
  hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, out);
  DDP_HIP_TRY(hipGetLastError(), "ddp_count_mismatches: zero launch");
  if (count == 0 || N == 1) return DDP_OK;
  RankPtrs P{};
  for (int r = 0; r < N; ++r) P.p[r] = bufs[r];
  const int64_t blocks = std::min<int64_t>((count + kThreads - 1) / kThreads, 8192);
  if (eb == 4)
    hipLaunchKernelGGL(k_count_mismatch<4>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, P, N, count, out);
  else
    hipLaunchKernelGGL(k_count_mismatch<2>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, P, N, count, out);
  DDP_HIP_TRY(hipGetLastError(), "ddp_count_mismatches: launch");
  return DDP_OK;
}

extern "C" int ddp_device_alloc(int64_t nbytes, int32_t flags, void** out) {
  const char* fn = "ddp_device_alloc";
  if (out == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": out is NULL");
  *out = nullptr;
  if (nbytes <= 0) return fail(DDP_EINVAL, std::string(fn) + ": nbytes must be positive");
  if (flags != 0 && flags != DDP_ALLOC_CONTIGUOUS)
    return fail(DDP_EINVAL, std::string(fn) + ": flags must be 0 or DDP_ALLOC_CONTIGUOUS");
  void* p = nullptr;
  const hipError_t e = flags == DDP_ALLOC_CONTIGUOUS
                           ? hipExtMallocWithFlags(&p, size_t(nbytes), hipDeviceMallocContiguous)
                           : hipMalloc(&p, size_t(nbytes));
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(DDP_ENOMEM, std::string(fn) + ": " + std::to_string(nbytes) + " bytes" +
                                (flags == DDP_ALLOC_CONTIGUOUS ? " of contiguous memory" : "") + ": " +
                                hipGetErrorString(e));
  }
  *out = p;
  return DDP_OK;
}

extern "C" int ddp_device_free(void* p) {
  if (p == nullptr) return DDP_OK;
  DDP_HIP_TRY(hipFree(p), "ddp_device_free: hipFree");
  return DDP_OK;
}

extern "C" int ddp_copy_probe(void* dst, const void* src, int64_t nbytes, void* stream) {
  const char* fn = "ddp_copy_probe";
  if (nbytes < 0 || nbytes % 16 != 0)
    return fail(DDP_EINVAL, std::string(fn) + ": nbytes must be a non-negative multiple of 16");
  if (nbytes == 0) return DDP_OK;
  if (reinterpret_cast<uintptr_t>(dst) % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return fail(DDP_EINVAL, std::string(fn) + ": pointers must be 16-byte aligned");
  int st = check_range(dst, nbytes, fn, "dst");
  if (st != DDP_OK) return st;
  st = check_range(src, nbytes, fn, "src");
  if (st != DDP_OK) return st;
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), q = reinterpret_cast<uintptr_t>(src);
  if ((d < q ? q - d : d - q) < uint64_t(nbytes))
    return fail(DDP_EINVAL, std::string(fn) + ": src and dst overlap");
  const int64_t nvec = nbytes / 16;
  const int64_t blocks = std::min<int64_t>((nvec + kCopyThreads - 1) / kCopyThreads, int64_t(1) << 24);
  hipLaunchKernelGGL(k_copy16, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, as_stream(stream),
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), nvec);
  DDP_HIP_TRY(hipGetLastError(), "ddp_copy_probe: launch");
  return DDP_OK;
}
