// Gradient <-> bucket copies of a DDP sync, and the whole sync.
//
// Page "DDP 与 Ring All-Reduce" (blog.vllbc.top), sections 03 and 05: with
// DDP's default gradient_as_bucket_view=False the gradients are copied into
// each bucket's flat buffer before its all-reduce, and the reduced bucket is
// copied back into every parameter's .grad; the reducer divides the summed
// gradient by the world size. Page "Day 17 数据并行 DP/DDP" (blog.ans20xx.com),
// part "源码阅读路线": after a bucket's all-reduce completes it is divided by
// the world size and copied back. Here the division is a multiplication by
// the caller's fp32 `scale` (1/N), fused into the copy back.
//
// A plan may keep fp32 gradients in bf16 buckets: the bf16 compression hook
// (page "Day 17 数据并行 DP/DDP", reading list, "PyTorch DDP Communication
// Hooks"). Packing then rounds each gradient to bf16, the ring runs in bf16,
// and the copy back widens to fp32 and rounds the scaled value once.
//
// A bucket is a list of segments (each member's slot, then the zero padding);
// each segment is covered by whole tiles so a block never mixes segments, and
// a block finds its segment with one load from the plan's tile-to-segment
// table. Members and arena offsets start on 16-byte boundaries, so everything
// but the last partial vector of a member moves as 16-byte vectors.
#include <algorithm>

#include "hip_common.h"

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

namespace ddp {
namespace {

// NTL: non-temporal loads of the gradients, for arenas that together exceed
// the Infinity Cache: they are not read again before the copy back
// overwrites them, and streaming them leaves the cache to the bucket the
// all-reduce reads next (ResNet-50 over 8 ranks: whole copying sync 0.778
// against 0.790 ms).
template <int DT, bool NTL>
__global__ __launch_bounds__(kThreads) void k_pack(const Segment* segs, const int32_t* tile_seg, int64_t n_tiles,
                                                   RankPtrs arenas, RankPtrs buckets) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  constexpr int U = kPackVecsPerThread;
  constexpr int64_t kTile = int64_t(kThreads) * U * V;
  const void* arena = arenas.p[blockIdx.y];
  void* bucket = buckets.p[blockIdx.y];
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const Segment sg = segs[tile_seg[tile]];
    const int64_t first = (tile - sg.tile_begin) * kTile;
    // All of the tile's loads are issued before its first store (the
    // compiler cannot tell the arena from the bucket, so it would not move a
    // load above an earlier store on its own).
    u32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;  // element in the slot
      x[u] = e + V <= sg.numel ? ld16<NTL>(static_cast<const u32x4*>(arena) + (sg.src_off + e) / V)
                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;
      if (e >= sg.slot) continue;
      if (e + V <= sg.numel || e >= sg.numel) {
        static_cast<u32x4*>(bucket)[(sg.dst_off + e) / V] = x[u];  // a vector of the member, or padding zeros
      } else {
        for (int i = 0; i < V; ++i)
          O::store1(bucket, sg.dst_off + e + i, e + i < sg.numel ? O::load1(arena, sg.src_off + e + i) : 0.0f);
      }
    }
  }
}

// NTS: non-temporal stores, for gradients that together exceed the Infinity
// Cache (nothing in the sync reads them again; ResNet-50 over 8 ranks: whole
// copying sync 0.79 against 0.83 ms with cached stores). Pack keeps cached
// stores: the all-reduce that follows reads the bucket from the cache
// (streaming them made the same sync 0.90 ms).
// True if the persistent all-reduce whose arrival word this is gave up (a
// NULL word: no such all-reduce precedes this copy back).
__device__ __forceinline__ bool aborted(const unsigned int* abort_word) {
  return abort_word != nullptr &&
         (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kAbortBit) != 0u;
}

template <int DT, bool NTS>
__global__ __launch_bounds__(kThreads) void k_unpack_scale(const Segment* segs, const int32_t* tile_seg, int64_t n_tiles,
                                                           RankPtrs buckets, RankPtrs arenas, float scale,
                                                           const unsigned int* abort_word) {
  using O = Ops<DT>;
  if (aborted(abort_word)) return;  // leave the gradients as they were
  constexpr int V = O::V;
  constexpr int U = kPackVecsPerThread;
  constexpr int64_t kTile = int64_t(kThreads) * U * V;
  const void* bucket = buckets.p[blockIdx.y];
  void* arena = arenas.p[blockIdx.y];
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const Segment sg = segs[tile_seg[tile]];
    const int64_t first = (tile - sg.tile_begin) * kTile;
    u32x4 x[U];  // every load before the first store, as in k_pack
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;
      if (e + V <= sg.numel) x[u] = static_cast<const u32x4*>(bucket)[(sg.dst_off + e) / V];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;
      if (e >= sg.numel) continue;  // padding and slack stay in the bucket
      if (e + V <= sg.numel) {
        st16<NTS>(static_cast<u32x4*>(arena) + (sg.src_off + e) / V, O::scale(x[u], scale));
      } else {
        for (int64_t i = e; i < sg.numel; ++i)
          O::store1(arena, sg.src_off + i, O::mul1(O::load1(bucket, sg.dst_off + i), scale));
      }
    }
  }
}

// fp32 gradients into a bf16 bucket (the bf16 compression hook): every
// gradient is rounded to the nearest bf16, ties to even. A bucket vector is 8
// bf16 elements; it reads two 16-byte vectors of fp32 gradients. NTL as in
// k_pack: streaming the gradients keeps the bucket in the Infinity Cache for
// the all-reduce (compressed ResNet-50 sync over 8 ranks: 0.589 against
// 0.658 ms with cached loads, although the packs alone took 0.243 against
// 0.237 ms).
template <bool NTL>
__global__ __launch_bounds__(kThreads) void k_pack_f32_to_bf16(const Segment* segs, const int32_t* tile_seg, int64_t n_tiles,
                                                               RankPtrs arenas, RankPtrs buckets) {
  constexpr int V = 8;
  constexpr int U = kPackVecsPerThread;
  constexpr int64_t kTile = int64_t(kThreads) * U * V;
  const float* arena = static_cast<const float*>(arenas.p[blockIdx.y]);
  void* bucket = buckets.p[blockIdx.y];
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const Segment sg = segs[tile_seg[tile]];
    const int64_t first = (tile - sg.tile_begin) * kTile;
    u32x4 a[U], b[U];  // every load before the first store, as in k_pack
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;
      if (e + V <= sg.numel) {
        const u32x4* src = reinterpret_cast<const u32x4*>(arena + sg.src_off + e);
        a[u] = ld16<NTL>(src);
        b[u] = ld16<NTL>(src + 1);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = first + (int64_t(u) * kThreads + threadIdx.x) * V;
      if (e >= sg.slot) continue;
      u32x4* d = static_cast<u32x4*>(bucket) + (sg.dst_off + e) / V;
      if (e + V <= sg.numel) {
        *d = u32x4{round_bf16x2(__uint_as_float(a[u].x), __uint_as_float(a[u].y)),
                   round_bf16x2(__uint_as_float(a[u].z), __uint_as_float(a[u].w)),
                   round_bf16x2(__uint_as_float(b[u].x), __uint_as_float(b[u].y)),
                   round_bf16x2(__uint_as_float(b[u].z), __uint_as_float(b[u].w))};
      } else if (e >= sg.numel) {
        *d = u32x4{0u, 0u, 0u, 0u};
      } else {
        for (int i = 0; i < V; ++i)
          Ops<DDP_BF16>::store1(bucket, sg.dst_off + e + i,
                                e + i < sg.numel ? round_bf16(arena[sg.src_off + e + i]) : 0.0f);
      }
    }
  }
}

// bf16 bucket back into fp32 gradients: each bf16 value (exact in fp32) is
// multiplied by `scale` and rounded once to fp32. A lane takes 4 elements
// (8 bytes of bucket, one 16-byte fp32 vector), so every store instruction
// covers whole cache lines and the stores can stream (NTS, arenas beyond the
// Infinity Cache). Lanes that each wrote 32 bytes as two 16-byte stores
// covered half a line per instruction and had to stay cached for the L2 to
// merge the halves: the six unpacks of the compressed ResNet-50 sync over 8
// ranks took 0.302 against 0.238 ms now, the whole sync 0.588 against 0.568.
template <bool NTS>
__global__ __launch_bounds__(kThreads) void k_unpack_bf16_to_f32(const Segment* segs, const int32_t* tile_seg, int64_t n_tiles,
                                                                 RankPtrs buckets, RankPtrs arenas, float scale,
                                                                 const unsigned int* abort_word) {
  if (aborted(abort_word)) return;  // leave the gradients as they were
  constexpr int U = kPackVecsPerThread;
  constexpr int64_t kTile = int64_t(kThreads) * U * 8;  // elements: U bf16 vectors of 8 per thread
  constexpr int kRow = kThreads * 4;                     // elements: one fp32 vector per thread
  const uint16_t* bucket = static_cast<const uint16_t*>(buckets.p[blockIdx.y]);
  float* arena = static_cast<float*>(arenas.p[blockIdx.y]);
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const Segment sg = segs[tile_seg[tile]];
    const int64_t first = (tile - sg.tile_begin) * kTile;
    u32x2 xs[2 * U];  // every load before the first store, as in k_pack
#pragma unroll
    for (int k = 0; k < 2 * U; ++k) {
      const int64_t e = first + int64_t(k) * kRow + threadIdx.x * 4;
      if (e + 4 <= sg.numel) xs[k] = *reinterpret_cast<const u32x2*>(bucket + sg.dst_off + e);
    }
#pragma unroll
    for (int k = 0; k < 2 * U; ++k) {
      const int64_t e = first + int64_t(k) * kRow + threadIdx.x * 4;
      if (e >= sg.numel) continue;
      if (e + 4 <= sg.numel) {
        const u32x2 x = xs[k];
        st16<NTS>(reinterpret_cast<u32x4*>(arena + sg.src_off + e),
                  u32x4{__float_as_uint(bf16_lo(x.x) * scale), __float_as_uint(bf16_hi(x.x) * scale),
                        __float_as_uint(bf16_lo(x.y) * scale), __float_as_uint(bf16_hi(x.y) * scale)});
      } else {
        for (int64_t i = e; i < sg.numel; ++i)
          arena[sg.src_off + i] = Ops<DDP_BF16>::load1(bucket, sg.dst_off + i) * scale;
      }
    }
  }
}

bool spans_overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return abytes > 0 && bbytes > 0 && x < y + uint64_t(bbytes) && y < x + uint64_t(abytes);
}

// Checks shared by pack and unpack.
int check_copy(const char* fn, const ddp_plan* plan, int32_t b, const void* const* arenas,
               const void* const* buckets, int32_t N) {
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (b < 0 || b >= int32_t(plan->buckets.size()))
    return fail(DDP_EINVAL, std::string(fn) + ": bucket index out of range");
  if (N != plan->world_size)
    return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  const int64_t abytes = plan->arena_numel * elem_bytes(plan->dtype);
  const int64_t bbytes = plan->buckets[b].padded_numel * elem_bytes(plan->comm_dtype);
  int st = check_rank_buffers(const_cast<void* const*>(arenas), N, abytes, 16, fn, "grad_arenas");
  if (st != DDP_OK) return st;
  st = check_rank_buffers(const_cast<void* const*>(buckets), N, bbytes, 16, fn, "bucket_bufs");
  if (st != DDP_OK) return st;
  for (int i = 0; i < N; ++i)
    for (int j = 0; j < N; ++j)
      if (spans_overlap(arenas[i], abytes, buckets[j], bbytes))
        return fail(DDP_EINVAL, std::string(fn) + ": grad_arenas[" + std::to_string(i) +
                                    "] overlaps bucket_bufs[" + std::to_string(j) + "]");
  return DDP_OK;
}

unsigned copy_grid(int64_t tiles) { return unsigned(std::max<int64_t>(1, std::min<int64_t>(tiles, 1 << 16))); }

}  // namespace

int device_tables(ddp_plan* plan, const Segment** segs, const uint16_t** vec_info, const int32_t** tile_seg) {
  int dev = 0;
  DDP_HIP_TRY(hipGetDevice(&dev), "plan tables: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(DDP_EINVAL, "plan tables: device index beyond 64");
  std::lock_guard<std::mutex> lock(plan->mu);
  DeviceTable& t = plan->device[dev];
  const size_t seg_bytes = size_t(round_up(int64_t(sizeof(Segment) * plan->segments.size()), 256));
  const size_t ts_bytes = size_t(round_up(int64_t(sizeof(int32_t) * plan->tile_seg.size()), 256));
  const size_t map_bytes = sizeof(uint16_t) * plan->vec_info.size();
  if (t.segs == nullptr && seg_bytes + ts_bytes + map_bytes > 0) {
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, seg_bytes + ts_bytes + map_bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(DDP_ENOMEM, std::string("plan tables: hipMalloc: ") + hipGetErrorString(e));
    }
    char* base = static_cast<char*>(p);
    e = hipMemcpy(base, plan->segments.data(), sizeof(Segment) * plan->segments.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && !plan->tile_seg.empty())
      e = hipMemcpy(base + seg_bytes, plan->tile_seg.data(), sizeof(int32_t) * plan->tile_seg.size(),
                    hipMemcpyHostToDevice);
    if (e == hipSuccess && map_bytes > 0)
      e = hipMemcpy(base + seg_bytes + ts_bytes, plan->vec_info.data(), map_bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p);
      return hip_fail(e, "plan tables: hipMemcpy");
    }
    t.segs = reinterpret_cast<Segment*>(base);
    t.tile_seg = reinterpret_cast<int32_t*>(base + seg_bytes);
    t.vec_info = reinterpret_cast<uint16_t*>(base + seg_bytes + ts_bytes);
  }
  if (segs) *segs = t.segs;
  if (vec_info) *vec_info = t.vec_info;
  if (tile_seg) *tile_seg = t.tile_seg;
  return DDP_OK;
}

void release_device_tables(ddp_plan* plan) {
  std::lock_guard<std::mutex> lock(plan->mu);
  for (DeviceTable& t : plan->device) {
    if (t.segs != nullptr) {
      (void)hipFree(t.segs);
      t.segs = nullptr;
      t.tile_seg = nullptr;
      t.vec_info = nullptr;
    }
  }
}

}  // namespace ddp

using namespace ddp;

extern "C" int bucket_pack(const ddp_plan* plan, int32_t b, const void* const* grad_arenas,
                           void* const* bucket_bufs, int32_t N, void* stream) {
  const char* fn = "bucket_pack";
  int st = check_copy(fn, plan, b, grad_arenas, bucket_bufs, N);
  if (st != DDP_OK) return st;
  const Bucket& bk = plan->buckets[b];
  if (bk.n_tiles == 0) return DDP_OK;
  const Segment* segs = nullptr;
  const int32_t* tile_seg = nullptr;
  st = device_tables(const_cast<ddp_plan*>(plan), &segs, nullptr, &tile_seg);
  if (st != DDP_OK) return st;
  RankPtrs A{}, B{};
  for (int r = 0; r < N; ++r) {
    A.p[r] = const_cast<void*>(grad_arenas[r]);
    B.p[r] = bucket_bufs[r];
  }
  const dim3 g(copy_grid(bk.n_tiles), unsigned(N)), blk(kThreads);
  hipStream_t s = as_stream(stream);
  const Segment* sg = segs + bk.seg_begin;
  const int32_t* ts = tile_seg + bk.tile_seg_begin;
  const bool ntl = int64_t(N) * plan->arena_numel * elem_bytes(plan->dtype) > kInfinityCacheBytes;
  if (plan->dtype != plan->comm_dtype) {
    if (ntl)
      hipLaunchKernelGGL(k_pack_f32_to_bf16<true>, g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
    else
      hipLaunchKernelGGL(k_pack_f32_to_bf16<false>, g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
  } else if (plan->dtype == DDP_FP32) {
    if (ntl)
      hipLaunchKernelGGL((k_pack<DDP_FP32, true>), g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
    else
      hipLaunchKernelGGL((k_pack<DDP_FP32, false>), g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
  } else {
    if (ntl)
      hipLaunchKernelGGL((k_pack<DDP_BF16, true>), g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
    else
      hipLaunchKernelGGL((k_pack<DDP_BF16, false>), g, blk, 0, s, sg, ts, bk.n_tiles, A, B);
  }
  DDP_HIP_TRY(hipGetLastError(), "bucket_pack: launch");
  return DDP_OK;
}

namespace ddp {

int unpack_scale_guarded(const ddp_plan* plan, int32_t b, const void* const* bucket_bufs, void* const* grad_arenas,
                         int32_t N, float scale, const unsigned int* abort_word, hipStream_t s) {
  const Bucket& bk = plan->buckets[b];
  if (bk.n_tiles == 0) return DDP_OK;
  const Segment* segs = nullptr;
  const int32_t* tile_seg = nullptr;
  int st = device_tables(const_cast<ddp_plan*>(plan), &segs, nullptr, &tile_seg);
  if (st != DDP_OK) return st;
  RankPtrs A{}, B{};
  for (int r = 0; r < N; ++r) {
    A.p[r] = grad_arenas[r];
    B.p[r] = const_cast<void*>(bucket_bufs[r]);
  }
  const dim3 g(copy_grid(bk.n_tiles), unsigned(N)), blk(kThreads);
  const Segment* sg = segs + bk.seg_begin;
  const int32_t* ts = tile_seg + bk.tile_seg_begin;
  // Non-temporal stores (same-dtype plans) once the N gradient arenas
  // together exceed the Infinity Cache: they would not stay cached for a
  // consumer anyway.
  const bool nts = int64_t(N) * plan->arena_numel * elem_bytes(plan->dtype) > kInfinityCacheBytes;
  const float sc = scale;
  if (plan->dtype != plan->comm_dtype) {
    if (nts)
      hipLaunchKernelGGL(k_unpack_bf16_to_f32<true>, g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
    else
      hipLaunchKernelGGL(k_unpack_bf16_to_f32<false>, g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
  } else if (plan->dtype == DDP_FP32) {
    if (nts)
      hipLaunchKernelGGL((k_unpack_scale<DDP_FP32, true>), g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
    else
      hipLaunchKernelGGL((k_unpack_scale<DDP_FP32, false>), g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
  } else {
    if (nts)
      hipLaunchKernelGGL((k_unpack_scale<DDP_BF16, true>), g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
    else
      hipLaunchKernelGGL((k_unpack_scale<DDP_BF16, false>), g, blk, 0, s, sg, ts, bk.n_tiles, B, A, sc, abort_word);
  }
  DDP_HIP_TRY(hipGetLastError(), "bucket_unpack_scale: launch");
  return DDP_OK;
}

int sync_bucket_persistent(const ddp_plan* plan, int32_t b, void* const* grad_arenas, void* const* bufs, int32_t N,
                           float scale, hipStream_t s) {
  // bucket_pack checks the arenas and buffers that the copy back uses too
  int st = bucket_pack(plan, b, const_cast<const void* const*>(grad_arenas), bufs, N, s);
  if (st != DDP_OK) return st;
  // One lease covers the all-reduce and the copy back, which reads the
  // launch's abort bit: the slot is not handed on before both have run.
  BarrierGuard lease(s);
  st = lease.acquire();
  if (st != DDP_OK) return st;
  st = persistent_allreduce_leased(bufs, N, plan->buckets[b].padded_numel, plan->comm_dtype, lease.words(),
                                   lease.status(), s);
  if (st != DDP_OK) return st;
  st = unpack_scale_guarded(plan, b, const_cast<const void* const*>(bufs), grad_arenas, N, scale, lease.words(), s);
  if (st != DDP_OK) return st;
  return lease.release();
}

}  // namespace ddp

extern "C" int bucket_unpack_scale(const ddp_plan* plan, int32_t b, const void* const* bucket_bufs,
                                   void* const* grad_arenas, int32_t N, float scale, void* stream) {
  int st = check_copy("bucket_unpack_scale", plan, b, grad_arenas, bucket_bufs, N);
  if (st != DDP_OK) return st;
  return unpack_scale_guarded(plan, b, bucket_bufs, grad_arenas, N, scale, nullptr, as_stream(stream));
}

extern "C" int ddp_sync(const ddp_plan* plan, void* const* grad_arenas, void* const* bucket_bufs,
                        int32_t N, int32_t variant, float scale, void* stream) {
  const char* fn = "ddp_sync";
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (variant != DDP_VARIANT_FUSED && variant != DDP_VARIANT_STEPS && variant != DDP_VARIANT_PERSISTENT &&
      variant != DDP_VARIANT_VIEW)
    return fail(DDP_EINVAL, std::string(fn) + ": unknown variant");
  if (grad_arenas == nullptr || (bucket_bufs == nullptr && variant != DDP_VARIANT_VIEW))
    return fail(DDP_EINVAL, std::string(fn) + ": pointer array is NULL");
  if (N != plan->world_size) return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  if (variant == DDP_VARIANT_VIEW) {
    // Every bucket is ready, so one launch covers the whole arena: each
    // element still takes its own bucket's chunk and ring order (the arena
    // map), so the result is that of the bucket-by-bucket sync.
    int st = check_view_arenas(plan, grad_arenas, N, fn);
    if (st != DDP_OK) return st;
    RankPtrs P{};
    for (int r = 0; r < N; ++r) P.p[r] = grad_arenas[r];
    return launch_view_arena(plan, P, N, scale, as_stream(stream));
  }
  for (int32_t b = 0; b < int32_t(plan->buckets.size()); ++b) {
    void* const* bufs = bucket_bufs + size_t(b) * N;
    const int64_t count = plan->buckets[b].padded_numel;
    if (variant == DDP_VARIANT_PERSISTENT) {
      // a persistent all-reduce that times out leaves the gradients unchanged
      int st = sync_bucket_persistent(plan, b, grad_arenas, bufs, N, scale, as_stream(stream));
      if (st != DDP_OK) return st;
      continue;
    }
    int st = bucket_pack(plan, b, const_cast<const void* const*>(grad_arenas), bufs, N, stream);
    if (st != DDP_OK) return st;
    if (variant == DDP_VARIANT_FUSED) {
      st = ring_allreduce_fused(bufs, N, count, plan->comm_dtype, stream);
    } else {
      for (int ph = DDP_RS; ph <= DDP_AG && st == DDP_OK; ++ph)
        for (int s = 0; s + 1 < N && st == DDP_OK; ++s)
          st = ring_allreduce_step(bufs, N, count, plan->comm_dtype, s, ph, stream);
    }
    if (st != DDP_OK) return st;
    st = bucket_unpack_scale(plan, b, const_cast<const void* const*>(bufs), grad_arenas, N, scale, stream);
    if (st != DDP_OK) return st;
  }
  return DDP_OK;
}
