// Reduce-scatter output of the ring: every rank's gradient shard.
//
// Page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03: after the N-1
// reduce-scatter steps each rank holds one chunk reduced over all ranks; page
// "DDP 与 Ring-AllReduce" (xuesongtap.github.io), §1.3.2.1: that chunk is chunk
// r on rank r. Section 07 of the first page separates DDP (every rank keeps
// the whole gradient) from FSDP/ZeRO (each rank keeps a shard); the shard is
// what the reduce-scatter phase alone produces.
//
// One pass: each element of chunk c is read once from every rank, summed in
// the order the hops add it (rank c+1 first, then c+2, ..., c; one rounding
// per add), multiplied by `scale` (one rounding) and written to rank c's
// shard. N*S bytes are read and S written; the input buffers are not
// modified. Launch shape and tile grid as for the fused all-reduce.
#include <algorithm>

#include "ring_common.h"

namespace ddp {
namespace {

constexpr int kScatterThreads = 64;
constexpr int kScatterBatch = 16;

// Vector vi of the N ranks summed in ring order from rank `first` (one
// rounding per add). NR > 0: compile-time rank count; NR == 0: any N, loaded
// kScatterBatch at a time.
template <int DT, int NR, bool NTL>
__device__ __forceinline__ typename Ops<DT>::Acc ring_sum_vec(const RankPtrs& P, int n, int first, int64_t vi) {
  using O = Ops<DT>;
  typename O::Acc a;
  if constexpr (NR > 0) {
    u32x4 x[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) x[k] = ld16<NTL>(static_cast<const u32x4*>(P.p[wrap(first + k, NR)]) + vi);
    a = O::from(x[0]);
#pragma unroll
    for (int k = 1; k < NR; ++k) O::add(a, x[k]);
  } else {
    a = O::from(ld16<NTL>(static_cast<const u32x4*>(P.p[first]) + vi));
    for (int k = 1; k < n; k += kScatterBatch) {
      u32x4 x[kScatterBatch];
#pragma unroll
      for (int j = 0; j < kScatterBatch; ++j)
        if (k + j < n) x[j] = ld16<NTL>(static_cast<const u32x4*>(P.p[wrap(first + k + j, n)]) + vi);
#pragma unroll
      for (int j = 0; j < kScatterBatch; ++j)
        if (k + j < n) O::add(a, x[j]);
    }
  }
  return a;
}

// Element e of the N ranks summed in ring order from rank `first`, scaled.
template <int DT>
__device__ __forceinline__ float ring_sum_elem(const RankPtrs& P, int n, int first, int64_t e, float scale) {
  using O = Ops<DT>;
  float acc = O::load1(P.p[first], e);
  for (int k = 1; k < n; ++k) acc = O::add1(acc, O::load1(P.p[wrap(first + k, n)], e));
  return O::mul1(acc, scale);
}

template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kScatterThreads) void k_scatter_vec(RankPtrs P, RankPtrs S, int n_rt, int64_t count,
                                                                 int64_t L, int64_t tiles_per_chunk,
                                                                 int64_t total_tiles, float scale) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  const int n = NR > 0 ? NR : n_rt;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int c = int(tile / tiles_per_chunk);
    const int64_t t = tile - int64_t(c) * tiles_per_chunk;
    const int64_t lo = int64_t(c) * L;
    const int64_t hi = min(lo + L, count);
    const int64_t vi = tile_vector(lo, t, kScatterThreads, V);
    if (vi * V < lo || vi * V >= hi) continue;
    const int first = wrap(c + 1, n);
    void* shard = S.p[c];
    if ((vi + 1) * V <= hi) {
      const typename O::Acc a = ring_sum_vec<DT, NR, NTL>(P, n, first, vi);
      st16<true>(static_cast<u32x4*>(shard) + (vi - lo / V), O::scale(O::to(a), scale));
    } else {
      for (int64_t e = vi * V; e < hi; ++e) O::store1(shard, e - lo, ring_sum_elem<DT>(P, n, first, e, scale));
    }
  }
}

// Chunk lengths that are not whole vectors: tiles run over the whole buffer
// from its 16-byte aligned start, so the loads stay 16-byte vectors. A
// vector inside one chunk is summed as a vector and written to the shard
// element by element (the shard's elements do not line up with the buffer's
// vectors); a vector cut by a chunk boundary or by the end of the buffer is
// done element by element, each element in its own chunk's order. A tile is
// never longer than a chunk here, so it crosses at most one boundary.
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kScatterThreads) void k_scatter_any(RankPtrs P, RankPtrs S, int n_rt, int64_t count,
                                                                 int64_t L, int64_t total_tiles, float scale) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  const int n = NR > 0 ? NR : n_rt;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int64_t tile_e = tile * kScatterThreads * V;
    const int64_t c0 = tile_e / L;  // chunk of the tile's first element
    const int64_t next = (c0 + 1) * L;
    const int64_t vi = tile * kScatterThreads + threadIdx.x;
    const int64_t e0 = vi * V;
    if (e0 >= count) continue;
    const int c = int(c0) + (e0 >= next ? 1 : 0);
    const int64_t lo = int64_t(c) * L;
    if (e0 + V <= min(lo + L, count)) {
      const typename O::Acc a = ring_sum_vec<DT, NR, NTL>(P, n, wrap(c + 1, n), vi);
      const u32x4 y = O::scale(O::to(a), scale);
      for (int j = 0; j < V; ++j) O::store1(S.p[c], e0 - lo + j, Word<DT>::elem(y, j));
    } else {
      for (int64_t e = e0; e < e0 + V && e < count; ++e) {
        const int ce = int(c0) + (e >= next ? 1 : 0);
        O::store1(S.p[ce], e - int64_t(ce) * L, ring_sum_elem<DT>(P, n, wrap(ce + 1, n), e, scale));
      }
    }
  }
}

// Fallback for unaligned buffers and for chunks shorter than a tile whose
// length is not a whole number of vectors: one element per thread.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_scatter_scalar(RankPtrs P, RankPtrs S, int n, int64_t count, int64_t L,
                                                             int64_t tiles_per_chunk, int64_t total_tiles,
                                                             float scale) {
  using O = Ops<DT>;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    const int c = int(tile / tiles_per_chunk);
    const int64_t lo = int64_t(c) * L;
    const int64_t hi = min(lo + L, count);
    const int64_t e = lo + (tile - int64_t(c) * tiles_per_chunk) * kThreads + threadIdx.x;
    if (e >= hi) continue;
    const int first = wrap(c + 1, n);
    float acc = O::load1(P.p[first], e);
    for (int k = 1; k < n; ++k) acc = O::add1(acc, O::load1(P.p[wrap(first + k, n)], e));
    O::store1(S.p[c], e - lo, O::mul1(acc, scale));
  }
}

// Many ranks, equal chunks of whole vectors (spans: ring_common.h): each
// block sums one span of its chunk rank by rank, then writes the scaled sums
// to the chunk's shard. Grid: (spans of a chunk from span s0 on, N chunks).
template <int DT, bool NTL, bool EDGE>
__device__ __forceinline__ void span_scatter(const RankPtrs& P, void* shard, int n, int c, int64_t lo, int64_t hi,
                                             int64_t v0, float scale) {
  using O = Ops<DT>;
  typename O::Acc acc[kSpanVecs];
  span_ring_sum<DT, NTL, EDGE>(P, n, c, lo, hi, v0, acc);
#pragma unroll
  for (int j = 0; j < kSpanVecs; ++j) {
    const int64_t v = v0 + int64_t(j) * kSpanThreads;
    if (!EDGE || (v >= lo && v < hi)) st16<true>(static_cast<u32x4*>(shard) + (v - lo), O::scale(O::to(acc[j]), scale));
  }
}

template <int DT, bool NTL>
__global__ __launch_bounds__(kSpanThreads) void k_scatter_span(RankPtrs P, RankPtrs S, int n, int64_t Lv, int64_t s0,
                                                               float scale) {
  const int c = int(blockIdx.y);
  const int64_t lo = int64_t(c) * Lv;
  const int64_t hi = lo + Lv;
  const int64_t b0 = span_start(lo, s0 + int64_t(blockIdx.x));
  if (b0 >= hi) return;
  if (b0 >= lo && b0 + kSpanLen <= hi)
    span_scatter<DT, NTL, false>(P, S.p[c], n, c, lo, hi, b0 + threadIdx.x, scale);
  else
    span_scatter<DT, NTL, true>(P, S.p[c], n, c, lo, hi, b0 + threadIdx.x, scale);
}

template <int DT, bool NTL>
void launch_scatter_span(const RingArgs& a, const RankPtrs& S, float scale, hipStream_t s) {
  const int64_t Lv = a.L / Ops<DT>::V;
  const int64_t spc = spans_per_chunk(Lv);
  for (int64_t s0 = 0; s0 < spc; s0 += kMaxGrid) {
    const dim3 g(unsigned(std::min(spc - s0, kMaxGrid)), unsigned(a.n));
    hipLaunchKernelGGL((k_scatter_span<DT, NTL>), g, dim3(kSpanThreads), 0, s, a.P, S, a.n, Lv, s0, scale);
  }
}

template <int DT, bool NTL>
void launch_scatter_vec(const RingArgs& a, const RankPtrs& S, float scale, hipStream_t s) {
  constexpr int V = Ops<DT>::V;
  const int64_t tpc = aligned_tiles_per_chunk(a.L, int64_t(kScatterThreads) * V);
  const int64_t total = tpc * a.n;
  const dim3 g(grid_for(total)), b(kScatterThreads);
  switch (a.n) {
#define DDP_SCATTER_CASE(NR)                                                                                  \
  case NR:                                                                                                    \
    hipLaunchKernelGGL((k_scatter_vec<DT, NR, NTL>), g, b, 0, s, a.P, S, a.n, a.count, a.L, tpc, total, scale); \
    break;
    DDP_SCATTER_CASE(1)
    DDP_SCATTER_CASE(2)
    DDP_SCATTER_CASE(3)
    DDP_SCATTER_CASE(4)
    DDP_SCATTER_CASE(5)
    DDP_SCATTER_CASE(6)
    DDP_SCATTER_CASE(7)
    DDP_SCATTER_CASE(8)
#undef DDP_SCATTER_CASE
    default:
      hipLaunchKernelGGL((k_scatter_vec<DT, 0, NTL>), g, b, 0, s, a.P, S, a.n, a.count, a.L, tpc, total, scale);
  }
}

template <int DT, bool NTL>
void launch_scatter_any(const RingArgs& a, const RankPtrs& S, float scale, hipStream_t s) {
  constexpr int V = Ops<DT>::V;
  const int64_t total = (a.count + int64_t(kScatterThreads) * V - 1) / (int64_t(kScatterThreads) * V);
  const dim3 g(grid_for(total)), b(kScatterThreads);
  switch (a.n) {
#define DDP_SCATTER_ANY_CASE(NR)                                                                           \
  case NR:                                                                                                 \
    hipLaunchKernelGGL((k_scatter_any<DT, NR, NTL>), g, b, 0, s, a.P, S, a.n, a.count, a.L, total, scale); \
    break;
    DDP_SCATTER_ANY_CASE(1)
    DDP_SCATTER_ANY_CASE(2)
    DDP_SCATTER_ANY_CASE(3)
    DDP_SCATTER_ANY_CASE(4)
    DDP_SCATTER_ANY_CASE(5)
    DDP_SCATTER_ANY_CASE(6)
    DDP_SCATTER_ANY_CASE(7)
    DDP_SCATTER_ANY_CASE(8)
#undef DDP_SCATTER_ANY_CASE
    default:
      hipLaunchKernelGGL((k_scatter_any<DT, 0, NTL>), g, b, 0, s, a.P, S, a.n, a.count, a.L, total, scale);
  }
}

template <int DT>
int launch_scatter(const RingArgs& a, const RankPtrs& S, bool shards_aligned, float scale, hipStream_t s) {
  const bool ntl = int64_t(a.n) * a.count * elem_bytes(DT) > kInfinityCacheBytes;
  if (a.vec && shards_aligned && a.count == int64_t(a.n) * a.L && a.n >= kSpanMinRanks) {
    if (ntl)
      launch_scatter_span<DT, true>(a, S, scale, s);
    else
      launch_scatter_span<DT, false>(a, S, scale, s);
  } else if (a.vec && shards_aligned) {
    if (ntl)
      launch_scatter_vec<DT, true>(a, S, scale, s);
    else
      launch_scatter_vec<DT, false>(a, S, scale, s);
  } else if (all_aligned16(const_cast<void* const*>(a.P.p), a.n) &&
             a.L >= int64_t(kScatterThreads) * Ops<DT>::V) {
    if (ntl)
      launch_scatter_any<DT, true>(a, S, scale, s);
    else
      launch_scatter_any<DT, false>(a, S, scale, s);
  } else {
    const int64_t tpc = (a.L + kThreads - 1) / kThreads;
    const int64_t total = tpc * a.n;
    hipLaunchKernelGGL((k_scatter_scalar<DT>), dim3(grid_for(total)), dim3(kThreads), 0, s, a.P, S, a.n, a.count,
                       a.L, tpc, total, scale);
  }
  DDP_HIP_TRY(hipGetLastError(), "ring_reduce_scatter_fused: launch");
  return DDP_OK;
}

}  // namespace
}  // namespace ddp

using namespace ddp;

extern "C" int ring_reduce_scatter_fused(const void* const* bufs, void* const* shards, int32_t N, int64_t count,
                                         int32_t dtype, float scale, void* stream) {
  const char* fn = "ring_reduce_scatter_fused";
  RingArgs a;
  int st = prepare(fn, const_cast<void* const*>(bufs), N, count, dtype, &a);
  if (st != DDP_OK) return st;
  if (shards == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": shards array is NULL");
  const int eb = elem_bytes(dtype);
  bool aligned = true;
  for (int c = 0; c < N; ++c) {
    const int64_t lo = std::min<int64_t>(int64_t(c) * a.L, count);
    const int64_t len = std::min<int64_t>(lo + a.L, count) - lo;
    const std::string name = "shards[" + std::to_string(c) + "]";
    if (len == 0) continue;
    if (shards[c] == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": " + name + " is NULL");
    if (reinterpret_cast<uintptr_t>(shards[c]) % uintptr_t(eb) != 0)
      return fail(DDP_EINVAL, std::string(fn) + ": " + name + " is not element-aligned");
    aligned = aligned && reinterpret_cast<uintptr_t>(shards[c]) % 16 == 0;
    st = check_range(shards[c], len * eb, fn, name.c_str());
    if (st != DDP_OK) return st;
    // a shard must not overlap any input buffer or another shard
    const uintptr_t x = reinterpret_cast<uintptr_t>(shards[c]);
    for (int r = 0; r < N; ++r) {
      const uintptr_t y = reinterpret_cast<uintptr_t>(bufs[r]);
      if (count > 0 && x < y + uint64_t(count * eb) && y < x + uint64_t(len * eb))
        return fail(DDP_EINVAL, std::string(fn) + ": " + name + " overlaps bufs[" + std::to_string(r) + "]");
      if (r != c && r < N) {
        const int64_t lo2 = std::min<int64_t>(int64_t(r) * a.L, count);
        const int64_t len2 = std::min<int64_t>(lo2 + a.L, count) - lo2;
        const uintptr_t z = reinterpret_cast<uintptr_t>(shards[r]);
        if (len2 > 0 && shards[r] != nullptr && x < z + uint64_t(len2 * eb) && z < x + uint64_t(len * eb))
          return fail(DDP_EINVAL, std::string(fn) + ": " + name + " overlaps shards[" + std::to_string(r) + "]");
      }
    }
  }
  if (count == 0) return DDP_OK;
  RankPtrs S{};
  for (int c = 0; c < N; ++c) S.p[c] = shards[c];
  hipStream_t s = as_stream(stream);
  return dtype == DDP_FP32 ? launch_scatter<DDP_FP32>(a, S, aligned, scale, s)
                           : launch_scatter<DDP_BF16>(a, S, aligned, scale, s);
}
