// Fused ring all-reduce: the whole two-phase ring in one pass over HBM.
//
// Per element, the steps of the ring (page "DDP 与 Ring All-Reduce",
// blog.vllbc.top, section 03; page "DDP 与 Ring-AllReduce", xuesongtap.github.io,
// §1.3.2.1 and §1.3.2.2) only ever combine the N ranks' values at the same
// position: chunk c's running sum starts as rank c+1's value, picks up ranks
// c+2, ..., c in that order with one rounding per add, and the finished sum
// is then copied to every rank. This kernel reads each element once from
// every rank, adds in exactly that order and writes the result to all N
// ranks: the final state of the 2(N-1) steps, bit for bit, with 2*N*S bytes
// of HBM traffic instead of 5*(N-1)*S.
#include "ring_common.h"

namespace ddp {
namespace {

// ---------------------------------------------------------------- fused
//
// Launch shape, measured on MI355X at 8 ranks x 1 GiB: one wave (64 threads)
// per block, one 16-byte vector per thread per rank, one tile per block, and
// non-temporal stores (the result is not read again by this kernel).
// Single-wave blocks retire independently, which kept the memory system
// busier than 256-thread blocks (5.86 vs 5.50 TB/s for fp32); grid-stride
// loops over a resident grid were slower still. Loads are non-temporal when
// the N buffers together exceed the 256 MB Infinity Cache; when they fit
// (a DDP bucket: 8 x 25 MiB) cached loads find data written just before
// (7.05 vs 6.65 TB/s). Tiles are numbered either chunk-major (tile t of
// chunk c is block c * tiles_per_chunk + t) or interleaved across chunks
// (block t * N + c); fp32 ran faster interleaved and bf16 chunk-major.

constexpr int kFusedThreads = 64;
constexpr int64_t kFusedCacheResidentBytes = int64_t(256) << 20;
constexpr int kFusedBatch = 16;   // ranks loaded together by the any-N kernel

template <int DT>
struct FusedOrder {
  static constexpr bool interleave = DT == DDP_FP32;
};

__device__ __forceinline__ void fused_tile(int64_t tile, int n, int64_t tiles_per_chunk, bool interleave,
                                           int* c, int64_t* t) {
  if (interleave) {
    *c = int(tile % n);
    *t = tile / n;
  } else {
    *c = int(tile / tiles_per_chunk);
    *t = tile - int64_t(*c) * tiles_per_chunk;
  }
}

template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kFusedThreads) void k_fused_vec(RankPtrs P, int64_t count, int64_t L,
                                                             int64_t tiles_per_chunk, int64_t total_tiles) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    int c;
    int64_t t;
    fused_tile(tile, NR, tiles_per_chunk, FusedOrder<DT>::interleave, &c, &t);
    const int64_t lo = int64_t(c) * L;
    const int64_t hi = min(lo + L, count);
    const int64_t vi = tile_vector(lo, t, kFusedThreads, V);
    if (vi * V < lo || vi * V >= hi) continue;
    // Ring order of chunk c: rank c+1 first, then c+2, ..., c.
    const void* src[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) src[k] = P.p[wrap(c + 1 + k, NR)];
    if ((vi + 1) * V <= hi) {
      u32x4 x[NR];
#pragma unroll
      for (int k = 0; k < NR; ++k) x[k] = ld16<NTL>(static_cast<const u32x4*>(src[k]) + vi);
      typename O::Acc a = O::from(x[0]);
#pragma unroll
      for (int k = 1; k < NR; ++k) O::add(a, x[k]);
      const u32x4 y = O::to(a);
#pragma unroll
      for (int r = 0; r < NR; ++r) st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    } else {
      // Ragged end of the buffer: the elements of this vector below `hi`.
      for (int64_t e = vi * V; e < hi; ++e) {
        float acc = O::load1(src[0], e);
        for (int k = 1; k < NR; ++k) acc = O::add1(acc, O::load1(src[k], e));
        for (int r = 0; r < NR; ++r) O::store1(P.p[r], e, acc);
      }
    }
  }
}

template <int DT, bool NTL>
__global__ __launch_bounds__(kFusedThreads) void k_fused_vec_n(RankPtrs P, int n, int64_t count, int64_t L,
                                                               int64_t tiles_per_chunk, int64_t total_tiles) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  for (int64_t tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    int c;
    int64_t t;
    fused_tile(tile, n, tiles_per_chunk, FusedOrder<DT>::interleave, &c, &t);
    const int64_t lo = int64_t(c) * L;
    const int64_t hi = min(lo + L, count);
    const int64_t vi = tile_vector(lo, t, kFusedThreads, V);
    if (vi * V < lo || vi * V >= hi) continue;
    const int first = wrap(c + 1, n);
    if ((vi + 1) * V <= hi) {
      typename O::Acc a = O::from(ld16<NTL>(static_cast<const u32x4*>(P.p[first]) + vi));
      // Ranks c+2, ..., c in order, loaded kFusedBatch at a time.
      for (int k = 1; k < n; k += kFusedBatch) {
        u32x4 x[kFusedBatch];
#pragma unroll
        for (int j = 0; j < kFusedBatch; ++j)
          if (k + j < n) x[j] = ld16<NTL>(static_cast<const u32x4*>(P.p[wrap(first + k + j, n)]) + vi);
#pragma unroll
        for (int j = 0; j < kFusedBatch; ++j)
          if (k + j < n) O::add(a, x[j]);
      }
      const u32x4 y = O::to(a);
      for (int r = 0; r < n; ++r) st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    } else {
      for (int64_t e = vi * V; e < hi; ++e) {
        float acc = O::load1(P.p[first], e);
        for (int k = 1; k < n; ++k) acc = O::add1(acc, O::load1(P.p[wrap(first + k, n)], e));
        for (int r = 0; r < n; ++r) O::store1(P.p[r], e, acc);
      }
    }
  }
}

// ---------------------------------------------------------------- one element per thread
// Fallback for chunks that do not start on 16-byte boundaries.

template <int DT>
__global__ __launch_bounds__(kThreads) void k_fused_scalar(RankPtrs P, int n, int64_t count, int64_t L,
                                                           int64_t tiles_per_chunk, int64_t total_tiles) {
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
    for (int r = 0; r < n; ++r) O::store1(P.p[r], e, acc);
  }
}

template <int DT, bool NTL>
void launch_fused_vec(const RingArgs& a, hipStream_t s) {
  constexpr int V = Ops<DT>::V;
  const int64_t tpc = aligned_tiles_per_chunk(a.L, int64_t(kFusedThreads) * V);
  const int64_t total = tpc * a.n;
  const dim3 g(grid_for(total)), b(kFusedThreads);
  switch (a.n) {
#define DDP_FUSED_CASE(NR)                                                                      \
  case NR:                                                                                      \
    hipLaunchKernelGGL((k_fused_vec<DT, NR, NTL>), g, b, 0, s, a.P, a.count, a.L, tpc, total);  \
    break;
    DDP_FUSED_CASE(2)
    DDP_FUSED_CASE(3)
    DDP_FUSED_CASE(4)
    DDP_FUSED_CASE(5)
    DDP_FUSED_CASE(6)
    DDP_FUSED_CASE(7)
    DDP_FUSED_CASE(8)
#undef DDP_FUSED_CASE
    default:
      hipLaunchKernelGGL((k_fused_vec_n<DT, NTL>), g, b, 0, s, a.P, a.n, a.count, a.L, tpc, total);
  }
}

template <int DT>
int launch_fused(const RingArgs& a, hipStream_t s) {
  if (a.vec) {
    if (int64_t(a.n) * a.count * elem_bytes(DT) > kFusedCacheResidentBytes)
      launch_fused_vec<DT, true>(a, s);
    else
      launch_fused_vec<DT, false>(a, s);
  } else {
    const int64_t tpc = (a.L + kThreads - 1) / kThreads;
    const int64_t total = tpc * a.n;
    hipLaunchKernelGGL((k_fused_scalar<DT>), dim3(grid_for(total)), dim3(kThreads), 0, s, a.P, a.n,
                       a.count, a.L, tpc, total);
  }
  DDP_HIP_TRY(hipGetLastError(), "ring_allreduce_fused: launch");
  return DDP_OK;
}

}  // namespace
}  // namespace ddp

using namespace ddp;

extern "C" int ring_allreduce_fused(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                    void* stream) {
  RingArgs a;
  int st = prepare("ring_allreduce_fused", bufs, N, count, dtype, &a);
  if (st != DDP_OK) return st;
  if (count == 0 || N == 1) return DDP_OK;  // one rank: the ring has no steps
  return dtype == DDP_FP32 ? launch_fused<DDP_FP32>(a, as_stream(stream))
                           : launch_fused<DDP_BF16>(a, as_stream(stream));
}

