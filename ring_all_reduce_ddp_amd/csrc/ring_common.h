// Argument checking and launch helpers shared by the ring kernels
// (ring_kernels.hip: step and persistent forms; fused_kernels.hip: fused form).
#pragma once

#include <algorithm>

#include "hip_common.h"

namespace ddp {

constexpr int64_t kMaxGrid = int64_t(1) << 22;

__device__ __forceinline__ int wrap(int x, int n) {  // x in [0, 2n)
  return x >= n ? x - n : x;
}

struct RingArgs {
  RankPtrs P{};
  int n = 0;
  int64_t count = 0;
  int64_t L = 0;
  bool vec = false;
};

inline int prepare(const char* fn, void* const* bufs, int32_t N, int64_t count, int32_t dtype, RingArgs* a) {
  if (!valid_dtype(dtype)) return fail(DDP_EINVAL, std::string(fn) + ": unknown dtype");
  if (N < 1 || N > DDP_MAX_RANKS) return fail(DDP_EINVAL, std::string(fn) + ": N must lie in [1, 64]");
  if (count < 0) return fail(DDP_EINVAL, std::string(fn) + ": count < 0");
  const int eb = elem_bytes(dtype);
  if (count > (int64_t(1) << 40)) return fail(DDP_EINVAL, std::string(fn) + ": count too large");
  int st = check_rank_buffers(bufs, N, count * eb, eb, fn, "bufs");
  if (st != DDP_OK) return st;
  a->n = N;
  a->count = count;
  a->L = (count + N - 1) / N;
  const int V = kVectorBytes / eb;
  a->vec = (a->L % V == 0) && all_aligned16(bufs, N);
  for (int r = 0; r < N; ++r) a->P.p[r] = bufs[r];
  return DDP_OK;
}

// Tiles of `tile` elements on a grid aligned to multiples of `tile` (not to
// chunk starts): a chunk [lo, lo + L) is covered by the tiles that intersect
// it, at most ceil(L / tile) + 1 of them.
inline int64_t aligned_tiles_per_chunk(int64_t L, int64_t tile) { return (L + tile - 1) / tile + 1; }

// Vector index handled by this thread in tile t of the chunk starting at
// element lo (the first tile starts at lo rounded down to a whole tile).
__device__ __forceinline__ int64_t tile_vector(int64_t lo, int64_t t, int threads, int V) {
  const int64_t tile = int64_t(threads) * V;
  return (lo / tile + t) * threads + threadIdx.x;
}

// Word d of a staged tile summed down the LDS rows (one row of `row_words`
// words per rank) in ring order: row `first`, then first+1, ..., first+n-1
// (mod n), one rounding per add. With a compile-time rank count the loop
// unrolls; otherwise rows are read eight at a time, so their LDS reads are in
// flight together instead of one round trip per rank.
template <int DT, int NR>
__device__ __forceinline__ typename Word<DT>::Acc ring_sum_rows(const uint32_t* words, int row_words, int first,
                                                               int n, int d) {
  using Wd = Word<DT>;
  typename Wd::Acc a = Wd::from(words[first * row_words + d]);
  if constexpr (NR > 0) {
#pragma unroll
    for (int k = 1; k < NR; ++k) Wd::add(a, words[wrap(first + k, NR) * row_words + d]);
  } else {
    int k = 1;
    for (; k + 8 <= n; k += 8) {
      uint32_t x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = words[wrap(first + k + j, n) * row_words + d];
#pragma unroll
      for (int j = 0; j < 8; ++j) Wd::add(a, x[j]);
    }
    for (; k < n; ++k) Wd::add(a, words[wrap(first + k, n) * row_words + d]);
  }
  return a;
}

// ---------------------------------------------------------------- spans (many ranks)
//
// With many ranks (kSpanMinRanks and up) a block that stages one tile of
// every rank touches N rank buffers, N distinct pages, at once, and the
// per-CU address-translation cache misses on ~5 % of requests at 64 ranks
// (0.01 % at 8). The span kernels (fused all-reduce, reduce-scatter output)
// instead have each block walk one span of kSpanVecs x kSpanThreads vectors
// of its chunk rank by rank, in the chunk's ring order, keeping the running
// sums in registers: at any moment a block reads one rank's pages (0.5 % of
// translation requests missed at 64 ranks). Same adds in the same order, so
// the same bits. Measured on MI355X at 64 ranks, fused all-reduce: 300M fp32
// 24.8 ms (6.2 TB/s) against 27.4 ms staged, 2^28 fp32 22.3 against 25.0 ms,
// 2^28 bf16 11.1 against 13.0 ms. At 24, 32 and 40 ranks the two forms ran
// alike, and at 52 and 56 the staged one was as fast or 1.5 % faster, so the
// span form starts between 56 and 64. Equal chunks of whole vectors only
// (count = N * L, L a multiple of V). Spans lie on a grid that starts at the
// chunk's start rounded down to 64 vectors (1 KiB), so interior spans begin
// on cache-line boundaries; the spans at a chunk's two ends clamp their loads
// into the chunk and store only their own vectors.

constexpr int kSpanThreads = 256;
constexpr int kSpanVecs = 4;  // vectors per thread per rank
constexpr int kSpanMinRanks = 60;
constexpr int64_t kSpanLen = int64_t(kSpanVecs) * kSpanThreads;  // vectors per span
constexpr int64_t kSpanAlign = 64;                                // span grid alignment, in vectors

// Spans per chunk of Lv vectors (the chunk's span grid starts up to 63
// vectors before the chunk).
inline int64_t spans_per_chunk(int64_t Lv) { return (Lv + kSpanAlign - 1 + kSpanLen - 1) / kSpanLen; }

// First vector of span s of the chunk that starts at vector lo.
__device__ __forceinline__ int64_t span_start(int64_t lo, int64_t s) { return lo / kSpanAlign * kSpanAlign + s * kSpanLen; }

// acc[j] = the ring-order sum (rank c+1 first, then c+2, ..., c; one rounding
// per add) of vector v0 + j * kSpanThreads of the N ranks. EDGE: the span
// reaches outside [lo, hi), so its loads are clamped into the chunk (the
// clamped lanes' sums are not stored).
template <int DT, bool NTL, bool EDGE>
__device__ __forceinline__ void span_ring_sum(const RankPtrs& P, int n, int c, int64_t lo, int64_t hi, int64_t v0,
                                              typename Ops<DT>::Acc (&acc)[kSpanVecs]) {
  using O = Ops<DT>;
  int64_t at[kSpanVecs];
#pragma unroll
  for (int j = 0; j < kSpanVecs; ++j) {
    const int64_t v = v0 + int64_t(j) * kSpanThreads;
    at[j] = EDGE ? std::min(std::max(v, lo), hi - 1) : v;
  }
  int r = wrap(c + 1, n);
  {
    const u32x4* src = static_cast<const u32x4*>(P.p[r]);
    u32x4 x[kSpanVecs];
#pragma unroll
    for (int j = 0; j < kSpanVecs; ++j) x[j] = ld16<NTL>(src + at[j]);
#pragma unroll
    for (int j = 0; j < kSpanVecs; ++j) acc[j] = O::from(x[j]);
  }
  for (int k = 1; k < n; ++k) {
    r = r + 1 == n ? 0 : r + 1;
    const u32x4* src = static_cast<const u32x4*>(P.p[r]);
    u32x4 x[kSpanVecs];
#pragma unroll
    for (int j = 0; j < kSpanVecs; ++j) x[j] = ld16<NTL>(src + at[j]);
#pragma unroll
    for (int j = 0; j < kSpanVecs; ++j) O::add(acc[j], x[j]);
  }
}

inline unsigned grid_for(int64_t total_tiles) {
  return unsigned(std::max<int64_t>(1, std::min(total_tiles, kMaxGrid)));
}

}  // namespace ddp
