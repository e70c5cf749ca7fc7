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

inline unsigned grid_for(int64_t total_tiles) {
  return unsigned(std::max<int64_t>(1, std::min(total_tiles, kMaxGrid)));
}

}  // namespace ddp
