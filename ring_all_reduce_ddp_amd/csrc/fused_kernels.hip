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
// Launch shape, measured on MI355X at 8 ranks x 1 GiB fp32. A tile is 64
// vectors of 16 bytes of one chunk, on a grid aligned to whole tiles, and a
// block has one wave per rank (N <= 8; above that eight waves, each taking
// every eighth rank). Wave w loads rank w's tile into LDS row w, the block
// sums each 32-bit word down the rows in ring order, and wave w stores the
// result to rank w: every wave streams one rank's buffer, one load and one
// store per lane. That ran at 6.3-6.4 TB/s, where one-wave blocks that each
// read all N ranks and write all N ranks reached 5.7-5.9 TB/s on the same
// parts (the best copy kernel: 6.7 TB/s); the staged form also leaves far
// more room to a compute kernel running beside it on another stream. Tiles go chunk by chunk (chunk-major
// and chunk-interleaved orders ran alike at 1 GiB, chunk-major faster at
// 24 MiB per rank). Stores are non-temporal (the result is not read again
// here); loads are too when the N buffers together exceed the 256 MB
// Infinity Cache, and cached when they fit (a DDP bucket: 8 x 25 MiB), so
// they find data written just before.

constexpr int kFusedThreads = 64;   // threads per wave and vectors per rank tile
constexpr int kFusedMaxWaves = 8;

// LDS for one tile of every rank: a fixed array for a compile-time rank
// count, else the launch's dynamic LDS (N KiB).
template <int NR>
__device__ __forceinline__ u32x4* staged_tile() {
  if constexpr (NR > 0) {
    __shared__ u32x4 tile[NR * kFusedThreads];
    return tile;
  } else {
    extern __shared__ u32x4 dyn[];
    return dyn;
  }
}

// NR > 0: compile-time rank count and NR waves; NR == 0: any N, kFusedMaxWaves
// waves, each taking every kFusedMaxWaves-th rank. LDS: N rows of one tile
// (N KiB); the sum overwrites row 0 word by word (each word is read and
// written by one thread only). Grid: (tiles of a chunk from tile t0 on, N
// chunks); each block does one tile, so it knows its chunk without a
// division, blocks run chunk by chunk, and nothing loops (a grid-stride
// form of the same kernel, with a barrier before each refill of the stage,
// ran ~6 % slower).
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kFusedThreads * kFusedMaxWaves) void k_fused_staged(RankPtrs P, int n_rt, int64_t count,
                                                                               int64_t L, int64_t t0) {
  using O = Ops<DT>;
  using Wd = Word<DT>;
  constexpr int V = O::V;
  constexpr int W = NR > 0 ? NR : kFusedMaxWaves;
  constexpr int kSlots = NR > 0 ? 1 : DDP_MAX_RANKS / kFusedMaxWaves;  // ranks per wave, at most
  constexpr int kWords = kFusedThreads * 4;  // 32-bit words per rank tile
  constexpr int64_t kTile = int64_t(kFusedThreads) * V;
  u32x4* stage = staged_tile<NR>();
  const int n = NR > 0 ? NR : n_rt;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kFusedThreads);
  const int lane = int(threadIdx.x) % kFusedThreads;
  const int c = int(blockIdx.y);
  const int64_t lo = int64_t(c) * L;
  const int64_t hi = min(lo + L, count);
  const int64_t vi = (lo / kTile + t0 + blockIdx.x) * kFusedThreads + lane;
  const int64_t e0 = vi * V;
  const bool mine = e0 >= lo && e0 < hi;
  const bool full = e0 + V <= hi;
  if (mine) {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int r = wave + j * W;
      if (r < n) {
        const u32x4* src = static_cast<const u32x4*>(P.p[r]);
        stage[r * kFusedThreads + lane] = full ? ld16<NTL>(src + vi) : Wd::load_partial(src, e0, int(hi - e0));
      }
    }
  }
  __syncthreads();
  // Ring order of chunk c: rank c+1 first, then c+2, ..., c.
  const int first = wrap(c + 1, n);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(stage);
  uint32_t* result = reinterpret_cast<uint32_t*>(stage);
  for (int d = threadIdx.x; d < kWords; d += W * kFusedThreads) {
    result[d] = Wd::out(ring_sum_rows<DT, NR>(words, kWords, first, n, d));
  }
  __syncthreads();
  if (!mine) return;
  const u32x4 y = stage[lane];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int r = wave + j * W;
    if (r >= n) continue;
    if (full) {
      st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    } else {
      // Ragged end of the buffer: the elements of this vector below `hi`.
      for (int i = 0; i < int(hi - e0); ++i) O::store1(P.p[r], e0 + i, Wd::elem(y, i));
    }
  }
}

// Buffers cut into N equal chunks of whole tiles (count = N * L, L a multiple
// of 64 vectors: 8 x 1 GiB, one 8 x 25 MiB bucket): every tile lies inside
// its chunk, so nothing is bounds-checked, and each rank's tile is staged in
// the LDS row of its place in the chunk's ring order (rank c+1 in row 0, rank
// c+2 in row 1, ...), so the sum reads rows 0, 1, ..., N-1 at fixed offsets.
// The additions and their order are those of k_fused_staged; the lighter
// index work before the loads measured 6.55 against 6.47 TB/s at 8 x 1 GiB
// fp32 in a stand-alone copy of the same access pattern.
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kFusedThreads * kFusedMaxWaves) void k_fused_whole(RankPtrs P, int n_rt,
                                                                              int64_t tiles_per_chunk, int64_t t0) {
  using Wd = Word<DT>;
  constexpr int W = NR > 0 ? NR : kFusedMaxWaves;
  constexpr int kSlots = NR > 0 ? 1 : DDP_MAX_RANKS / kFusedMaxWaves;
  constexpr int kWords = kFusedThreads * 4;
  u32x4* stage = staged_tile<NR>();
  const int n = NR > 0 ? NR : n_rt;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kFusedThreads);
  const int lane = int(threadIdx.x) % kFusedThreads;
  const int c = int(blockIdx.y);
  const int first = wrap(c + 1, n);  // the chunk's ring order starts at rank c+1
  const int64_t vi = (int64_t(c) * tiles_per_chunk + t0 + blockIdx.x) * kFusedThreads + lane;
  if constexpr (NR > 0) {
    // One wave per rank: wave w is rank w.
    u32x4* buf = static_cast<u32x4*>(P.p[wave]);
    stage[wrap(wave + NR - first, NR) * kFusedThreads + lane] = ld16<NTL>(buf + vi);
  } else {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int r = wave + j * W;
      if (r < n)
        stage[wrap(r + n - first, n) * kFusedThreads + lane] = ld16<NTL>(static_cast<const u32x4*>(P.p[r]) + vi);
    }
  }
  __syncthreads();
  const uint32_t* words = reinterpret_cast<const uint32_t*>(stage);
  uint32_t* result = reinterpret_cast<uint32_t*>(stage);
  for (int d = threadIdx.x; d < kWords; d += W * kFusedThreads)
    result[d] = Wd::out(ring_sum_rows<DT, NR>(words, kWords, 0, n, d));
  __syncthreads();
  const u32x4 y = stage[lane];
  if constexpr (NR > 0) {
    st16<true>(static_cast<u32x4*>(P.p[wave]) + vi, y);
  } else {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int r = wave + j * W;
      if (r < n) st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    }
  }
}

// Chunk lengths that are not whole 16-byte vectors (an all-reduce of any
// count; DDP buckets are padded and never need this): the tiles run over the
// whole buffer from its 16-byte aligned start, so loads and stores stay
// 16-byte vectors and staged as above, and in the sum each element takes the
// ring order of its own chunk (a tile is never longer than a chunk here, so
// it crosses at most one chunk boundary). A bf16 word whose two elements lie
// in different chunks sums each half in its own order.
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kFusedThreads * kFusedMaxWaves) void k_fused_any(RankPtrs P, int n_rt, int64_t count,
                                                                            int64_t L, int64_t t0) {
  using O = Ops<DT>;
  using Wd = Word<DT>;
  constexpr int V = O::V;
  constexpr int W = NR > 0 ? NR : kFusedMaxWaves;
  constexpr int kSlots = NR > 0 ? 1 : DDP_MAX_RANKS / kFusedMaxWaves;
  constexpr int kWords = kFusedThreads * 4;
  constexpr int EPW = V / 4;  // elements per 32-bit word: 1 for fp32, 2 for bf16
  u32x4* stage = staged_tile<NR>();
  const int n = NR > 0 ? NR : n_rt;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kFusedThreads);
  const int lane = int(threadIdx.x) % kFusedThreads;
  const int64_t tile = t0 + blockIdx.x;
  const int64_t tile_e = tile * kFusedThreads * V;  // the tile's first element
  const int64_t vi = tile * kFusedThreads + lane;
  const int64_t e0 = vi * V;
  const bool mine = e0 < count;
  const bool full = e0 + V <= count;
  if (mine) {
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const int r = wave + j * W;
      if (r < n) {
        const u32x4* src = static_cast<const u32x4*>(P.p[r]);
        stage[r * kFusedThreads + lane] = full ? ld16<NTL>(src + vi) : Wd::load_partial(src, e0, int(count - e0));
      }
    }
  }
  __syncthreads();
  const int64_t c0 = tile_e / L;  // chunk of the tile's first element
  const int64_t next = (c0 + 1) * L;
  const uint32_t* words = reinterpret_cast<const uint32_t*>(stage);
  uint32_t* result = reinterpret_cast<uint32_t*>(stage);
  for (int d = threadIdx.x; d < kWords; d += W * kFusedThreads) {
    const int64_t e = tile_e + int64_t(d) * EPW;  // first element of word d
    if (e >= count) continue;
    const int c = int(c0) + (e >= next ? 1 : 0);
    if constexpr (EPW == 1) {
      result[d] = Wd::out(ring_sum_rows<DT, NR>(words, kWords, wrap(c + 1, n), n, d));
    } else {
      const int c_hi = int(c0) + (e + 1 >= next ? 1 : 0);
      if (c_hi == c || e + 1 >= count) {
        result[d] = Wd::out(ring_sum_rows<DT, NR>(words, kWords, wrap(c + 1, n), n, d));
      } else {
        // Each half in its own chunk's order, one rounding per add.
        const int f_lo = wrap(c + 1, n), f_hi = wrap(c_hi + 1, n);
        float lo = bf16_lo(words[f_lo * kWords + d]);
        float hi = bf16_hi(words[f_hi * kWords + d]);
        for (int k = 1; k < n; ++k) {
          lo = round_bf16(lo + bf16_lo(words[wrap(f_lo + k, n) * kWords + d]));
          hi = round_bf16(hi + bf16_hi(words[wrap(f_hi + k, n) * kWords + d]));
        }
        result[d] = bf16_pack(lo, hi);
      }
    }
  }
  __syncthreads();
  if (!mine) return;
  const u32x4 y = stage[lane];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int r = wave + j * W;
    if (r >= n) continue;
    if (full) {
      st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    } else {
      for (int i = 0; i < int(count - e0); ++i) O::store1(P.p[r], e0 + i, Wd::elem(y, i));
    }
  }
}

// ---------------------------------------------------------------- many ranks
// The span form of the fused all-reduce (spans: ring_common.h): each block
// sums one span of its chunk rank by rank and then writes it to every rank.

template <int DT, bool NTL, bool EDGE>
__device__ __forceinline__ void span_allreduce(const RankPtrs& P, int n, int c, int64_t lo, int64_t hi, int64_t v0) {
  using O = Ops<DT>;
  typename O::Acc acc[kSpanVecs];
  span_ring_sum<DT, NTL, EDGE>(P, n, c, lo, hi, v0, acc);
  u32x4 y[kSpanVecs];
#pragma unroll
  for (int j = 0; j < kSpanVecs; ++j) y[j] = O::to(acc[j]);
  for (int q = 0; q < n; ++q) {
    u32x4* dst = static_cast<u32x4*>(P.p[q]);
#pragma unroll
    for (int j = 0; j < kSpanVecs; ++j) {
      const int64_t v = v0 + int64_t(j) * kSpanThreads;
      if (!EDGE || (v >= lo && v < hi)) st16<true>(dst + v, y[j]);
    }
  }
}

// Grid: (spans of a chunk from span s0 on, N chunks). Lv is the chunk length
// in vectors.
template <int DT, bool NTL>
__global__ __launch_bounds__(kSpanThreads) void k_fused_span(RankPtrs P, int n, int64_t Lv, int64_t s0) {
  const int c = int(blockIdx.y);
  const int64_t lo = int64_t(c) * Lv;
  const int64_t hi = lo + Lv;
  const int64_t b0 = span_start(lo, s0 + int64_t(blockIdx.x));
  if (b0 >= hi) return;
  if (b0 >= lo && b0 + kSpanLen <= hi)
    span_allreduce<DT, NTL, false>(P, n, c, lo, hi, b0 + threadIdx.x);
  else
    span_allreduce<DT, NTL, true>(P, n, c, lo, hi, b0 + threadIdx.x);
}

// ---------------------------------------------------------------- one element per thread
// Fallback for buffers that do not start on 16-byte boundaries, and for
// chunks shorter than a tile whose length is not a whole number of vectors.

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
  // One block per tile; chunks longer than kMaxGrid tiles take several launches.
  for (int64_t t0 = 0; t0 < tpc; t0 += kMaxGrid) {
    const dim3 g(unsigned(std::min(tpc - t0, kMaxGrid)), unsigned(a.n));
    switch (a.n) {
#define DDP_FUSED_CASE(NR)                                                                                 \
  case NR:                                                                                                 \
    hipLaunchKernelGGL((k_fused_staged<DT, NR, NTL>), g, dim3(kFusedThreads * NR), 0, s, a.P, a.n, a.count, \
                       a.L, t0);                                                                            \
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
        hipLaunchKernelGGL((k_fused_staged<DT, 0, NTL>), g, dim3(kFusedThreads * kFusedMaxWaves),
                           size_t(a.n) * kFusedThreads * sizeof(u32x4), s, a.P, a.n, a.count, a.L, t0);
    }
  }
}

template <int DT, bool NTL>
void launch_fused_whole(const RingArgs& a, hipStream_t s) {
  const int64_t tpc = a.L / (int64_t(kFusedThreads) * Ops<DT>::V);
  for (int64_t t0 = 0; t0 < tpc; t0 += kMaxGrid) {
    const dim3 g(unsigned(std::min(tpc - t0, kMaxGrid)), unsigned(a.n));
    switch (a.n) {
#define DDP_FUSED_WHOLE_CASE(NR)                                                                            \
  case NR:                                                                                                  \
    hipLaunchKernelGGL((k_fused_whole<DT, NR, NTL>), g, dim3(kFusedThreads * NR), 0, s, a.P, a.n, tpc, t0); \
    break;
      DDP_FUSED_WHOLE_CASE(2)
      DDP_FUSED_WHOLE_CASE(3)
      DDP_FUSED_WHOLE_CASE(4)
      DDP_FUSED_WHOLE_CASE(5)
      DDP_FUSED_WHOLE_CASE(6)
      DDP_FUSED_WHOLE_CASE(7)
      DDP_FUSED_WHOLE_CASE(8)
#undef DDP_FUSED_WHOLE_CASE
      default:
        hipLaunchKernelGGL((k_fused_whole<DT, 0, NTL>), g, dim3(kFusedThreads * kFusedMaxWaves),
                           size_t(a.n) * kFusedThreads * sizeof(u32x4), s, a.P, a.n, tpc, t0);
    }
  }
}

template <int DT, bool NTL>
void launch_fused_any(const RingArgs& a, hipStream_t s) {
  constexpr int V = Ops<DT>::V;
  const int64_t tiles = (a.count + int64_t(kFusedThreads) * V - 1) / (int64_t(kFusedThreads) * V);
  for (int64_t t0 = 0; t0 < tiles; t0 += kMaxGrid) {
    const dim3 g(unsigned(std::min(tiles - t0, kMaxGrid)));
    switch (a.n) {
#define DDP_FUSED_ANY_CASE(NR)                                                                            \
  case NR:                                                                                                \
    hipLaunchKernelGGL((k_fused_any<DT, NR, NTL>), g, dim3(kFusedThreads * NR), 0, s, a.P, a.n, a.count,  \
                       a.L, t0);                                                                           \
    break;
      DDP_FUSED_ANY_CASE(2)
      DDP_FUSED_ANY_CASE(3)
      DDP_FUSED_ANY_CASE(4)
      DDP_FUSED_ANY_CASE(5)
      DDP_FUSED_ANY_CASE(6)
      DDP_FUSED_ANY_CASE(7)
      DDP_FUSED_ANY_CASE(8)
#undef DDP_FUSED_ANY_CASE
      default:
        hipLaunchKernelGGL((k_fused_any<DT, 0, NTL>), g, dim3(kFusedThreads * kFusedMaxWaves),
                           size_t(a.n) * kFusedThreads * sizeof(u32x4), s, a.P, a.n, a.count, a.L, t0);
    }
  }
}

template <int DT, bool NTL>
void launch_fused_span(const RingArgs& a, hipStream_t s) {
  const int64_t Lv = a.L / Ops<DT>::V;
  const int64_t spc = spans_per_chunk(Lv);
  for (int64_t s0 = 0; s0 < spc; s0 += kMaxGrid) {
    const dim3 g(unsigned(std::min(spc - s0, kMaxGrid)), unsigned(a.n));
    hipLaunchKernelGGL((k_fused_span<DT, NTL>), g, dim3(kSpanThreads), 0, s, a.P, a.n, Lv, s0);
  }
}

template <int DT>
int launch_fused(const RingArgs& a, hipStream_t s) {
  const bool ntl = int64_t(a.n) * a.count * elem_bytes(DT) > kInfinityCacheBytes;
  const int64_t tile = int64_t(kFusedThreads) * Ops<DT>::V;
  if (a.vec && a.count == int64_t(a.n) * a.L && a.n >= kSpanMinRanks) {
    if (ntl)
      launch_fused_span<DT, true>(a, s);
    else
      launch_fused_span<DT, false>(a, s);
  } else if (a.vec && a.count == int64_t(a.n) * a.L && a.L % tile == 0) {
    if (ntl)
      launch_fused_whole<DT, true>(a, s);
    else
      launch_fused_whole<DT, false>(a, s);
  } else if (a.vec) {
    if (ntl)
      launch_fused_vec<DT, true>(a, s);
    else
      launch_fused_vec<DT, false>(a, s);
  } else if (all_aligned16(const_cast<void* const*>(a.P.p), a.n) &&
             a.L >= int64_t(kFusedThreads) * Ops<DT>::V) {
    if (ntl)
      launch_fused_any<DT, true>(a, s);
    else
      launch_fused_any<DT, false>(a, s);
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

