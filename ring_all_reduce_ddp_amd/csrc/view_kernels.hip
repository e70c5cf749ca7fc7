// In-place DDP sync: the gradients are the bucket (the analogue of DDP's
// gradient_as_bucket_view=True).
//
// Page "DDP 与 Ring All-Reduce" (blog.vllbc.top), sections 03 and 05, and page
// "Day 17 数据并行 DP/DDP" (blog.ans20xx.com), part "bucket 与 overlap": with
// gradient_as_bucket_view=True each .grad is a view into its bucket, so the
// copies between gradients and bucket disappear, along with one gradient's
// worth of peak memory. Here the bucket is never materialised at all: every
// element keeps its position in the bucket's layout (so it belongs to the
// same ring chunk and is summed in the same rank order as in the copying
// path), but it is read from and written back to the gradient arena where it
// lives. One launch per bucket reads each member element from all N ranks,
// sums in ring order (chunk c: rank c+1 first, then c+2, ..., c; one rounding
// per add), multiplies by `scale` (one rounding) and writes the result to all
// N ranks: bit for bit the result of bucket_pack + ring all-reduce +
// bucket_unpack_scale, with 2*N*S bytes of traffic per bucket instead of
// 6*N*S. The padding of the bucket is never touched.
//
// A bucket's members are a run of consecutive parameters, so they fill one
// stretch of the arena (with the alignment padding between them). Tiles of
// 64 vectors of 16 bytes per rank cover that stretch on a grid aligned to
// whole tiles, so a block's addresses follow from its index alone. The plan
// keeps a map with one entry per arena vector (its ring chunk, or padding),
// loaded alongside the data; a per-tile descriptor fetched first (one
// dependent load before the data loads could go out) cost ~13 % of the
// bandwidth on ResNet-50's buckets, a binary search over the members' runs
// a third. Each tile is staged through LDS so that each wave streams one
// rank's arena (one load and one store per lane and rank) instead of every
// wave touching all N arenas. Measured on MI355X under a concurrent
// compute-bound kernel on another stream, the staged form hid all but
// ~0.05 ms of a 0.30 ms sync, where one-wave blocks that each read all N
// ranks exposed ~0.21 ms of it. Stores are non-temporal; loads are too when
// the ranks' arenas together exceed the Infinity Cache.
//
// A plan with fp32 gradients and bf16 buckets (the bf16 compression hook;
// page "Day 17 数据并行 DP/DDP", reading list, "PyTorch DDP Communication
// Hooks") syncs in place too, like DDP with gradient_as_bucket_view=True and
// the bf16 hook: the fp32 gradients are the bucket, and the hook rounds them
// to bf16, all-reduces in bf16 and writes the result back in fp32. Per
// element: each rank's gradient is rounded to bf16 as it enters the ring,
// every hop adds in bf16 with one rounding, and the sum times `scale` is
// rounded once to fp32: bit for bit the bf16 pack, the bf16 ring and the
// copy back to fp32, with no bf16 bucket in memory.
#include <algorithm>

#include "ring_common.h"

namespace ddp {

// Element type of the in-place sync of a compressed plan: fp32 in memory,
// bf16 in the ring's arithmetic.
constexpr int kF32ViaBf16 = 2;

template <>
struct Ops<kF32ViaBf16> : Ops<DDP_FP32> {};

template <>
struct Word<kF32ViaBf16> {
  struct Acc {
    float v;  // a bf16 value, as an fp32 number with the low 16 bits clear
  };
  static __device__ __forceinline__ Acc from(uint32_t w) { return Acc{round_bf16(__uint_as_float(w))}; }
  static __device__ __forceinline__ void add(Acc& a, uint32_t w) {
    a.v = round_bf16(a.v + round_bf16(__uint_as_float(w)));
  }
  static __device__ __forceinline__ uint32_t out(const Acc& a, float s) { return __float_as_uint(a.v * s); }
  static __device__ __forceinline__ float elem(u32x4 y, int j) { return __uint_as_float(y[j]); }
};

namespace {

constexpr int kViewMaxWaves = 8;  // waves per block (one rank each, or every 8th rank when N > 8)

// One tile of the in-place sync: arena vectors [64 * tile, 64 * tile + 64),
// those of them inside the bucket's span [v_begin, v_end). The tile's
// position alone gives every address, so the loads go out at once; the map
// entry of each vector (its ring chunk, or padding) arrives alongside. The
// tile is staged through LDS so that every wave streams a single rank's
// arena: wave w loads ranks w, w+W, ... into LDS row r (one 16-byte vector
// per lane), the block sums each 32-bit word down the rows in the ring
// order of its vector's chunk (chunk c: rank c+1 first, then c+2, ..., c;
// one rounding per add) and scales it, and wave w stores the result to its
// ranks, member elements only. NR > 0: compile-time rank count and NR
// waves; NR == 0: any N, kViewMaxWaves waves. LDS: N rows of one tile
// (N KiB); the scaled result overwrites row 0 word by word (each word is
// read and written by one thread only).
template <int DT, int NR, bool NTL>
__device__ __forceinline__ void view_tile(int64_t tile, const uint16_t* info, int64_t v_begin, int64_t v_end,
                                          u32x4* stage, uint16_t* info_of, const RankPtrs& P, int n, float scale) {
  using O = Ops<DT>;
  using Wd = Word<DT>;
  constexpr int V = O::V;
  constexpr int W = NR > 0 ? NR : kViewMaxWaves;
  constexpr int kWords = kViewThreads * 4;  // 32-bit words per rank tile (4 per vector)
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kViewThreads);
  const int lane = int(threadIdx.x) % kViewThreads;
  constexpr int kSlots = NR > 0 ? 1 : DDP_MAX_RANKS / kViewMaxWaves;  // ranks per wave, at most
  const int64_t vi = tile * kViewThreads + lane;
  const bool in = vi >= v_begin && vi < v_end;
  // One wave fetches the map entries and shares them through LDS; every
  // load is issued before any is waited for.
  const uint16_t f = (wave == 0 && in) ? info[vi] : kVecSlack;
  u32x4 x[kSlots];
  if (in) {
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      if (wave + j * W < n) x[j] = ld16<NTL>(static_cast<const u32x4*>(P.p[wave + j * W]) + vi);
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      if (wave + j * W < n) stage[(wave + j * W) * kViewThreads + lane] = x[j];
  }
  if (wave == 0) info_of[lane] = f;
  __syncthreads();
  const uint32_t* words = reinterpret_cast<const uint32_t*>(stage);
  uint32_t* result = reinterpret_cast<uint32_t*>(stage);
  for (int d = threadIdx.x; d < kWords; d += W * kViewThreads) {
    const int c = info_of[d >> 2] & 0xff;
    if (c == 0xff) continue;  // padding between members
    const int first = wrap(c + 1, n);
    result[d] = Wd::out(ring_sum_rows<DT, NR>(words, kWords, first, n, d), scale);
  }
  __syncthreads();
  const uint16_t g = info_of[lane];
  if (g == kVecSlack) return;
  const int valid = g >> 8;
  const u32x4 y = stage[lane];
  if (valid == V) {
    for (int r = wave; r < n; r += W) st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
  } else {
    // A member's last vector: its elements only, not the padding after it.
    for (int r = wave; r < n; r += W)
      for (int j = 0; j < valid; ++j) O::store1(P.p[r], vi * V + j, Wd::elem(y, j));
  }
}

template <int NR>
__device__ __forceinline__ u32x4* view_stage() {
  if constexpr (NR > 0) {
    __shared__ u32x4 rows[NR * kViewThreads];
    return rows;
  } else {
    extern __shared__ u32x4 dyn[];
    return dyn;
  }
}

// One block per tile, tiles tile0, tile0 + 1, ... (nothing loops: a
// grid-stride loop cost the fused all-reduce ~6 % of its bandwidth).
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kViewThreads * kViewMaxWaves) void k_view_sync(const uint16_t* info, int64_t tile0,
                                                                          int64_t v_begin, int64_t v_end,
                                                                          RankPtrs P, int n_rt, float scale) {
  __shared__ uint16_t info_of[kViewThreads];
  view_tile<DT, NR, NTL>(tile0 + blockIdx.x, info, v_begin, v_end, view_stage<NR>(), info_of, P,
                         NR > 0 ? NR : n_rt, scale);
}

// A grid of at most max_blocks blocks, each looping over tiles: the narrow
// launches of syncs that overlap backward.
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kViewThreads * kViewMaxWaves) void k_view_sync_strided(
    const uint16_t* info, int64_t tile0, int64_t n_tiles, int64_t v_begin, int64_t v_end, RankPtrs P, int n_rt,
    float scale) {
  __shared__ uint16_t info_of[kViewThreads];
  u32x4* stage = view_stage<NR>();
  for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    view_tile<DT, NR, NTL>(tile0 + t, info, v_begin, v_end, stage, info_of, P, NR > 0 ? NR : n_rt, scale);
    __syncthreads();  // the stage is refilled by the block's next tile
  }
}

struct ViewSpan {
  const uint16_t* info;
  int64_t tile0, n_tiles, v_begin, v_end;
};

template <int DT, int NR, bool NTL>
void launch_view_n(const ViewSpan& sp, const RankPtrs& P, int n, float scale, int64_t max_blocks, hipStream_t s) {
  const dim3 b(kViewThreads * (NR > 0 ? NR : kViewMaxWaves));
  const size_t lds = NR > 0 ? 0 : size_t(n) * kViewThreads * sizeof(u32x4);
  if (max_blocks > 0 && max_blocks < sp.n_tiles) {
    hipLaunchKernelGGL((k_view_sync_strided<DT, NR, NTL>), dim3(unsigned(max_blocks)), b, lds, s, sp.info, sp.tile0,
                       sp.n_tiles, sp.v_begin, sp.v_end, P, n, scale);
    return;
  }
  for (int64_t t = 0; t < sp.n_tiles; t += kMaxGrid)
    hipLaunchKernelGGL((k_view_sync<DT, NR, NTL>), dim3(unsigned(std::min(sp.n_tiles - t, kMaxGrid))), b, lds, s,
                       sp.info, sp.tile0 + t, sp.v_begin, sp.v_end, P, n, scale);
}

template <int DT, bool NTL>
void launch_view(const ViewSpan& sp, const RankPtrs& P, int n, float scale, int64_t max_blocks, hipStream_t s) {
  switch (n) {
    case 1: launch_view_n<DT, 1, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 2: launch_view_n<DT, 2, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 3: launch_view_n<DT, 3, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 4: launch_view_n<DT, 4, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 5: launch_view_n<DT, 5, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 6: launch_view_n<DT, 6, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 7: launch_view_n<DT, 7, NTL>(sp, P, n, scale, max_blocks, s); break;
    case 8: launch_view_n<DT, 8, NTL>(sp, P, n, scale, max_blocks, s); break;
    default: launch_view_n<DT, 0, NTL>(sp, P, n, scale, max_blocks, s);
  }
}

// The kernels for the plan's dtypes (a compressed plan's arithmetic goes
// through bf16), with non-temporal loads when the ranks' arenas together
// exceed the Infinity Cache: buckets are reduced one after the other over
// the whole arena, so the arena's size, not one bucket's, decides whether
// loads can hit the cache.
void launch_view_plan(const ddp_plan* plan, const ViewSpan& sp, const RankPtrs& P, int N, float scale,
                      int64_t max_blocks, hipStream_t s) {
  const bool ntl = int64_t(N) * plan->arena_numel * elem_bytes(plan->dtype) > kInfinityCacheBytes;
  if (plan->dtype != plan->comm_dtype) {
    if (ntl) launch_view<kF32ViaBf16, true>(sp, P, N, scale, max_blocks, s);
    else launch_view<kF32ViaBf16, false>(sp, P, N, scale, max_blocks, s);
  } else if (plan->dtype == DDP_FP32) {
    if (ntl) launch_view<DDP_FP32, true>(sp, P, N, scale, max_blocks, s);
    else launch_view<DDP_FP32, false>(sp, P, N, scale, max_blocks, s);
  } else {
    if (ntl) launch_view<DDP_BF16, true>(sp, P, N, scale, max_blocks, s);
    else launch_view<DDP_BF16, false>(sp, P, N, scale, max_blocks, s);
  }
}

}  // namespace
}  // namespace ddp

using namespace ddp;

namespace ddp {

int launch_view_bucket(const ddp_plan* plan, int32_t b, const RankPtrs& P, int32_t N, float scale,
                       int64_t max_blocks, hipStream_t s) {
  const Bucket& bk = plan->buckets[b];
  if (bk.n_view_tiles == 0) return DDP_OK;
  const uint16_t* info = nullptr;
  int st = device_tables(const_cast<ddp_plan*>(plan), nullptr, &info);
  if (st != DDP_OK) return st;
  const ViewSpan sp{info, bk.view_vec_begin / kViewThreads, bk.n_view_tiles, bk.view_vec_begin, bk.view_vec_end};
  launch_view_plan(plan, sp, P, N, scale, max_blocks, s);
  DDP_HIP_TRY(hipGetLastError(), "bucket_allreduce_view: launch");
  return DDP_OK;
}

int launch_view_arena(const ddp_plan* plan, const RankPtrs& P, int32_t N, float scale, hipStream_t s) {
  const int64_t vecs = int64_t(plan->vec_info.size());
  if (vecs == 0) return DDP_OK;
  const uint16_t* info = nullptr;
  int st = device_tables(const_cast<ddp_plan*>(plan), nullptr, &info);
  if (st != DDP_OK) return st;
  const ViewSpan sp{info, 0, (vecs + kViewThreads - 1) / kViewThreads, 0, vecs};
  launch_view_plan(plan, sp, P, N, scale, 0, s);
  DDP_HIP_TRY(hipGetLastError(), "ddp_sync: launch");
  return DDP_OK;
}

int check_view_arenas(const ddp_plan* plan, void* const* grad_arenas, int32_t N, const char* fn) {
  const int eb = elem_bytes(plan->dtype);
  return check_rank_buffers(grad_arenas, N, plan->arena_numel * eb, 16, fn, "grad_arenas");
}

}  // namespace ddp

extern "C" int bucket_allreduce_view(const ddp_plan* plan, int32_t b, void* const* grad_arenas, int32_t N,
                                     float scale, void* stream) {
  const char* fn = "bucket_allreduce_view";
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (b < 0 || b >= int32_t(plan->buckets.size()))
    return fail(DDP_EINVAL, std::string(fn) + ": bucket index out of range");
  if (N != plan->world_size) return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  int st = check_view_arenas(plan, grad_arenas, N, fn);
  if (st != DDP_OK) return st;
  RankPtrs P{};
  for (int r = 0; r < N; ++r) P.p[r] = grad_arenas[r];
  return launch_view_bucket(plan, b, P, N, scale, 0, as_stream(stream));
}
