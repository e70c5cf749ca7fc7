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
// The plan cuts each member at the bucket's chunk boundaries ("pieces"), so
// every tile has one ring order, uniform across its block; a block finds its
// piece by a uniform binary search over the tile prefix sums. Launch shape
// as for the fused all-reduce: one wave per block, one 16-byte vector per
// thread, non-temporal stores, non-temporal loads when the ranks' arenas
// together exceed the Infinity Cache.
#include <algorithm>

#include "ring_common.h"

namespace ddp {
namespace {

constexpr int64_t kViewCacheResidentBytes = int64_t(256) << 20;
constexpr int kViewBatch = 16;  // ranks loaded together when N > 8

__device__ __forceinline__ int find_piece(const Piece* pieces, int n, int64_t tile) {
  int lo = 0, hi = n - 1;  // last piece whose tile_begin <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pieces[mid].tile_begin <= tile) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// NR > 0: compile-time rank count; NR == 0: any N, loaded kViewBatch at a time.
template <int DT, int NR, bool NTL>
__global__ __launch_bounds__(kViewThreads) void k_view_sync(const Piece* pieces, int n_pieces, int64_t n_tiles,
                                                            RankPtrs P, int n_rt, float scale) {
  using O = Ops<DT>;
  constexpr int V = O::V;
  const int n = NR > 0 ? NR : n_rt;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
    const Piece pc = pieces[find_piece(pieces, n_pieces, tile)];
    // Tiles sit on a grid aligned to whole tiles of the arena (1 KiB per wave
    // for fp32), so every wave touches whole cache lines.
    constexpr int64_t kTile = int64_t(kViewThreads) * V;
    const int64_t at = (pc.src_off / kTile + (tile - pc.tile_begin)) * kTile + int64_t(threadIdx.x) * V;
    const int64_t end = pc.src_off + pc.numel;
    if (at < pc.src_off || at >= end) continue;
    const int first = wrap(pc.chunk + 1, n);
    if (at + V <= end) {
      const int64_t vi = at / V;
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
        for (int k = 1; k < n; k += kViewBatch) {
          u32x4 x[kViewBatch];
#pragma unroll
          for (int j = 0; j < kViewBatch; ++j)
            if (k + j < n) x[j] = ld16<NTL>(static_cast<const u32x4*>(P.p[wrap(first + k + j, n)]) + vi);
#pragma unroll
          for (int j = 0; j < kViewBatch; ++j)
            if (k + j < n) O::add(a, x[j]);
        }
      }
      const u32x4 y = O::scale(O::to(a), scale);
      for (int r = 0; r < n; ++r) st16<true>(static_cast<u32x4*>(P.p[r]) + vi, y);
    } else {
      // The last, partial vector of a member: element by element.
      for (int64_t i = at; i < end; ++i) {
        float acc = O::load1(P.p[first], i);
        for (int k = 1; k < n; ++k) acc = O::add1(acc, O::load1(P.p[wrap(first + k, n)], i));
        acc = O::mul1(acc, scale);
        for (int r = 0; r < n; ++r) O::store1(P.p[r], i, acc);
      }
    }
  }
}

template <int DT, bool NTL>
void launch_view(const Piece* pieces, int n_pieces, int64_t n_tiles, const RankPtrs& P, int n, float scale,
                 hipStream_t s) {
  const dim3 g(grid_for(n_tiles)), b(kViewThreads);
  switch (n) {
#define DDP_VIEW_CASE(NR)                                                                               \
  case NR:                                                                                              \
    hipLaunchKernelGGL((k_view_sync<DT, NR, NTL>), g, b, 0, s, pieces, n_pieces, n_tiles, P, n, scale); \
    break;
    DDP_VIEW_CASE(1)
    DDP_VIEW_CASE(2)
    DDP_VIEW_CASE(3)
    DDP_VIEW_CASE(4)
    DDP_VIEW_CASE(5)
    DDP_VIEW_CASE(6)
    DDP_VIEW_CASE(7)
    DDP_VIEW_CASE(8)
#undef DDP_VIEW_CASE
    default:
      hipLaunchKernelGGL((k_view_sync<DT, 0, NTL>), g, b, 0, s, pieces, n_pieces, n_tiles, P, n, scale);
  }
}

}  // namespace
}  // namespace ddp

using namespace ddp;

extern "C" int bucket_allreduce_view(const ddp_plan* plan, int32_t b, void* const* grad_arenas, int32_t N,
                                     float scale, void* stream) {
  const char* fn = "bucket_allreduce_view";
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (b < 0 || b >= int32_t(plan->buckets.size()))
    return fail(DDP_EINVAL, std::string(fn) + ": bucket index out of range");
  if (N != plan->world_size) return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  if (plan->comm_dtype != plan->dtype)
    return fail(DDP_EINVAL, std::string(fn) + ": the in-place sync needs buckets of the gradients' dtype");
  const int eb = elem_bytes(plan->dtype);
  int st = check_rank_buffers(grad_arenas, N, plan->arena_numel * eb, 16, fn, "grad_arenas");
  if (st != DDP_OK) return st;
  const Bucket& bk = plan->buckets[b];
  if (bk.n_view_tiles == 0) return DDP_OK;
  const Piece* pieces = nullptr;
  st = device_tables(const_cast<ddp_plan*>(plan), nullptr, &pieces);
  if (st != DDP_OK) return st;
  RankPtrs P{};
  for (int r = 0; r < N; ++r) P.p[r] = grad_arenas[r];
  hipStream_t s = as_stream(stream);
  // Buckets are reduced one after the other over the whole arena, so the
  // arena's size, not one bucket's, decides whether loads can hit the cache.
  const bool ntl = int64_t(N) * plan->arena_numel * eb > kViewCacheResidentBytes;
  const Piece* pb = pieces + bk.piece_begin;
  const int np = int(bk.n_pieces);
  if (plan->dtype == DDP_FP32) {
    if (ntl) launch_view<DDP_FP32, true>(pb, np, bk.n_view_tiles, P, N, scale, s);
    else launch_view<DDP_FP32, false>(pb, np, bk.n_view_tiles, P, N, scale, s);
  } else {
    if (ntl) launch_view<DDP_BF16, true>(pb, np, bk.n_view_tiles, P, N, scale, s);
    else launch_view<DDP_BF16, false>(pb, np, bk.n_view_tiles, P, N, scale, s);
  }
  DDP_HIP_TRY(hipGetLastError(), "bucket_allreduce_view: launch");
  return DDP_OK;
}
