// Internal declarations shared by the host planner and the HIP launchers.
#pragma once

#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "ddp_ring.h"

namespace ddp {

constexpr int kVectorBytes = 16;
// MI355X's Infinity Cache (the memory-side last-level cache). Kernels whose
// buffers together exceed it stream them with non-temporal loads and stores;
// below it they use cached accesses, so data written by one kernel is read
// from the cache by the next.
constexpr int64_t kInfinityCacheBytes = int64_t(256) << 20;

inline int elem_bytes(int32_t dtype) { return dtype == DDP_BF16 ? 2 : 4; }
inline bool valid_dtype(int32_t dtype) { return dtype == DDP_FP32 || dtype == DDP_BF16; }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Records `msg` as the calling thread's last error and returns `status`.
int fail(int status, const std::string& msg);
void clear_error();

// One contiguous piece of a bucket: a member's slot (numel elements copied,
// the rest of the slot zero) or the tail padding (numel == 0).
struct Segment {
  int64_t dst_off;     // offset in the bucket, elements (multiple of V)
  int64_t src_off;     // offset in the gradient arena, elements (multiple of V)
  int64_t numel;       // elements that come from the gradient
  int64_t slot;        // elements of the bucket covered (multiple of V)
  int64_t tile_begin;  // first pack tile of this segment (prefix sum)
};

// The in-place sync's map of the gradient arena: one entry per 16-byte
// vector, kVecSlack for vectors that hold no member element (the padding
// between members), else the ring chunk of the vector's bucket that holds it
// (low byte) and how many of its elements belong to the member (high byte,
// 1..V; fewer than V only for a member's last vector). A vector never spans
// two chunks: chunk boundaries and member offsets are multiples of V.
constexpr uint16_t kVecSlack = 0xffff;
inline uint16_t make_vec_info(int64_t chunk, int64_t valid) { return uint16_t(chunk | (valid << 8)); }

struct Member {
  int32_t param;
  int64_t offset;
  int64_t numel;
};

struct Bucket {
  std::vector<Member> members;
  int64_t padded_numel = 0;
  int64_t seg_begin = 0;   // index of its first segment in plan.segments
  int64_t n_segs = 0;
  int64_t n_tiles = 0;     // pack/unpack tiles per rank
  int64_t tile_seg_begin = 0;  // index of its first tile in plan.tile_seg
  int64_t view_vec_begin = 0;  // the bucket's members span arena vectors
  int64_t view_vec_end = 0;    // [view_vec_begin, view_vec_end) (in-place sync)
  int64_t n_view_tiles = 0;    // view tiles covering that span
  int64_t data_numel = 0;  // sum of its members' element counts
};

constexpr int kMaxDevices = 64;

struct DeviceTable {
  Segment* segs = nullptr;       // device copy of plan.segments
  int32_t* tile_seg = nullptr;   // device copy of plan.tile_seg (same allocation)
  uint16_t* vec_info = nullptr;  // device copy of plan.vec_info (same allocation)
};

}  // namespace ddp

struct ddp_plan {
  int32_t dtype = DDP_FP32;             // the gradients' dtype (arena layout)
  int32_t comm_dtype = DDP_FP32;        // the buckets' dtype (bucket layout, ring)
  int32_t world_size = 1;
  int64_t cap_bytes = 0;
  int64_t first_bucket_bytes = 0;
  std::vector<int64_t> numels;          // registration order
  std::vector<int64_t> arena_offsets;   // registration order, elements
  int64_t arena_numel = 0;
  std::vector<ddp::Bucket> buckets;
  std::vector<ddp::Segment> segments;   // all buckets' segments, bucket-major
  std::vector<int32_t> tile_seg;        // per pack/unpack tile: its segment, counted from the bucket's first
  std::vector<uint16_t> vec_info;       // per arena vector (in-place sync; same dtypes only)
  int64_t tile_elems = 0;               // elements per pack tile (bucket vectors)
  std::mutex mu;                        // guards `device`
  ddp::DeviceTable device[ddp::kMaxDevices];
};

namespace ddp {
// Elements covered by one pack/unpack tile, in vectors of the bucket's dtype
// (16 bytes of it); fixed when the plan is built so the tile prefix sums in
// the segments match the kernels.
constexpr int kPackThreads = 256;
constexpr int kPackVecsPerThread = 4;
inline int64_t pack_tile_elems(int32_t comm_dtype) {
  return int64_t(kPackThreads) * kPackVecsPerThread * (kVectorBytes / elem_bytes(comm_dtype));
}
// Arena vectors covered by one tile of the in-place sync (one per lane of a wave).
constexpr int kViewThreads = 64;
// Device copies of the plan's segment table, tile-to-segment table and arena
// vector map on the current device, made on first use (defined with the HIP
// code). Any output pointer may be NULL.
int device_tables(ddp_plan* plan, const Segment** segs, const uint16_t** vec_info,
                  const int32_t** tile_seg = nullptr);
// Releases the device tables of a plan (defined with the HIP code).
void release_device_tables(ddp_plan* plan);
}  // namespace ddp
