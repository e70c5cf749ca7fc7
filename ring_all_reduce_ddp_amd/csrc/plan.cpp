// Host bucket planner: reverse-order assignment of gradients to flat buckets.
//
// Follows page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03, parts
// "Bucket" and "Overlap": small gradients are packed into one flat buffer per
// collective; buckets are filled in the reverse of the parameters'
// registration order (an approximation of the order backward produces them);
// regular buckets hold up to 25 MiB and the first up to 1 MiB; every rank uses
// the same assignment and order. Page "Day 17 数据并行 DP/DDP"
// (blog.ans20xx.com), part "bucket 与 overlap", names the capacity an upper
// limit: a tensor that would pass the capacity opens a new bucket, and one
// larger than the capacity sits alone in its bucket.
#include <algorithm>
#include <new>
#include <string>

#include "ddp_internal.h"

namespace ddp {

namespace {
thread_local std::string t_last_error;
}

int fail(int status, const std::string& msg) {
  t_last_error = msg;
  return status;
}

void clear_error() { t_last_error.clear(); }

const char* last_error() { return t_last_error.c_str(); }

}  // namespace ddp

using namespace ddp;

extern "C" const char* ddp_last_error(void) { return ddp::last_error(); }

extern "C" int ddp_bucket_plan(const int64_t* param_numels, int32_t n_params, int32_t dtype,
                               int64_t cap_bytes, int64_t first_bucket_bytes,
                               int32_t world_size, ddp_plan** out) {
  return ddp_bucket_plan_ex(param_numels, n_params, dtype, dtype, cap_bytes, first_bucket_bytes, world_size,
                            out);
}

// grad_dtype: the gradients (arena layout; capacities count their bytes).
// comm_dtype: the buckets (member alignment and padding in its 16-byte
// vectors). fp32 gradients with bf16 buckets is the bf16 compression hook.
extern "C" int ddp_bucket_plan_ex(const int64_t* param_numels, int32_t n_params, int32_t grad_dtype,
                                  int32_t comm_dtype, int64_t cap_bytes, int64_t first_bucket_bytes,
                                  int32_t world_size, ddp_plan** out) {
  if (out == nullptr) return fail(DDP_EINVAL, "ddp_bucket_plan: out is NULL");
  *out = nullptr;
  if (n_params < 0) return fail(DDP_EINVAL, "ddp_bucket_plan: n_params < 0");
  if (n_params > 0 && param_numels == nullptr)
    return fail(DDP_EINVAL, "ddp_bucket_plan: param_numels is NULL");
  if (!valid_dtype(grad_dtype) || !valid_dtype(comm_dtype))
    return fail(DDP_EINVAL, "ddp_bucket_plan: unknown dtype");
  if (grad_dtype != comm_dtype && !(grad_dtype == DDP_FP32 && comm_dtype == DDP_BF16))
    return fail(DDP_EINVAL, "ddp_bucket_plan: the only mixed pair is fp32 gradients in bf16 buckets");
  if (cap_bytes <= 0 || first_bucket_bytes <= 0)
    return fail(DDP_EINVAL, "ddp_bucket_plan: capacities must be positive");
  if (world_size < 1 || world_size > DDP_MAX_RANKS)
    return fail(DDP_EINVAL, "ddp_bucket_plan: world_size must lie in [1, 64]");
  const int64_t e = elem_bytes(grad_dtype);                 // capacity unit
  const int64_t va = kVectorBytes / e;                       // arena alignment
  const int64_t v = kVectorBytes / elem_bytes(comm_dtype);   // bucket alignment
  // Keep every size well inside int64 when multiplied by element sizes.
  const int64_t kMaxNumel = int64_t(1) << 50;
  for (int32_t p = 0; p < n_params; ++p) {
    if (param_numels[p] < 0 || param_numels[p] > kMaxNumel)
      return fail(DDP_EINVAL, "ddp_bucket_plan: parameter " + std::to_string(p) +
                                  " has a negative or oversized element count");
  }

  ddp_plan* plan = new (std::nothrow) ddp_plan();
  if (plan == nullptr) return fail(DDP_ENOMEM, "ddp_bucket_plan: out of host memory");
  try {
    plan->dtype = grad_dtype;
    plan->comm_dtype = comm_dtype;
    plan->world_size = world_size;
    plan->cap_bytes = cap_bytes;
    plan->first_bucket_bytes = first_bucket_bytes;
    plan->numels.assign(param_numels, param_numels + n_params);
    plan->tile_elems = pack_tile_elems(comm_dtype);

    // Gradient arena: registration order, each parameter on a 16-byte boundary.
    plan->arena_offsets.resize(n_params);
    int64_t pos = 0;
    for (int32_t p = 0; p < n_params; ++p) {
      plan->arena_offsets[p] = pos;
      pos += round_up(param_numels[p], va);
    }
    plan->arena_numel = pos;
    plan->vec_info.assign(pos / va, kVecSlack);

    // Buckets: reverse registration order.
    Bucket open;
    int64_t used = 0;  // elements used by the open bucket (multiple of v)
    auto close = [&]() {
      open.padded_numel = round_up(used, int64_t(world_size) * v);
      plan->buckets.push_back(std::move(open));
      open = Bucket();
      used = 0;
    };
    for (int32_t p = n_params - 1; p >= 0; --p) {
      const int64_t slot = round_up(param_numels[p], v);
      const int64_t capacity = plan->buckets.empty() ? first_bucket_bytes : cap_bytes;
      if (!open.members.empty() && (used + slot) * e > capacity) close();
      open.members.push_back(Member{p, used, param_numels[p]});
      used += slot;
    }
    if (!open.members.empty()) close();

    // Segments and pack tiles of every bucket.
    for (Bucket& b : plan->buckets) {
      b.seg_begin = int64_t(plan->segments.size());
      int64_t tiles = 0;
      int64_t end = 0;
      for (const Member& m : b.members) {
        Segment s;
        s.dst_off = m.offset;
        s.src_off = plan->arena_offsets[m.param];
        s.numel = m.numel;
        s.slot = round_up(m.numel, v);
        s.tile_begin = tiles;
        tiles += (s.slot + plan->tile_elems - 1) / plan->tile_elems;
        end = m.offset + s.slot;
        plan->segments.push_back(s);
      }
      if (b.padded_numel > end) {
        Segment s;
        s.dst_off = end;
        s.src_off = 0;
        s.numel = 0;
        s.slot = b.padded_numel - end;
        s.tile_begin = tiles;
        tiles += (s.slot + plan->tile_elems - 1) / plan->tile_elems;
        plan->segments.push_back(s);
      }
      b.n_segs = int64_t(plan->segments.size()) - b.seg_begin;
      b.n_tiles = tiles;
      // Each pack tile's segment, so a block finds it with one load.
      b.tile_seg_begin = int64_t(plan->tile_seg.size());
      for (int64_t i = 0; i < b.n_segs; ++i) {
        const Segment& sg = plan->segments[size_t(b.seg_begin + i)];
        const int64_t nt = (sg.slot + plan->tile_elems - 1) / plan->tile_elems;
        plan->tile_seg.insert(plan->tile_seg.end(), size_t(nt), int32_t(i));
      }
      if (int64_t(plan->tile_seg.size()) - b.tile_seg_begin != b.n_tiles) {
        delete plan;
        return fail(DDP_EINVAL, "ddp_bucket_plan: internal error: tile table does not match the bucket's tiles");
      }

      for (const Member& m : b.members) b.data_numel += m.numel;
      // The in-place sync: the bucket's members are a run of consecutive
      // parameters, so they span one stretch of the arena. Each arena vector
      // lies in one ring chunk: arena offsets are multiples of va, bucket
      // offsets and the chunk length L multiples of v, and va <= v (with
      // bf16 buckets, an fp32 arena vector of 4 elements sits inside one
      // 8-element bucket vector).
      if (!b.members.empty()) {
        const Member& last = b.members.back();    // lowest parameter index
        const Member& first = b.members.front();  // highest
        b.view_vec_begin = plan->arena_offsets[last.param] / va;
        b.view_vec_end = (plan->arena_offsets[first.param] + round_up(first.numel, va)) / va;
        b.n_view_tiles = (b.view_vec_end + kViewThreads - 1) / kViewThreads - b.view_vec_begin / kViewThreads;
        const int64_t L = b.padded_numel / world_size;
        for (const Member& m : b.members) {
          const int64_t a0 = plan->arena_offsets[m.param];
          for (int64_t e = 0; e < m.numel; e += va)
            plan->vec_info[(a0 + e) / va] = make_vec_info((m.offset + e) / L, std::min<int64_t>(va, m.numel - e));
        }
      }
    }
  } catch (const std::bad_alloc&) {
    delete plan;
    return fail(DDP_ENOMEM, "ddp_bucket_plan: out of host memory");
  }
  *out = plan;
  return DDP_OK;
}

extern "C" void ddp_plan_free(ddp_plan* plan) {
  if (plan == nullptr) return;
  release_device_tables(plan);
  delete plan;
}

extern "C" int ddp_plan_num_buckets(const ddp_plan* plan, int32_t* out) {
  if (plan == nullptr || out == nullptr) return fail(DDP_EINVAL, "ddp_plan_num_buckets: NULL argument");
  *out = int32_t(plan->buckets.size());
  return DDP_OK;
}

extern "C" int ddp_plan_bucket(const ddp_plan* plan, int32_t b, int64_t* padded_numel,
                               int32_t* n_members) {
  if (plan == nullptr) return fail(DDP_EINVAL, "ddp_plan_bucket: plan is NULL");
  if (b < 0 || b >= int32_t(plan->buckets.size()))
    return fail(DDP_EINVAL, "ddp_plan_bucket: bucket index out of range");
  if (padded_numel) *padded_numel = plan->buckets[b].padded_numel;
  if (n_members) *n_members = int32_t(plan->buckets[b].members.size());
  return DDP_OK;
}

extern "C" int ddp_plan_member(const ddp_plan* plan, int32_t b, int32_t i, int32_t* param_idx,
                               int64_t* offset, int64_t* numel) {
  if (plan == nullptr) return fail(DDP_EINVAL, "ddp_plan_member: plan is NULL");
  if (b < 0 || b >= int32_t(plan->buckets.size()))
    return fail(DDP_EINVAL, "ddp_plan_member: bucket index out of range");
  const Bucket& bk = plan->buckets[b];
  if (i < 0 || i >= int32_t(bk.members.size()))
    return fail(DDP_EINVAL, "ddp_plan_member: member index out of range");
  if (param_idx) *param_idx = bk.members[i].param;
  if (offset) *offset = bk.members[i].offset;
  if (numel) *numel = bk.members[i].numel;
  return DDP_OK;
}

extern "C" int ddp_plan_arena_map(const ddp_plan* plan, uint16_t* out, int64_t n) {
  if (plan == nullptr || (out == nullptr && n > 0)) return fail(DDP_EINVAL, "ddp_plan_arena_map: NULL argument");
  if (n != int64_t(plan->vec_info.size()))
    return fail(DDP_EINVAL, "ddp_plan_arena_map: n must be the arena's vector count (" +
                                std::to_string(plan->vec_info.size()) + ")");
  std::copy(plan->vec_info.begin(), plan->vec_info.end(), out);
  return DDP_OK;
}

extern "C" int ddp_plan_grad_arena(const ddp_plan* plan, int64_t* arena_numel,
                                   int64_t* param_offsets) {
  if (plan == nullptr || arena_numel == nullptr)
    return fail(DDP_EINVAL, "ddp_plan_grad_arena: NULL argument");
  *arena_numel = plan->arena_numel;
  if (param_offsets) {
    for (size_t p = 0; p < plan->arena_offsets.size(); ++p) param_offsets[p] = plan->arena_offsets[p];
  }
  return DDP_OK;
}
