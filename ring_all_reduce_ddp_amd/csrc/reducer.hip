// Reducer: starts each bucket's sync as soon as all of its gradients are
// ready, on a communication stream, so it overlaps the rest of backward.
//
// Page "DDP 与 Ring All-Reduce" (blog.vllbc.top), section 03, part "Overlap"
// and section 05 step 2: every gradient accumulator has a hook; when the hook
// of a bucket's last gradient fires, that bucket's all-reduce is launched
// asynchronously, overlapping the backward computation of earlier layers; all
// processes use the same bucket order, and bucket i+1 is never launched
// before bucket i. Page "Day 17 数据并行 DP/DDP" (blog.ans20xx.com), parts
// "梯度同步时机" and "源码阅读路线": mark the parameter ready, launch the
// bucket's all-reduce when all are ready; at the end of backward wait for
// every bucket, divide by the world size and copy back. Section 05 step 5 of
// the first page: all buckets must finish before the optimizer reads the
// gradients.
//
// Host side only: events order the streams; the syncs themselves are the
// library's kernels (bucket_allreduce_view, or pack + all-reduce + unpack).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "hip_common.h"

struct ddp_reducer {
  const ddp_plan* plan = nullptr;
  int32_t n = 0;
  int32_t variant = DDP_VARIANT_VIEW;
  float scale = 1.0f;
  int64_t comm_max_blocks = 0;          // width of the in-place syncs launched during backward
  hipStream_t comm = nullptr;
  std::vector<void*> arenas;            // N
  ddp::RankPtrs arena_ptrs{};           // the same, checked once at creation (in-place variant)
  std::vector<void*> bucket_bufs;       // B*N, empty for the in-place variant
  std::vector<int32_t> bucket_of;       // parameter -> bucket
  std::vector<int32_t> pending;         // per bucket: gradients not yet ready
  std::vector<hipEvent_t> ready_event;  // per bucket: recorded when it became ready
  std::vector<char> marked;             // per parameter
  int32_t next = 0;                     // next bucket to launch (launch order = plan order)
  hipEvent_t done = nullptr;
};

namespace {

using ddp::fail;

int hip_err(hipError_t e, const std::string& where) {
  return fail(DDP_EHIP, where + ": " + hipGetErrorString(e));
}

int launch_bucket(ddp_reducer* r, int32_t b) {
  const ddp_plan* plan = r->plan;
  void* s = r->comm;
  if (r->variant == DDP_VARIANT_VIEW) {
    // Buckets before the last one run while backward still computes: at most
    // comm_max_blocks blocks then, so the sync leaves most compute units to
    // the backward kernels. The last bucket is ready only when backward has
    // produced every gradient, so it takes the whole device.
    const bool last = b + 1 == int32_t(plan->buckets.size());
    return ddp::launch_view_bucket(plan, b, r->arena_ptrs, r->n, r->scale, last ? 0 : r->comm_max_blocks, r->comm);
  }
  void* const* bufs = r->bucket_bufs.data() + size_t(b) * r->n;
  const int64_t count = plan->buckets[b].padded_numel;
  if (r->variant == DDP_VARIANT_PERSISTENT)  // a time-out leaves the gradients unchanged
    return ddp::sync_bucket_persistent(plan, b, r->arenas.data(), bufs, r->n, r->scale, r->comm);
  int st = bucket_pack(plan, b, const_cast<const void* const*>(r->arenas.data()), bufs, r->n, s);
  if (st != DDP_OK) return st;
  if (r->variant == DDP_VARIANT_FUSED) {
    st = ring_allreduce_fused(bufs, r->n, count, plan->comm_dtype, s);
  } else {
    for (int ph = DDP_RS; ph <= DDP_AG && st == DDP_OK; ++ph)
      for (int k = 0; k + 1 < r->n && st == DDP_OK; ++k)
        st = ring_allreduce_step(bufs, r->n, count, plan->comm_dtype, k, ph, s);
  }
  if (st != DDP_OK) return st;
  return bucket_unpack_scale(plan, b, const_cast<const void* const*>(bufs), r->arenas.data(), r->n, r->scale, s);
}

}  // namespace

extern "C" int ddp_reducer_create(const ddp_plan* plan, void* const* grad_arenas, void* const* bucket_bufs,
                                  int32_t N, int32_t variant, float scale, int64_t comm_max_blocks,
                                  void* comm_stream, ddp_reducer** out) {
  const char* fn = "ddp_reducer_create";
  if (out == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": out is NULL");
  *out = nullptr;
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (N != plan->world_size) return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  if (variant != DDP_VARIANT_FUSED && variant != DDP_VARIANT_STEPS && variant != DDP_VARIANT_PERSISTENT &&
      variant != DDP_VARIANT_VIEW)
    return fail(DDP_EINVAL, std::string(fn) + ": unknown variant");
  if (grad_arenas == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": grad_arenas is NULL");
  if (variant != DDP_VARIANT_VIEW && bucket_bufs == nullptr)
    return fail(DDP_EINVAL, std::string(fn) + ": bucket_bufs is NULL");
  if (comm_max_blocks < 0) return fail(DDP_EINVAL, std::string(fn) + ": comm_max_blocks < 0");
  if (comm_max_blocks > 0 && variant != DDP_VARIANT_VIEW)
    return fail(DDP_EINVAL, std::string(fn) + ": comm_max_blocks applies to the in-place variant only");
  if (variant == DDP_VARIANT_VIEW) {
    // Checked once here: the reducer's launches skip the per-call checks, so
    // the arenas must stay allocated while the reducer exists.
    int st = ddp::check_view_arenas(plan, grad_arenas, N, fn);
    if (st != DDP_OK) return st;
  }
  ddp_reducer* r = new (std::nothrow) ddp_reducer();
  if (r == nullptr) return fail(DDP_ENOMEM, std::string(fn) + ": out of host memory");
  try {
    const int32_t B = int32_t(plan->buckets.size());
    r->plan = plan;
    r->n = N;
    r->variant = variant;
    r->scale = scale;
    r->comm_max_blocks = comm_max_blocks;
    r->comm = reinterpret_cast<hipStream_t>(comm_stream);
    r->arenas.assign(grad_arenas, grad_arenas + N);
    for (int32_t i = 0; i < N; ++i) r->arena_ptrs.p[i] = grad_arenas[i];
    if (variant != DDP_VARIANT_VIEW) r->bucket_bufs.assign(bucket_bufs, bucket_bufs + size_t(B) * N);
    r->bucket_of.assign(plan->numels.size(), -1);
    r->pending.assign(B, 0);
    for (int32_t b = 0; b < B; ++b)
      for (const ddp::Member& m : plan->buckets[b].members) {
        r->bucket_of[m.param] = b;
        ++r->pending[b];
      }
    r->marked.assign(plan->numels.size(), 0);
    r->ready_event.assign(B, nullptr);
    for (int32_t b = 0; b < B; ++b) {
      hipError_t e = hipEventCreateWithFlags(&r->ready_event[b], hipEventDisableTiming);
      if (e != hipSuccess) {
        ddp_reducer_free(r);
        return hip_err(e, std::string(fn) + ": hipEventCreateWithFlags");
      }
    }
    hipError_t e = hipEventCreateWithFlags(&r->done, hipEventDisableTiming);
    if (e != hipSuccess) {
      ddp_reducer_free(r);
      return hip_err(e, std::string(fn) + ": hipEventCreateWithFlags");
    }
  } catch (const std::bad_alloc&) {
    ddp_reducer_free(r);
    return fail(DDP_ENOMEM, std::string(fn) + ": out of host memory");
  }
  *out = r;
  return DDP_OK;
}

extern "C" void ddp_reducer_free(ddp_reducer* r) {
  if (r == nullptr) return;
  for (hipEvent_t e : r->ready_event)
    if (e != nullptr) (void)hipEventDestroy(e);
  if (r->done != nullptr) (void)hipEventDestroy(r->done);
  delete r;
}

extern "C" int ddp_reducer_prepare(ddp_reducer* r) {
  if (r == nullptr) return fail(DDP_EINVAL, "ddp_reducer_prepare: reducer is NULL");
  const int32_t B = int32_t(r->plan->buckets.size());
  for (int32_t b = 0; b < B; ++b) r->pending[b] = int32_t(r->plan->buckets[b].members.size());
  std::fill(r->marked.begin(), r->marked.end(), 0);
  r->next = 0;
  return DDP_OK;
}

extern "C" int ddp_reducer_mark_ready(ddp_reducer* r, int32_t param, void* producer_stream) {
  const char* fn = "ddp_reducer_mark_ready";
  if (r == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": reducer is NULL");
  if (param < 0 || param >= int32_t(r->marked.size()))
    return fail(DDP_EINVAL, std::string(fn) + ": parameter index out of range");
  if (r->marked[param]) return fail(DDP_EINVAL, std::string(fn) + ": parameter " + std::to_string(param) +
                                                    " marked ready twice in one backward pass");
  r->marked[param] = 1;
  const int32_t b = r->bucket_of[param];
  if (--r->pending[b] > 0) return DDP_OK;
  // The bucket's last gradient: everything that produced it is already on the
  // producer stream, so an event recorded now gates the bucket's sync.
  hipError_t e = hipEventRecord(r->ready_event[b], reinterpret_cast<hipStream_t>(producer_stream));
  if (e != hipSuccess) return hip_err(e, std::string(fn) + ": hipEventRecord");
  // Launch in plan order: bucket i+1 never before bucket i.
  const int32_t B = int32_t(r->plan->buckets.size());
  while (r->next < B && r->pending[r->next] == 0) {
    e = hipStreamWaitEvent(r->comm, r->ready_event[r->next], 0);
    if (e != hipSuccess) return hip_err(e, std::string(fn) + ": hipStreamWaitEvent");
    int st = launch_bucket(r, r->next);
    if (st != DDP_OK) return st;
    ++r->next;
  }
  return DDP_OK;
}

extern "C" int ddp_reducer_finalize(ddp_reducer* r, void* stream) {
  const char* fn = "ddp_reducer_finalize";
  if (r == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": reducer is NULL");
  const int32_t B = int32_t(r->plan->buckets.size());
  if (r->next < B) {
    for (size_t p = 0; p < r->marked.size(); ++p)
      if (!r->marked[p])
        return fail(DDP_EINVAL, std::string(fn) + ": parameter " + std::to_string(p) +
                                    " was never marked ready, so bucket " + std::to_string(r->bucket_of[p]) +
                                    " cannot be reduced (DDP would wait for it forever)");
  }
  hipError_t e = hipEventRecord(r->done, r->comm);
  if (e != hipSuccess) return hip_err(e, std::string(fn) + ": hipEventRecord");
  e = hipStreamWaitEvent(reinterpret_cast<hipStream_t>(stream), r->done, 0);
  if (e != hipSuccess) return hip_err(e, std::string(fn) + ": hipStreamWaitEvent");
  return DDP_OK;
}

extern "C" int ddp_synthetic_backward_pass(const ddp_plan* plan, const void* const* src_arenas,
                                           void* const* grad_arenas, int32_t N, int32_t work, int32_t lds_kib,
                                           ddp_reducer* reducer, void* stream) {
  const char* fn = "ddp_synthetic_backward_pass";
  if (plan == nullptr) return fail(DDP_EINVAL, std::string(fn) + ": plan is NULL");
  if (N != plan->world_size) return fail(DDP_EINVAL, std::string(fn) + ": N differs from the plan's world size");
  if (work < 0) return fail(DDP_EINVAL, std::string(fn) + ": work < 0");
  if (lds_kib < 0 || lds_kib > 64) return fail(DDP_EINVAL, std::string(fn) + ": lds_kib must lie in [0, 64]");
  if (reducer != nullptr && reducer->plan != plan)
    return fail(DDP_EINVAL, std::string(fn) + ": the reducer was made for another plan");
  const int eb = ddp::elem_bytes(plan->dtype);
  int st = ddp::check_rank_buffers(const_cast<void* const*>(src_arenas), N, plan->arena_numel * eb, eb, fn,
                                   "src_arenas");
  if (st != DDP_OK) return st;
  st = ddp::check_rank_buffers(grad_arenas, N, plan->arena_numel * eb, eb, fn, "grad_arenas");
  if (st != DDP_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (reducer != nullptr) {
    st = ddp_reducer_prepare(reducer);
    if (st != DDP_OK) return st;
  }
  for (int32_t p = int32_t(plan->numels.size()) - 1; p >= 0; --p) {
    ddp::RankPtrs S{}, D{};
    const int64_t off = plan->arena_offsets[p] * eb;
    for (int r = 0; r < N; ++r) {
      S.p[r] = static_cast<char*>(const_cast<void*>(src_arenas[r])) + off;
      D.p[r] = static_cast<char*>(grad_arenas[r]) + off;
    }
    st = ddp::launch_synthetic_backward(S, D, N, plan->numels[p], plan->dtype, work, lds_kib, s);
    if (st != DDP_OK) return st;
    if (reducer != nullptr) {
      st = ddp_reducer_mark_ready(reducer, p, stream);
      if (st != DDP_OK) return st;
    }
  }
  return reducer != nullptr ? ddp_reducer_finalize(reducer, stream) : DDP_OK;
}
