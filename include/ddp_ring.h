/*
 * ddp_ring.h -- C ABI of the MI355X (gfx950) bucketed ring all-reduce of DDP
 * gradients over N virtual ranks whose buffers all live in one GPU's HBM.
 *
 * The operations follow three pages:
 *   [R]  "DDP 与 Ring All-Reduce" (blog.vllbc.top/visual-reading/ddp-ring-allreduce),
 *        sections 03 (two phases, buckets, overlap), 04 (traffic), 05 (step timing);
 *   [D]  "Day 17 数据并行 DP/DDP" (blog.ans20xx.com/posts/ai/day17),
 *        parts "bucket 与 overlap" and "源码阅读路线";
 *   [X]  "DDP 与 Ring-AllReduce" (xuesongtap.github.io/2025/09/06/ddp.html),
 *        §1.3.1 and the worked example of §1.3.2.
 *
 * Conventions shared by every entry point:
 *   - Every function returns DDP_OK (0) or a negative status; on failure
 *     ddp_last_error() gives a message for the calling thread. No C++
 *     exception crosses this boundary.
 *   - "device pointer" means memory from hipMalloc (or an allocator built on
 *     it, such as PyTorch's caching allocator) on the current HIP device.
 *     The library checks, with hipMemGetAddressRange, that every byte range it
 *     will touch lies inside one allocation, and that buffers written by one
 *     call do not overlap; a failed check returns DDP_EINVAL before anything
 *     is launched.
 *   - Arrays of device pointers (bufs, grad_arenas, bucket_bufs) are HOST
 *     arrays; the library copies them into the kernel arguments.
 *   - All device memory belongs to the caller. The library allocates only
 *     tables of its own: per plan and device, a copy of the bucket layout (a
 *     few bytes per member and per 16 KiB of bucket) and, for plans whose
 *     gradients and buckets share a dtype, the in-place sync's map of the
 *     gradient arena (2 bytes per 16 bytes of one rank's arena), made on the
 *     plan's first pack, unpack or in-place sync on that device and freed by
 *     ddp_plan_free; and per device, the persistent launches' barrier
 *     words (64 slots of 512 bytes plus a 512-byte status line, 32.5 KiB,
 *     allocated on the first persistent call on that device) and the
 *     allocation-free entry point's fixed 1 KiB array, both kept until the
 *     process ends.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without waiting; completion follows stream order,
 *     the analogue of waiting on the collective's work handle ([D], "源码阅读路线").
 *   - Chunking ([R] section 03; [X] §1.3.2.1): a buffer of `count` elements is
 *     cut into N chunks of L = ceil(count / N) elements; chunk c covers
 *     [c*L, min((c+1)*L, count)) and may be short or empty. In reduce-scatter
 *     step s rank r passes chunk (r-1-s) mod N to rank (r+1) mod N, which adds
 *     it into its own copy, rounded once to the buffer dtype (nearest, ties to
 *     even, subnormals kept); in all-gather step s rank r passes chunk
 *     (r-s) mod N and the receiver overwrites its copy. Chunk c therefore
 *     starts at rank c+1 and ends fully reduced on rank c ([X] §1.3.2.1).
 *   - N (the world size) lies in [1, DDP_MAX_RANKS]. Buffers are in place:
 *     rank r's buffer is read and overwritten.
 *   - Concurrency: calls may be issued from several host threads. Calls
 *     enqueued on different streams must not touch the same buffers at the
 *     same time (as with any kernels).
 */
#ifndef DDP_RING_H
#define DDP_RING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDP_MAX_RANKS 64

/* status codes */
#define DDP_OK 0
#define DDP_EINVAL (-1)       /* bad argument; nothing was launched */
#define DDP_EHIP (-2)         /* a HIP runtime call failed; message has hipGetErrorString */
#define DDP_ENORESOURCE (-3)  /* the persistent grid cannot be made co-resident */
#define DDP_ETIMEOUT (-4)     /* a persistent grid barrier gave up waiting */
#define DDP_ENOMEM (-5)       /* a host or device allocation of the library failed */

/* buffer element types */
#define DDP_FP32 0            /* IEEE binary32, 4 bytes */
#define DDP_BF16 1            /* bfloat16, 2 bytes: the upper half of a binary32 */

/* ring phases ([R] section 03) */
#define DDP_RS 0              /* reduce-scatter: add the received chunk */
#define DDP_AG 1              /* all-gather: overwrite with the received chunk */

/* all-reduce variants for ddp_sync */
#define DDP_VARIANT_FUSED 0
#define DDP_VARIANT_STEPS 1
#define DDP_VARIANT_PERSISTENT 2
#define DDP_VARIANT_VIEW 3       /* in place, no bucket buffers: bucket_allreduce_view */

typedef struct ddp_plan ddp_plan; /* opaque; host memory owned by the library */

/* Message describing the last failure of the calling thread ("" if none).
 * Every entry point checks its arguments and reports a bad call instead of
 * launching it: the fail-fast answer to [D] "常见疑问", where ranks that do not
 * make matching collective calls wait forever. */
const char* ddp_last_error(void);

/* ---------------------------------------------------------------- planner
 * ddp_bucket_plan: assign parameters to flat buckets ([R] section 03, parts
 * "Bucket" and "Overlap"; [D] "bucket 与 overlap").
 *   param_numels[n_params]: element counts in registration order (host array;
 *       each >= 0; n_params >= 0).
 *   dtype: DDP_FP32 or DDP_BF16 (the gradients' and the buckets' type).
 *   cap_bytes: capacity of every bucket after the first (> 0; 25 MiB =
 *       26214400 is DDP's default); first_bucket_bytes: capacity of bucket 0
 *       (> 0; 1 MiB = 1048576 is DDP's default).
 *   world_size: N, used to pad each bucket.
 *   *out receives a new plan, to be released with ddp_plan_free.
 * Rules: parameters are taken in reverse registration order; a parameter
 * that would push the open bucket past its capacity opens the next bucket; a
 * parameter larger than the capacity has a bucket of its own. With
 * V = 16 / element size, each member starts at a multiple of V elements and
 * takes round_up(numel, V) elements; a bucket's length is padded with zeros
 * to a multiple of N*V elements, so its N ring chunks are equal and start on
 * 16-byte boundaries. Buckets are numbered in launch order; every rank uses
 * the same plan and order.
 */
int ddp_bucket_plan(const int64_t* param_numels, int32_t n_params, int32_t dtype,
                    int64_t cap_bytes, int64_t first_bucket_bytes, int32_t world_size,
                    ddp_plan** out);

/* ddp_bucket_plan_ex: as ddp_bucket_plan, with gradients and buckets in
 * different dtypes. grad_dtype lays out the gradient arena and is the unit of
 * the capacities (DDP forms buckets over the gradients); comm_dtype is the
 * buckets' dtype: members start at multiples of its 16-byte vector and the
 * ring runs in it. The supported pairs are equal dtypes and fp32 gradients in
 * bf16 buckets: the bf16 compression hook ([D] reading list, "PyTorch DDP
 * Communication Hooks"), in which bucket_pack rounds every gradient to bf16
 * (nearest, ties to even), the ring adds in bf16 with one rounding per hop,
 * and bucket_unpack_scale widens to fp32 and rounds scale * value once. The
 * in-place sync (bucket_allreduce_view) does the same arithmetic on the fp32
 * gradients themselves. */
int ddp_bucket_plan_ex(const int64_t* param_numels, int32_t n_params, int32_t grad_dtype,
                       int32_t comm_dtype, int64_t cap_bytes, int64_t first_bucket_bytes,
                       int32_t world_size, ddp_plan** out);

/* Releases a plan ([R] section 03 "Bucket": built once, when DDP is
 * constructed) and its device tables (NULL is accepted). Must not be called
 * while work that uses the plan is still running. */
void ddp_plan_free(ddp_plan* plan);

/* Number of buckets ([R] section 03 "Bucket": each is one collective). */
int ddp_plan_num_buckets(const ddp_plan* plan, int32_t* out);

/* Bucket b's padded length in elements and its number of members ([R]
 * section 03 "Bucket": the gradients of a bucket form one flat buffer). */
int ddp_plan_bucket(const ddp_plan* plan, int32_t b, int64_t* padded_numel, int32_t* n_members);

/* Member i of bucket b: parameter index, offset in the bucket (elements) and
 * element count. Members are listed in bucket order, which is reverse
 * parameter order ([R] section 03 "Overlap"). */
int ddp_plan_member(const ddp_plan* plan, int32_t b, int32_t i, int32_t* param_idx,
                    int64_t* offset, int64_t* numel);

/* Layout of a rank's gradient arena (the parameters' .grad tensors that the
 * copy back of [R] section 05 writes): all parameters' gradients in
 * registration order, parameter p starting at param_offsets[p] elements (a
 * multiple of V, i.e. 16-byte aligned). Writes *arena_numel and, if
 * param_offsets is not NULL, n_params offsets into the host array. */
int ddp_plan_grad_arena(const ddp_plan* plan, int64_t* arena_numel, int64_t* param_offsets);

/* The in-place sync's map of the gradient arena ([R] sections 03 and 05,
 * gradient_as_bucket_view=True: each .grad is a view of its bucket), one entry
 * per 16-byte vector of one rank's arena (n = arena_numel / V entries, written to the
 * host array `out`): 0xFFFF for a vector holding no member element (the
 * alignment padding between parameters); otherwise the ring chunk of its
 * bucket that holds the vector (low byte) and how many of its V elements
 * belong to the member (high byte, V except in a member's last vector). The
 * kernels read the device copy of this map; the accessor lets the layout be
 * checked on the host. With fp32 gradients in bf16 buckets the entries
 * describe the fp32 arena (V = 4) and the chunks come from the bf16 buckets'
 * layout; no arena vector spans two chunks. */
int ddp_plan_arena_map(const ddp_plan* plan, uint16_t* out, int64_t n);

/* ---------------------------------------------------------------- pack / unpack
 * bucket_pack: copy gradients into bucket b's flat buffer on every rank
 * (the gradient-to-bucket copy of DDP's default gradient_as_bucket_view=False,
 * [R] sections 03 and 05).
 *   grad_arenas[N]: device pointers, 16-byte aligned, each holding one rank's
 *       arena as laid out by ddp_plan_grad_arena (arena_numel elements of the
 *       gradients' dtype).
 *   bucket_bufs[N]: device pointers, 16-byte aligned, each padded_numel
 *       elements (of the buckets' dtype) of bucket b; positions not covered
 *       by a member are zeroed.
 *   N must equal the plan's world size.
 */
int bucket_pack(const ddp_plan* plan, int32_t b, const void* const* grad_arenas,
                void* const* bucket_bufs, int32_t N, void* stream);

/* bucket_unpack_scale: copy bucket b back into every rank's gradients,
 * multiplying each element by `scale` (fp32) with one rounding to the dtype:
 * grad = rnd(scale * bucket). scale = 1/N turns the ring's sum into DDP's mean
 * ([R] section 05, step 3; [D] "源码阅读路线": divide by the world size, then
 * copy back). For N a power of two this equals division by N bit for bit.
 * Arguments as for bucket_pack; only members' elements are written. */
int bucket_unpack_scale(const ddp_plan* plan, int32_t b, const void* const* bucket_bufs,
                        void* const* grad_arenas, int32_t N, float scale, void* stream);

/* ---------------------------------------------------------------- ring all-reduce
 * bufs[N]: device pointers to the N rank buffers, `count` elements of `dtype`
 * each, aligned to the element size, pairwise disjoint. count >= 0; with
 * count = 0 nothing is read or written and the pointers may be NULL.
 */

/* One step of the ring ([R] section 03; [X] §1.3.2.1 / §1.3.2.2): all N
 * (rank r -> rank r+1) transfers of `step` in `phase`, in one launch.
 * phase = DDP_RS: buf[r+1][chunk (r-1-step) mod N] += buf[r][same chunk];
 * phase = DDP_AG: buf[r+1][chunk (r-step) mod N]  = buf[r][same chunk].
 * step in [0, N-2]. A full all-reduce is RS steps 0..N-2 then AG steps
 * 0..N-2, in order on one stream: 2(N-1) launches ([X] §1.3.1). */
int ring_allreduce_step(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                        int32_t step, int32_t phase, void* stream);

/* The first n_steps of the 2(N-1) steps ([X] §1.3.1: N-1 reduce-scatter
 * steps, then N-1 all-gather steps) in one cooperative launch, with a
 * grid-wide barrier between consecutive steps: the fixed per-step
 * synchronisation cost of [R] section 04 (2(N-1) steps, each with its own
 * latency) is paid inside one launch instead of at every launch. The barrier
 * words come from 64 slots per device, handed out in turn; a launch that
 * reuses a slot first makes its stream wait (on the GPU, not the host) for
 * the slot's previous user, whatever stream that was on. Not for graph
 * capture: use ring_allreduce_persistent_noalloc there. n_steps in [0, 2(N-1)]; 2(N-1) is the whole all-reduce. When the
 * N buffers exceed the 256 MB Infinity Cache, each step's tiles are handed
 * to the blocks by a ticket counter (in the launch's library-owned barrier
 * words), so no block's fixed share holds a step back; the result does not
 * depend on which block does which tile. Returns DDP_ENORESOURCE if the grid
 * cannot be co-resident, DDP_EINVAL if the launch would need 2^32 tiles or
 * more (far beyond any buffers that fit in device memory). A block that
 * waits at a barrier longer than 10 s aborts the launch (every block exits,
 * the result is incomplete) and sets a sticky flag read by
 * ddp_persistent_status. */
int ring_allreduce_persistent(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                              int32_t n_steps, void* stream);

/* As ring_allreduce_persistent ([X] §1.3.1; [R] section 04), with the
 * launch's knobs exposed:
 *   max_blocks: cooperative grid size (0: the default, 1024-thread blocks,
 *       seven for every eight compute units when the N buffers exceed the
 *       256 MB Infinity Cache; five for every eight when they fit, lowered
 *       until every block has the same number of tiles per step); it is
 *       never more than one block per tile of a step, nor more than one
 *       block per compute unit below the occupancy limit (at least one per
 *       compute unit);
 *   timeout_us: how long a block waits at a grid barrier before the launch
 *       gives up (ring_allreduce_persistent uses 10 s); in (0, 3600 s];
 *   extra_arrivals: added to every barrier's expected arrival count. It must
 *       be 0 except in tests of the time-out path, where a non-zero value makes
 *       every barrier wait for blocks that do not exist, so the launch times
 *       out after timeout_us and every block exits. */
int ring_allreduce_persistent_ex(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                 int32_t n_steps, int32_t max_blocks, int64_t timeout_us,
                                 uint32_t extra_arrivals, void* stream);

/* ring_allreduce_persistent_noalloc: ring_allreduce_persistent for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, kernels
 * and results; the launch's barrier words live in a fixed 1 KiB array
 * that the library holds in device memory from load time (one per GPU, until
 * the process ends), so no call allocates: no hipMalloc, no hipFree, no
 * allocating library routine. The array is one launch's worth and its size
 * does not depend on the inputs, so no input size is refused for it (the
 * limits are those of ring_allreduce_persistent). Every call on a GPU shares
 * that GPU's array: the barrier words are cleared on `stream` before each
 * launch, so calls on one stream are ordered, but calls that overlap on one
 * GPU (other streams, other host threads) race on the words and must not be
 * made. A barrier time-out sets the array's sticky status, which
 * ddp_persistent_status reports and clears. */
int ring_allreduce_persistent_noalloc(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                                      int32_t n_steps, void* stream);

/* ddp_persistent_test_hook: for tests of the time-out path only ([D]
 * "常见疑问": a collective that a participant never joins waits forever; here
 * it gives up and reports). With timeout_us > 0, every later persistent
 * launch of the process that takes default options (ring_allreduce_persistent,
 * its _noalloc form, and ddp_sync and the reducer with DDP_VARIANT_PERSISTENT)
 * expects extra_arrivals more blocks at each grid barrier and gives up after
 * timeout_us; timeout_us = 0 restores the defaults (10 s, no extra arrivals).
 * timeout_us in [0, 3600 s]. */
int ddp_persistent_test_hook(uint32_t extra_arrivals, int64_t timeout_us);

/* Cooperative grid size ring_allreduce_persistent ([X] §1.3.1) would use
 * for these arguments on the current device, and the device's compute-unit
 * count. */
int ddp_persistent_grid(int32_t N, int64_t count, int32_t dtype, int32_t* grid, int32_t* compute_units);

/* Waits for `stream`, then reports DDP_ETIMEOUT if any persistent launch on
 * the current device timed out since the last call (and clears the flag);
 * the message gives the arrivals seen and expected at that barrier. ([D]
 * "常见疑问": a collective that a participant never joins waits forever; a
 * grid barrier here gives up after its time-out and reports instead.) */
int ddp_persistent_status(void* stream);

/* The whole all-reduce in one pass: every element is read once from each of
 * the N ranks, summed in the exact order the ring adds it ([X] §1.3.2.1:
 * chunk c's sum starts with rank c+1 and adds ranks c+2, ..., c, one rounding
 * per add) and written to all N ranks ([X] §1.3.2.2: every rank ends with the
 * whole sum). The final state is bit-identical to the 2(N-1)
 * steps; the HBM traffic is 2*N*count*element bytes instead of
 * 5*(N-1)*count*element. */
int ring_allreduce_fused(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                         void* stream);

/* bucket_allreduce_view: the all-reduce of bucket b done in place on the
 * gradients, with no bucket buffer (the analogue of DDP's
 * gradient_as_bucket_view=True, [R] sections 03 and 05; [D] "bucket 与
 * overlap": the gradients are views of the bucket, so the gradient<->bucket
 * copies and one gradient's worth of memory disappear). Every member element
 * keeps its position in the bucket's layout, hence its ring chunk c and its
 * summation order (rank c+1 first, then c+2, ..., c, one rounding per add);
 * the sum is multiplied by `scale` (one rounding) and written to every rank's
 * gradient. The result equals bucket_pack + ring_allreduce_fused +
 * bucket_unpack_scale bit for bit, with 2*N*S_b bytes of traffic instead of
 * 6*N*S_b. For a plan of fp32 gradients in bf16 buckets (ddp_bucket_plan_ex:
 * DDP's bf16 compression hook on gradients that are the bucket) every
 * gradient is rounded to bf16 as it enters the sum, each add is rounded to
 * bf16, and scale * sum is rounded once to fp32: again bit for bit the
 * copying path, with no bf16 bucket.
 *   grad_arenas[N]: device pointers, 16-byte aligned, each arena_numel elements
 *       laid out by ddp_plan_grad_arena; read and overwritten (members only).
 *   N must equal the plan's world size. */
int bucket_allreduce_view(const ddp_plan* plan, int32_t b, void* const* grad_arenas, int32_t N,
                          float scale, void* stream);

/* ring_reduce_scatter_fused: the reduce-scatter phase alone, as its output:
 * every rank's gradient shard ([R] section 03: after the N-1 reduce-scatter
 * steps each rank holds one fully reduced chunk; [X] §1.3.2.1: chunk r on rank
 * r; [R] section 07: sharded data parallelism keeps such a shard per rank).
 * For every chunk c: shards[c][i] = rnd(scale * sum), where sum adds the N
 * ranks' element c*L+i in ring order (rank c+1 first, then c+2, ..., c, one
 * rounding per add) -- the value the N-1 reduce-scatter steps leave on rank c.
 *   bufs[N]: device pointers to the N input buffers (count elements each,
 *       element-aligned, pairwise disjoint); read only.
 *   shards[N]: device pointers; shards[c] receives chunk c's
 *       min(L, count - c*L) elements (L = ceil(count/N)); may be NULL for an
 *       empty chunk; must not overlap the inputs or each other.
 *   scale: fp32 multiplier (1 for the sum, 1/N for the mean).
 * Reads N*S bytes and writes S. */
int ring_reduce_scatter_fused(const void* const* bufs, void* const* shards, int32_t N, int64_t count,
                              int32_t dtype, float scale, void* stream);

/* ---------------------------------------------------------------- whole sync
 * ddp_sync: one DDP gradient synchronisation. For every bucket b in plan
 * order: bucket_pack, the all-reduce chosen by `variant` (DDP_VARIANT_FUSED,
 * _STEPS or _PERSISTENT) on bucket b's N buffers, bucket_unpack_scale with
 * `scale` (pass 1/N for DDP's mean). With DDP_VARIANT_PERSISTENT, a bucket
 * whose all-reduce gives up at a grid barrier (ring_allreduce_persistent) is
 * not copied back: its gradients keep their values, and ddp_persistent_status
 * reports DDP_ETIMEOUT once the stream has reached it. Bucket i+1 is never started before
 * bucket i ([R] section 03). For DDP_VARIANT_VIEW the gradients themselves
 * are reduced in place, all buckets in one launch over the arenas (every
 * bucket is ready when ddp_sync is called): each element is summed in its
 * own bucket's chunk order, so the result is bit for bit that of
 * bucket_allreduce_view on every bucket. To sync buckets as they become
 * ready, use the reducer below.
 *   grad_arenas[N]: as for bucket_pack.
 *   bucket_bufs[B*N]: bucket b of rank r at index b*N + r (host array); may
 *       be NULL for DDP_VARIANT_VIEW.
 */
int ddp_sync(const ddp_plan* plan, void* const* grad_arenas, void* const* bucket_bufs,
             int32_t N, int32_t variant, float scale, void* stream);

/* ---------------------------------------------------------------- overlap with backward
 * The reducer launches each bucket's sync as soon as its last gradient is
 * ready, on a communication stream, so that it overlaps the rest of backward
 * ([R] section 03 "Overlap" and section 05 step 2: a hook per gradient; the
 * last gradient of a bucket launches its all-reduce asynchronously; the same
 * bucket order on every rank, bucket i+1 never before bucket i; [D]
 * "梯度同步时机", "源码阅读路线"). One host thread drives a reducer.
 *
 * ddp_reducer_create: for `plan`, gradient arenas grad_arenas[N] and, unless
 *   variant is DDP_VARIANT_VIEW, bucket buffers bucket_bufs[B*N] (layout as
 *   for ddp_sync); each bucket's sync is the `variant` one with `scale`, and
 *   runs on comm_stream. The pointer arrays are copied; the plan must outlive
 *   the reducer. For DDP_VARIANT_VIEW the arenas are checked here, once, and
 *   must stay allocated while the reducer exists.
 *   comm_max_blocks (DDP_VARIANT_VIEW only; 0 for no limit): the syncs of all
 *   buckets but the last run on at most this many blocks (of min(N, 8)
 *   waves each), so they take few of the compute units that backward is
 *   still using (the way a
 *   collective library limits the channels a collective occupies); the last
 *   bucket, ready only once backward is over, runs full width. Results do not
 *   depend on it.
 *   The reducer starts prepared for a backward pass. */
typedef struct ddp_reducer ddp_reducer;
int ddp_reducer_create(const ddp_plan* plan, void* const* grad_arenas, void* const* bucket_bufs, int32_t N,
                       int32_t variant, float scale, int64_t comm_max_blocks, void* comm_stream,
                       ddp_reducer** out);
/* Releases a reducer ([R] section 03 "Overlap"); must not be called while
 * its syncs are still running (ddp_reducer_finalize waits for them). */
void ddp_reducer_free(ddp_reducer* reducer);
/* Start of a backward pass: no gradient is ready ([R] section 05, step 2: the
 * hooks fire as backward produces the gradients). */
int ddp_reducer_prepare(ddp_reducer* reducer);
/* Gradient `param` (of every rank) has been produced by work already enqueued
 * on producer_stream ([R] section 05, step 2: the hook of a gradient; the
 * last one of a bucket launches its all-reduce). If it completes its bucket, an event recorded on
 * producer_stream gates that bucket's sync, which is enqueued on the
 * communication stream once every earlier bucket has been. Marking a
 * parameter twice in one pass is an error. */
int ddp_reducer_mark_ready(ddp_reducer* reducer, int32_t param, void* producer_stream);
/* End of backward: `stream` waits until every bucket's sync has finished
 * ([R] section 05, step 5: every bucket's all-reduce completes before the
 * optimizer reads the gradients). With DDP_VARIANT_PERSISTENT a bucket whose
 * all-reduce timed out keeps its gradients (see ddp_sync); check
 * ddp_persistent_status after this stream is done.
 * Returns DDP_EINVAL, naming the parameter, if some gradient was never marked
 * ready (where DDP would wait for it forever). */
int ddp_reducer_finalize(ddp_reducer* reducer, void* stream);

/* ddp_synthetic_backward: a stand-in for the backward kernels that produce
 * gradients ([R] section 03 "Overlap": communication is hidden behind the
 * backward computation of earlier layers), for overlap measurements: dsts[r][i] = srcs[r][i] for every rank
 * r < N and i < numel, after `work` dependent fused multiply-adds per element
 * that do not change the copied value. Each 256-thread block reserves
 * lds_kib KiB of LDS (0..64) that it never uses, which caps how many blocks
 * share a compute unit (64 KiB: two blocks, two waves per SIMD), the way
 * register- or LDS-hungry backward kernels are capped. */
int ddp_synthetic_backward(const void* const* srcs, void* const* dsts, int32_t N, int64_t numel, int32_t dtype,
                           int32_t work, int32_t lds_kib, void* stream);

/* ddp_synthetic_backward_pass: one synthetic backward pass over the plan's
 * parameters in reverse registration order (the order DDP's bucketing
 * assumes backward produces them, [R] section 03 "Overlap"): for every
 * parameter p, ddp_synthetic_backward copies src_arenas[r]'s gradient p into
 * grad_arenas[r] on `stream` for all N ranks (with `work` and lds_kib as
 * there), then, if `reducer` is not NULL,
 * marks p ready. With a reducer the pass starts with ddp_reducer_prepare and
 * ends with ddp_reducer_finalize(stream). Arenas are laid out as for
 * bucket_pack. */
int ddp_synthetic_backward_pass(const ddp_plan* plan, const void* const* src_arenas, void* const* grad_arenas,
                                int32_t N, int32_t work, int32_t lds_kib, ddp_reducer* reducer, void* stream);

/* ---------------------------------------------------------------- checks and probes
 * ddp_count_mismatches: *out_dev (a device uint64, overwritten) receives the
 * number of element positions at which some rank's bits differ from rank 0's
 * (0 after a complete all-reduce, [X] §1.3.2.2). */
int ddp_count_mismatches(void* const* bufs, int32_t N, int64_t count, int32_t dtype,
                         uint64_t* out_dev, void* stream);

/* ddp_device_alloc: device memory on the current device for the ring's N
 * rank buffers, DDP's buckets or the gradient arenas ([R] section 03: every
 * rank holds a buffer of the whole gradient, cut into N chunks), owned by the
 * caller and released with ddp_device_free. flags = 0 is hipMalloc;
 * DDP_ALLOC_CONTIGUOUS asks for physically contiguous memory: on MI355X
 * the 64 ranks x 300M fused all-reduce ran 25.0-25.2 ms on such buffers
 * whether they were a process's first allocations or not, where torch's
 * first allocations ran up to 29.7 ms on some machines (more second-level
 * address translation per request); at 8 ranks x 1 GiB it ran within 5 %
 * of torch's allocations, faster or slower from run to run. Returns
 * DDP_EINVAL for nbytes <= 0, an
 * unknown flag or a NULL out (*out is set to NULL on every failure), and
 * DDP_ENOMEM when the runtime cannot provide the memory (contiguous memory
 * can run out before memory does: the caller may retry with flags = 0). */
#define DDP_ALLOC_CONTIGUOUS 1
int ddp_device_alloc(int64_t nbytes, int32_t flags, void** out);

/* ddp_device_free: releases memory from ddp_device_alloc (NULL is
 * accepted); no work that uses it may still be running ([R] section 03's
 * buffers live as long as the training job). */
int ddp_device_free(void* p);

/* ddp_copy_probe: copies nbytes (a multiple of 16) from src to dst with 16-byte
 * vector loads and stores: a same-run reference for achievable HBM bandwidth
 * (on one GPU the ring's bandwidth term of [R] section 04 is paid in HBM
 * traffic) and for scaling memory-traffic counters. */
int ddp_copy_probe(void* dst, const void* src, int64_t nbytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DDP_RING_H */
