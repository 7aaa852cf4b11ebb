/*
 * pod_attn.h - C ABI of the MI355X (gfx950) Prefill-On-Decode attention library.
 *
 * One pod_run() call is one kernel launch that computes paged-KV-cache attention
 * for two roles at once: a (chunked, causal) prefill batch and a decode batch.
 * It writes O and a base-2 LSE per (query token, qo head) for each role.
 *
 * Sources, FlashInfer pages:
 *   [POD]   www.dpshk.com/news/5405057  (PODWithPagedKVCacheWrapper /
 *           BatchPODWithPagedKVCacheWrapper article)
 *   [TOUR]  www.gsyq.cn/news/442943     (FlashInfer README tour)
 *   [CUDNN] www.gsyq.cn/news/452757     (flashinfer.cudnn backend article)
 *
 * Lifecycle: plan once, run many ([POD] "plan/run 生命周期"). pod_plan() takes
 * host copies of the length arrays only and turns them into a work list that is
 * copied into the caller's int workspace; pod_run() may then be called once per
 * layer with different q / KV / output pointers of the same shapes. All policy
 * (causal, window, scale, sinks on/off) is fixed at plan time, as the batch
 * wrapper does ([POD] "BatchPOD 的 run 差异").
 *
 * Ownership: the caller allocates and owns every device buffer (queries, KV
 * pools, page indices, outputs, LSE, sinks and both workspaces). The library
 * keeps host plan state and two small pinned staging buffers; pod_run() never
 * allocates device memory and never synchronises the host.
 *
 * Errors: every entry point returns 0 on success or one of the POD_ERR_* codes;
 * pod_last_error() returns a message for the calling thread's last failure. On
 * an error nothing is enqueued on the stream.
 */
#ifndef POD_ATTN_H
#define POD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  POD_OK = 0,
  POD_ERR_INVALID = 1,      /* bad shapes, page tables, ranges or null pointers */
  POD_ERR_UNSUPPORTED = 2,  /* head_dim != 128, unknown dtype, group size > 128 */
  POD_ERR_NOT_PLANNED = 3,  /* pod_run before pod_plan, or args that contradict the plan */
  POD_ERR_WORKSPACE = 4,    /* a workspace is smaller than the plan needs */
  POD_ERR_HIP = 5           /* a HIP runtime call failed (message in pod_last_error) */
};

enum { POD_DTYPE_F16 = 0, POD_DTYPE_BF16 = 1, POD_DTYPE_FP8_E4M3 = 3 };

/* Item order policies for the fused grid (see pod_plan_desc.order). */
enum {
  POD_ORDER_INTERLEAVE = 0,
  POD_ORDER_PREFILL_FIRST = 1,
  POD_ORDER_DECODE_FIRST = 2,
  POD_ORDER_LONGEST_FIRST = 3
};

/*
 * One role of the POD call ([POD] "批量 POD" plan inputs: qo_indptr, kv_indptr,
 * last_page_len per side). All arrays are HOST memory, int32, read during
 * pod_plan() only.
 *   batch         number of requests; 0 leaves the role empty.
 *   qo_indptr     [batch+1] query-token offsets; qo_indptr[0] == 0, non-decreasing.
 *                 Rows of request b are q[qo_indptr[b] .. qo_indptr[b+1]).
 *   kv_indptr     [batch+1] offsets into kv_indices; kv_indptr[0] == 0, strictly
 *                 increasing (every request holds at least one page).
 *   last_page_len [batch] 1 <= last_page_len[b] <= page_size. The request's KV
 *                 length is (pages - 1) * page_size + last_page_len ([POD]
 *                 "plan 内部做了什么", get_seq_lens).
 *   causal        bottom-right causal mask: row i of a request with q_len rows
 *                 and kv_len keys sees keys 0 .. kv_len - q_len + i ([CUDNN]
 *                 "Decode 能力矩阵与参数", q_len_per_req). Requires kv_len >= q_len.
 *   window_left   -1 = off; else row i also drops keys before p_i - window_left,
 *                 p_i = kv_len - q_len + i, so window_left keys strictly before the
 *                 diagonal plus the diagonal remain ([CUDNN] window alignment note).
 *   sm_scale      softmax scale; <= 0 selects 1/sqrt(head_dim) ([POD] "Prefill 侧参数");
 *                 above 1e6 (or NaN) is refused with POD_ERR_INVALID.
 */
typedef struct pod_role_desc {
  int32_t batch;
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* last_page_len;
  int32_t causal;
  int32_t window_left;
  float sm_scale;
} pod_role_desc;

/*
 * Plan description.
 *   num_qo_heads, num_kv_heads  num_qo_heads must be a multiple of num_kv_heads;
 *                 qo head h reads kv head h / (num_qo_heads / num_kv_heads) (GQA,
 *                 [POD] "plan/run 生命周期"). Group size must be <= 128.
 *   head_dim      must be 128.
 *   page_size     tokens per page, >= 1.
 *   dtype         POD_DTYPE_F16 or POD_DTYPE_BF16; q, K/V and O share it. LSE is fp32.
 *   has_sinks     1: pod_run takes a per-qo-head fp32 sink logit, an extra softmax
 *                 term with a zero value row ([CUDNN] "Decode 能力矩阵与参数", sinks).
 *   num_cus       compute units to plan for; 0 asks the device (pod_plan) or uses 256
 *                 (pod_plan_compute / pod_workspace_bytes).
 *   decode_chunk  keys per split of a decode request: 0 = planner's choice,
 *                 -1 = never split, else rounded up to a multiple of 64.
 *   order         POD_ORDER_* policy for when a persistent workgroup runs its key
 *                 chunks (decode-style items) relative to its query tiles
 *                 (prefill-style items); every workgroup's list holds both kinds in
 *                 proportion to their estimated cost, placed by die:
 *                 INTERLEAVE (default): workgroups w with (w / 8) odd run their key
 *                 chunks first, the others their query tiles first, so half of each
 *                 die's workgroups start on each kind and both kinds run at once;
 *                 PREFILL_FIRST / DECODE_FIRST: every workgroup runs its query tiles
 *                 / its key chunks first; LONGEST_FIRST: a workgroup runs its key
 *                 chunks first when its heaviest key chunk costs more than its
 *                 heaviest query tile of either role. Results do not depend on the
 *                 order. Any other value is POD_ERR_INVALID.
 *   decode_kv_dtype  element type of the decode role's K/V pools: 0 = `dtype`, or
 *                 POD_DTYPE_FP8_E4M3 (OCP E4M3, 1 byte, strides still in elements):
 *                 the FP8 KV cache whose calibration scales the POD article lists
 *                 with the decode run parameters ([POD] "Decode 侧参数与'plan 覆盖'行为"). q and O stay
 *                 `dtype`; values are widened exactly to `dtype` inside the launch.
 *                 Every decode (request, kv head) then runs as key chunks: requests
 *                 with more than 32 rows (q_len * group) are cut into 32-row slices
 *                 over the same keys (each slice reads the K/V rows again, from the
 *                 die's L2 when its slices run together). The prefill role keeps
 *                 `dtype` K/V. An FP8 decode role needs kv_indices at pod_run
 *                 (POD_ERR_INVALID for NULL) and K/V strides that are multiples of
 *                 16 elements.
 */
typedef struct pod_plan_desc {
  pod_role_desc prefill;
  pod_role_desc decode;
  int32_t num_qo_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;
  int32_t has_sinks;
  int32_t num_cus;
  int32_t decode_chunk;
  int32_t order;
  int32_t decode_kv_dtype;
} pod_plan_desc;

/*
 * Device buffers of one role for pod_run(). Strides are in elements.
 *   q        [rows, num_qo_heads, 128]: element (t, h, d) at t*q_stride_tok +
 *            h*q_stride_head + d (head_dim innermost and dense).
 *   k_cache, v_cache  paged pools. Element (page, slot, kv_head, d) at
 *            page*kv_stride_page + slot*kv_stride_tok + kv_head*kv_stride_head + d,
 *            for K and V alike. The combined NHD cache [P, 2, page_size, H_kv, 128]
 *            of [POD] "批量 POD" is k_cache = base, v_cache = base + page_size*H_kv*128,
 *            kv_stride_page = 2*page_size*H_kv*128, kv_stride_tok = H_kv*128,
 *            kv_stride_head = 128. HND pools only change the strides.
 *   kv_indices  [kv_indptr[batch]] int32 physical page ids, or NULL for identity
 *            (logical page n is physical page n).
 *   out      [rows, num_qo_heads, 128] in dtype, element (t, h, d) at
 *            t*out_stride_tok + h*out_stride_head + d.
 *   lse      [rows, num_qo_heads] fp32 base-2 LSE (sink excluded), dense; or NULL.
 */
typedef struct pod_role_args {
  const void* q;
  int64_t q_stride_tok;
  int64_t q_stride_head;
  const void* k_cache;
  const void* v_cache;
  int64_t kv_stride_page;
  int64_t kv_stride_tok;
  int64_t kv_stride_head;
  const int32_t* kv_indices;
  void* out;
  int64_t out_stride_tok;
  int64_t out_stride_head;
  float* lse;
} pod_role_args;

/*
 * sinks: device fp32 [num_qo_heads]; required iff the plan had has_sinks.
 * q_scale_d, k_scale_d, v_scale_d: the decode role's calibration scales for an
 * FP8 KV cache ([POD] "Decode 侧参数与'plan 覆盖'行为": the only decode
 * parameters that take effect at run time): q_scale_d * k_scale_d multiply the
 * decode sm_scale, v_scale_d multiplies the decode output (folded into the
 * launch's final normalisation, before the cast to `dtype`; the LSE does not
 * see it). 0 means 1.0; they apply to any decode_kv_dtype. Each must be finite,
 * q_scale_d * k_scale_d must be > 0 and sm_scale_d * q_scale_d * k_scale_d must
 * stay <= 1e6 (the bound plan puts on sm_scale); otherwise pod_run returns
 * POD_ERR_INVALID and enqueues nothing.
 */
typedef struct pod_run_args {
  pod_role_args prefill;
  pod_role_args decode;
  const float* sinks;
  float q_scale_d;
  float k_scale_d;
  float v_scale_d;
} pod_run_args;

/* Counts of what a plan holds (filled by pod_plan_compute / pod_plan_stats). */
typedef struct pod_plan_info {
  int32_t n_items;          /* work items (workgroups with work) */
  int32_t n_prefill_items;
  int32_t n_decode_items;
  int32_t n_groups;         /* split (request, kv head) units that need the LSE merge */
  int32_t n_slots;          /* partial-state slots in the float workspace */
  int32_t grid;             /* persistent workgroups launched: one per CU, or, when
                               no die holds more items than it has CUs (outside
                               graph mode), 8 x the most items any die holds, each
                               workgroup then running one item */
  int32_t decode_chunk;     /* keys per decode split actually used */
  int32_t image_ints;       /* int32 words of the work-list image */
  int64_t float_ws_bytes;   /* float workspace the plan needs */
  int64_t int_ws_bytes;     /* int workspace the plan needs (two image halves) */
} pod_plan_info;

typedef struct pod_ctx* pod_ctx_t;

/*
 * Create a context bound to HIP device `device`. float_ws and int_ws are
 * caller-owned device buffers on that device (128 MB for the float workspace is
 * the pages' default, [POD] "使用建议与已知限制"). The context stores the
 * pointers; it does not take ownership.
 */
int pod_create(pod_ctx_t* out, int device, void* float_ws, size_t float_ws_bytes,
               void* int_ws, size_t int_ws_bytes);

/*
 * Graph mode ([POD] "CUDAGraph 模式的运行时约束": the batch size is fixed when the
 * wrapper is built and plan checks it). Like pod_create, plus:
 *   - every pod_plan must have prefill.batch == prefill_batch and
 *     decode.batch == decode_batch, and keep the first plan's heads, head_dim,
 *     page_size, dtype, has_sinks, num_cus and each role's causal, window_left
 *     and sm_scale; otherwise POD_ERR_INVALID;
 *   - the work-list image lives at the start of int_ws (one image, so int_ws
 *     needs only image_ints * 4 bytes) and pod_plan copies it on its `stream`;
 *   - pod_run is one plain kernel launch of the full persistent grid with no
 *     event operations: it can be captured into a HIP graph, and the captured
 *     launch reads whatever plan was copied last, so a graph replays correctly
 *     after any later plan on the same stream (the launch arguments carry only
 *     buffer pointers and plan-time policy; what a plan decides is read from
 *     the image). The caller keeps q, the K/V pools, kv_indices, out and lse at
 *     the captured addresses and sizes them for the largest plan.
 * pod_plan must still not be called during capture. batch sizes must be >= 0.
 */
int pod_create_graph(pod_ctx_t* out, int device, void* float_ws, size_t float_ws_bytes,
                     void* int_ws, size_t int_ws_bytes, int32_t prefill_batch,
                     int32_t decode_batch);

/*
 * Release the context's host state, staging buffers, events and copy stream
 * after the launches and copies it issued have completed ([POD] "使用建议与已知
 * 限制": the workspaces stay the caller's, on the caller's device). The caller's
 * workspaces are not freed. NULL is accepted; returns POD_OK.
 */
int pod_destroy(pod_ctx_t ctx);

/*
 * Build the work list from host length arrays and put it on the device: what
 * the pages' plan() does ([POD] "plan 内部做了什么": per-request KV lengths from
 * the page counts and last_page_len, split-KV decisions, the auxiliary data that
 * later runs reuse; "plan/run 生命周期": plan before any run, cached for many
 * runs; "Batch 版本 plan 的 colocated-CTA 调度细节": how the two roles share the
 * device). Unlike the pages' plan it takes no page indices: the work list
 * depends on lengths only, and kv_indices are pod_run arguments.
 *   Default context: plans alternate between the two halves of the int
 *   workspace. The copy runs on a stream the context owns, once the launches of
 *   the plan before last (which read the same half) have finished (the host
 *   waits for them only if they are still running), so it overlaps the
 *   previous plan's launches. While the previous plan's launch still runs,
 *   pod_plan then waits on the host for that copy alone (a few microseconds),
 *   so pod_run enqueues its launch without a cross-stream wait; when the GPU is
 *   idle pod_plan returns at once and pod_run orders its launch after the copy
 *   on the device.
 *   The first copy into each half is also ordered after the work queued on
 *   `stream` when pod_plan is called (so a caller that initialises int_ws on
 *   `stream` just before, or still uses that memory there, is safe); pod_plan
 *   then waits for that work too. `stream` serves only this in this mode.
 *   Graph context (pod_create_graph): the copy is enqueued on `stream`, ahead of
 *   the launches that follow there; pod_plan does not wait for it.
 * Errors: POD_ERR_INVALID / POD_ERR_UNSUPPORTED for descriptors the planner
 * rejects (the pages' ValueError / NotImplementedError cases),
 * POD_ERR_WORKSPACE if either workspace is too small for this plan, POD_ERR_HIP
 * for a failed copy; on any error the previous plan stays in force. Not to be
 * called during stream capture ([POD] "plan/run 生命周期"). Replaces any
 * previous plan of this context.
 */
int pod_plan(pod_ctx_t ctx, const pod_plan_desc* desc, void* stream);

/*
 * Counts of the context's current plan (the auxiliary data the pages' plan
 * caches for run, [POD] "plan/run 生命周期"). POD_ERR_NOT_PLANNED before the
 * first successful pod_plan.
 */
int pod_plan_stats(pod_ctx_t ctx, pod_plan_info* info);

/*
 * The pages' run() ([POD] "run 参数详解": one call produces both roles'
 * outputs; "BatchPOD 的 run 差异": every policy parameter comes from the plan,
 * and the batch wrapper returns both LSEs). Enqueues the fused attention
 * launch on `stream`: exactly one kernel launch (none if the plan holds no
 * work; the plan's work list is already on the device). Buffers must match the
 * plan's shapes and dtype; they are not read on the host. Asynchronous;
 * allocates nothing; leaves the workspace counters at zero when the launch
 * completes, so runs can be repeated without a re-plan. Errors (nothing is
 * enqueued): POD_ERR_NOT_PLANNED before a plan or for sinks that contradict it,
 * POD_ERR_INVALID for NULL required buffers, non-positive or misaligned
 * strides and bad scales (see pod_run_args), POD_ERR_UNSUPPORTED for pool
 * strides of 2^30 elements or more, POD_ERR_HIP if the launch fails.
 */
int pod_run(pod_ctx_t ctx, const pod_run_args* args, void* stream);

/*
 * Cascade merge of two attention states of the same rows over disjoint key
 * sets, e.g. a shared-prefix level and a per-request level ([TOUR] core
 * operator list, "Cascade Attention"; the base-2 LSE of [CUDNN] "LSE 契约" is
 * what such a merge consumes). Per (row, head):
 *   L = log2(2^lse_a + 2^lse_b),  O = 2^(lse_a - L) O_a + 2^(lse_b - L) O_b;
 * a state with lse = -inf holds no keys and weighs 0; if both do, O = 0 and
 * L = -inf. With `sinks` (device fp32 [num_heads], or NULL) the merged O is then
 * divided by 1 + 2^(sink * log2(e) - L) and L is kept: the sink is applied once,
 * so both inputs must be sink-free.
 *   o_a, o_b, o_out  device, `dtype`, dense [rows, num_heads, head_dim], 16-byte
 *                    aligned; o_out may be o_a or o_b itself (each element is
 *                    read before it is written), no other overlap.
 *   lse_a, lse_b, lse_out  device fp32 [rows, num_heads], 4-byte aligned; the
 *                    same aliasing rule.
 *   head_dim must be 128 (else POD_ERR_UNSUPPORTED); rows == 0 enqueues nothing.
 * One kernel launch on `stream` of device `device`; asynchronous; allocates
 * nothing. POD_ERR_INVALID for NULL buffers, negative sizes or misalignment.
 */
int pod_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                     void* o_out, float* lse_out, int64_t rows, int num_heads, int head_dim,
                     int dtype, const float* sinks, int device, void* stream);

/*
 * Message for the calling thread's last failed call ("" after a success). The
 * codes map to the pages' Python conventions: POD_ERR_INVALID is the
 * ValueError the wrappers raise for inputs that break their constraints
 * ([POD] "CUDAGraph 模式的运行时约束": mismatched batch sizes and buffers),
 * POD_ERR_UNSUPPORTED their NotImplementedError. The string stays valid until
 * the thread's next call into the library.
 */
const char* pod_last_error(void);

/*
 * Workspace sizes the plan of `desc` needs (host only; no device access):
 * float_ws_bytes for split-KV partial states, int_ws_bytes for the work list
 * (two alternating images). The pages recommend a 128 MB float workspace
 * ([POD] "使用建议与已知限制"); this query gives the exact need, which grows with
 * the number of split decode chunks. The sizes are those of a full grid (one
 * workgroup per CU, as a graph-mode context keeps), an upper bound for the
 * smaller grid pod_plan gives a plan with few items. Either output pointer may
 * be NULL. Errors as pod_plan's validation (POD_ERR_INVALID /
 * POD_ERR_UNSUPPORTED).
 */
int pod_workspace_bytes(const pod_plan_desc* desc, size_t* float_ws_bytes,
                        size_t* int_ws_bytes);

/*
 * The planner alone, on the host ([POD] "plan 内部做了什么", the host-side part
 * of plan): validate `desc` and write the work-list image
 * (the exact int32 words pod_plan copies to the device) into `image`, which has
 * room for `image_cap` words. `info` (optional) receives the counts. Returns
 * POD_ERR_WORKSPACE with info->image_ints set if `image` is too small. No device
 * access, so it runs without a GPU. Image layout: see pod_image_layout below.
 */
int pod_plan_compute(const pod_plan_desc* desc, int32_t* image, size_t image_cap,
                     pod_plan_info* info);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): pod_plan and
 * pod_run in one call, with no context and no workspaces. The work list and the
 * split-KV partial states live in the library's static device scratch (64 MiB
 * per device, held until the process ends: a 16 MiB work list and 48 MiB of
 * partial states, about 2,900 split chunks of 32 rows); plans that need more
 * are refused with POD_ERR_WORKSPACE before anything is enqueued.
 *   desc, args  as for pod_plan and pod_run (num_cus 0 asks `device`); the
 *               host arrays of desc are read during the call only.
 *   device      the HIP device whose scratch is used; made current for the
 *               call and restored after.
 *   stream      the work list is copied from host memory on `stream`, then
 *               the fused grid is launched there. The copy is from memory that
 *               is not pinned, so the call may wait on the host for work
 *               already queued on `stream`.
 * Calls no hipMalloc, hipHostMalloc or hipFree (the host planner's working
 * memory comes from the C++ heap). Every call on a device shares that device's
 * scratch and the library's host image buffer: calls are serialised on the
 * host, and calls whose launches can overlap on one device (different streams
 * without ordering between them) race on the scratch. Errors as pod_plan and
 * pod_run, plus POD_ERR_WORKSPACE for plans above the static limits.
 */
int pod_run_static(const pod_plan_desc* desc, const pod_run_args* args, int device, void* stream);

/*
 * Work-list image layout (int32 words), for inspection by tools and tests.
 *   header[POD_HDR_WORDS]: [0] magic POD_IMAGE_MAGIC, [1] n_items, [2] grid,
 *     [3] n_reqs, [4] n_groups, [5] reqs_off, [6] items_off, [7] groups_off,
 *     [8] counters_off, [9] n_slots, [10] slot_floats, [11] decode_chunk,
 *     [12] wgs_off, [13] blocks_off, [14] n_blocks, [15] pool_first,
 *     [16] pool_count, [17] queue_off, [18] tdesc_off.
 *   reqs[n_reqs][4]: {qo_start, qo_len, kv_len, page_start} per request, prefill
 *     requests first, then decode requests.
 *   items[n_items][8]: {flags, req, kv_head, tok0, ntok, kv_begin, kv_end, group}.
 *     flags bit 0: role (0 prefill, 1 decode); bit 1: kind (0 = query tile of up
 *     to 256 rows, tokens tok0 .. tok0 + ntok - 1; 1 = key chunk of up to 32 of the
 *     request's q_len*group rows, from row tok0 on (a multiple of 32; ntok =
 *     q_len)); bits 8..: split index. group == -1: the item writes its output
 *     directly. Items are grouped
 *     by workgroup (its query tiles, then its key chunks); the last pool_count
 *     items, from pool_first on, are key chunks that any workgroup takes from a
 *     shared queue once its own list is done.
 *   tdesc[n_items][8]: per query tile {first query row, tokens, kv head, diagonal
 *     key of the first token, key end, kv_len, 0, 0}; per key chunk its request's
 *     {qo_start, qo_len, kv_len, page_start, 0, 0, 0, 0}.
 *   wgs[grid][8]: per persistent workgroup {first item, query tiles, key chunks,
 *     first block, blocks, chunks run first (0/1), prefill-role tiles, blocks of
 *     those}. Workgroup w runs on die w % 8.
 *   blocks[n_blocks][4]: the query tiles' 64-key blocks in each workgroup's order:
 *     {first key, last key of the item, first page of the request, meta}; meta
 *     bit 31 first block of its item, bit 30 role, bits 16..29 kv head, bits
 *     0..15 tile index in the workgroup's list.
 *   groups[n_groups][4]: {n_splits, first_slot, req, kv_head}, one per (request,
 *     kv head, row slice) whose keys are split.
 *   counters[n_groups]: arrival counters, zero in the image.
 *   queue[2]: next pool item and workgroups done with the pool, zero in the image.
 */
enum { POD_HDR_WORDS = 24, POD_IMAGE_MAGIC = 0x504f4431 };

#ifdef __cplusplus
}
#endif

#endif /* POD_ATTN_H */
