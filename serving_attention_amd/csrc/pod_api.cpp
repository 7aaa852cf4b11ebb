// C ABI of the POD attention library: validation, plan upload, launch.
// The interface follows the plan-once / run-many wrappers of the POD article
// (www.dpshk.com/news/5405057, "plan/run 生命周期", "BatchPOD 的 run 差异").
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "pod_internal.h"

namespace {

thread_local std::string g_err;

int set_err(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_err(hipError_t e, const char* what) {
  g_err = std::string(what) + ": " + hipGetErrorString(e);
  return POD_ERR_HIP;
}

struct RolePlan {
  int32_t batch = 0;
  int32_t rows = 0;
  int32_t causal = 0;
  int32_t window_left = -1;
  float sm_scale = 0.f;
};

// What a plan fixes for the runs that use it (besides the work list itself).
struct PlanShape {
  RolePlan role[2];
  int32_t num_qo_heads = 0, num_kv_heads = 0, page_size = 0, dtype = 0, has_sinks = 0;
  bool decode_kv_fp8 = false;
};

// The shape of a validated plan descriptor.
void plan_shape(const pod_plan_desc& d, PlanShape& s) {
  const pod_role_desc* rd[2] = {&d.prefill, &d.decode};
  for (int r = 0; r < 2; ++r) {
    RolePlan& rp = s.role[r];
    rp.batch = rd[r]->batch;
    rp.rows = rd[r]->batch > 0 ? rd[r]->qo_indptr[rd[r]->batch] : 0;
    rp.causal = rd[r]->causal ? 1 : 0;
    rp.window_left = rd[r]->window_left;
    rp.sm_scale = rd[r]->sm_scale > 0.f ? rd[r]->sm_scale : 1.0f / std::sqrt((float)d.head_dim);
  }
  s.num_qo_heads = d.num_qo_heads;
  s.num_kv_heads = d.num_kv_heads;
  s.page_size = d.page_size;
  s.dtype = d.dtype;
  s.has_sinks = d.has_sinks ? 1 : 0;
  s.decode_kv_fp8 = d.decode_kv_dtype == POD_DTYPE_FP8_E4M3;
}

// Check the run arguments against the plan's shape and fill the launch
// parameters (all but the work-list image and the partial-state buffer).
int fill_params(const PlanShape& sh, const pod_run_args* args, pod::Params& p);

}  // namespace

namespace {

// pod_run_static: the work list is written here on the host and copied into
// the device's static scratch array; one call at a time.
std::mutex g_static_mu;
int32_t g_static_image[pod::kStaticImageBytes / sizeof(int32_t)];

}  // namespace

struct pod_ctx {
  int device = 0;
  void* float_ws = nullptr;
  size_t float_bytes = 0;
  void* int_ws = nullptr;
  size_t int_bytes = 0;
  int num_cus = 0;
  bool planned = false;
  PlanShape shape;
  pod_plan_info info{};
  int32_t hdr[POD_HDR_WORDS] = {};
  // Plans alternate between two halves of the int workspace, each with a
  // pinned staging buffer; the image goes up on a library stream while the
  // previous plan's kernels may still run, and pod_run waits for it.
  int32_t* staging[2] = {nullptr, nullptr};
  size_t staging_cap[2] = {0, 0};
  hipEvent_t staged[2] = {nullptr, nullptr};   // copy of plan k done (host and device side)
  bool staged_pending[2] = {false, false};
  hipEvent_t used[2] = {nullptr, nullptr};     // last launch that read half k done
  bool used_pending[2] = {false, false};
  hipStream_t copy_stream = nullptr;
  // The first copy into each half waits for the work the caller had queued on
  // its stream by then (its initialisation of the workspace, say); later
  // copies into a half are ordered by the launches that last read it.
  hipEvent_t caller_ready = nullptr;
  bool half_ordered[2] = {false, false};
  int next_staging = 0;
  int cur = 0;                                 // half of the current plan
  // Graph mode (pod_create_graph): fixed batch sizes, one image at the start of
  // the int workspace copied on the caller's stream, and the plan-time policy
  // of the first plan kept, so a captured pod_run stays valid across plans.
  bool graph = false;
  int32_t fixed_batch[2] = {0, 0};
  bool policy_set = false;
  pod_plan_desc policy{};                      // first plan (resolved num_cus, scales)
};

namespace {

// half k of the int workspace (256-byte aligned; each half holds one plan)
int32_t* int_half(const pod_ctx* c, int k) {
  const size_t half = (c->int_bytes / 2) & ~(size_t)255;
  return reinterpret_cast<int32_t*>(reinterpret_cast<char*>(c->int_ws) + (size_t)k * half);
}

struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

}  // namespace

namespace {

int fill_params(const PlanShape& sh, const pod_run_args* args, pod::Params& p) {
  if (sh.has_sinks && !args->sinks)
    return set_err(POD_ERR_NOT_PLANNED, "plan has sinks: args->sinks is required");
  if (!sh.has_sinks && args->sinks)
    return set_err(POD_ERR_NOT_PLANNED, "plan has no sinks: args->sinks must be NULL");
  // the decode role's calibration scales (0 = 1): the online softmax keeps its
  // running maximum in raw score units and needs a positive, bounded scale
  if (!std::isfinite(args->q_scale_d) || !std::isfinite(args->k_scale_d) || !std::isfinite(args->v_scale_d))
    return set_err(POD_ERR_INVALID, "q_scale_d, k_scale_d and v_scale_d must be finite");
  const auto one = [](float s) { return s == 0.f ? 1.f : s; };
  const float qk_d = one(args->q_scale_d) * one(args->k_scale_d);
  if (sh.role[1].rows > 0) {
    if (!(qk_d > 0.f)) return set_err(POD_ERR_INVALID, "q_scale_d * k_scale_d must be > 0");
    if (!(sh.role[1].sm_scale * qk_d <= 1e6f))
      return set_err(POD_ERR_INVALID, "sm_scale_d * q_scale_d * k_scale_d must be <= 1e6");
  }
  p = pod::Params{};
  const pod_role_args* ra[2] = {&args->prefill, &args->decode};
  static const char* names[2] = {"prefill", "decode"};
  for (int r = 0; r < 2; ++r) {
    const RolePlan& rp = sh.role[r];
    const pod_role_args& a = *ra[r];
    pod::RoleParams& o = p.role[r];
    const bool fp8 = r == 1 && sh.decode_kv_fp8;
    const int esz = fp8 ? 1 : 2;   // bytes per K/V element
    if (rp.rows > 0) {
      if (!a.q || !a.k_cache || !a.v_cache || !a.out)
        return set_err(POD_ERR_INVALID, std::string(names[r]) + ": q, k_cache, v_cache and out are required");
      if (a.q_stride_tok <= 0 || a.q_stride_head <= 0 || a.kv_stride_page <= 0 ||
          a.kv_stride_tok <= 0 || a.kv_stride_head <= 0 || a.out_stride_tok <= 0 ||
          a.out_stride_head <= 0)
        return set_err(POD_ERR_INVALID, std::string(names[r]) + ": strides must be positive");
      const uintptr_t mis = reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k_cache) |
                            reinterpret_cast<uintptr_t>(a.v_cache) | reinterpret_cast<uintptr_t>(a.out);
      const int64_t smis = a.q_stride_tok | a.q_stride_head | a.kv_stride_page | a.kv_stride_tok |
                           a.kv_stride_head | a.out_stride_tok | a.out_stride_head;
      if ((mis & 15) || (smis & 7))
        return set_err(POD_ERR_INVALID, std::string(names[r]) +
                                             ": buffers must be 16-byte aligned and strides multiples of 8 elements");
      if (fp8 && ((a.kv_stride_page | a.kv_stride_tok | a.kv_stride_head) & 15))
        return set_err(POD_ERR_INVALID, "decode: FP8 K/V strides must be multiples of 16 elements");
      if (fp8 && !a.kv_indices)
        return set_err(POD_ERR_INVALID, "decode: FP8 K/V needs kv_indices (no identity page table)");
      const int64_t lim = (int64_t)1 << 30;   // bytes = 2 * elements must stay below 2^31
      if (a.kv_stride_page >= lim || a.kv_stride_tok >= lim || a.kv_stride_head >= lim)
        return set_err(POD_ERR_UNSUPPORTED, std::string(names[r]) +
                                                ": KV pool strides must be below 2^30 elements");
      if (a.lse && (reinterpret_cast<uintptr_t>(a.lse) & 3))
        return set_err(POD_ERR_INVALID, std::string(names[r]) + ": lse must be 4-byte aligned");
    }
    o.q = a.q;
    o.q_st = a.q_stride_tok;
    o.q_sh = a.q_stride_head;
    o.k = a.k_cache;
    o.v = a.v_cache;
    o.kv_sp_b = (uint32_t)(a.kv_stride_page * esz);
    o.kv_st_b = (uint32_t)(a.kv_stride_tok * esz);
    o.kv_sh_b = (uint32_t)(a.kv_stride_head * esz);
    o.kv_fp8 = fp8 ? 1 : 0;
    o.indices = a.kv_indices;
    o.out = a.out;
    o.o_st = a.out_stride_tok;
    o.o_sh = a.out_stride_head;
    o.lse = a.lse;
    // the decode role's FP8 calibration: q_scale * k_scale fold into the scale,
    // v_scale into the output normalisation (0 = 1)
    const float qk = r == 1 ? qk_d : 1.f;
    o.scale_log2 = rp.sm_scale * qk * 1.4426950408889634f;
    o.v_scale = r == 1 ? one(args->v_scale_d) : 1.f;
    o.causal = rp.causal;
    o.window_left = rp.window_left;
  }
  p.sinks = args->sinks;
  p.num_qo_heads = sh.num_qo_heads;
  p.num_kv_heads = sh.num_kv_heads;
  p.group_size = sh.num_qo_heads / sh.num_kv_heads;
  p.page_size = sh.page_size;
  p.page_shift = -1;
  for (int b = 0; b < 31; ++b)
    if ((1 << b) == sh.page_size) p.page_shift = b;
  return POD_OK;
}

}  // namespace

extern "C" {

const char* pod_last_error(void) { return g_err.c_str(); }

int pod_plan_compute(const pod_plan_desc* desc, int32_t* image, size_t image_cap,
                     pod_plan_info* info) {
  if (!desc) return set_err(POD_ERR_INVALID, "desc is NULL");
  pod_plan_info inf;
  std::string err;
  bool fits = true;
  int rc = pod::plan_compute(*desc, [&](size_t n) -> int32_t* {
    fits = image != nullptr && n <= image_cap;
    return fits ? image : nullptr;
  }, inf, &err, false);
  if (rc) return set_err(rc, err);
  if (info) *info = inf;
  if (!fits) return set_err(POD_ERR_WORKSPACE, "image buffer too small for the plan");
  g_err.clear();
  return POD_OK;
}

int pod_workspace_bytes(const pod_plan_desc* desc, size_t* float_ws_bytes, size_t* int_ws_bytes) {
  if (!desc) return set_err(POD_ERR_INVALID, "desc is NULL");
  pod_plan_info inf;
  std::string err;
  int rc = pod::plan_compute(*desc, nullptr, inf, &err, true);   // the larger image
  if (rc) return set_err(rc, err);
  if (float_ws_bytes) *float_ws_bytes = (size_t)inf.float_ws_bytes;
  if (int_ws_bytes) *int_ws_bytes = (size_t)inf.int_ws_bytes;
  g_err.clear();
  return POD_OK;
}

int pod_create(pod_ctx_t* out, int device, void* float_ws, size_t float_ws_bytes, void* int_ws,
               size_t int_ws_bytes) {
  if (!out) return set_err(POD_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!int_ws || int_ws_bytes == 0) return set_err(POD_ERR_INVALID, "int workspace is required");
  if (!float_ws && float_ws_bytes) return set_err(POD_ERR_INVALID, "float workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(float_ws) & 15) || (reinterpret_cast<uintptr_t>(int_ws) & 15))
    return set_err(POD_ERR_INVALID, "workspaces must be 16-byte aligned");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_err(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev) return set_err(POD_ERR_INVALID, "device index out of range");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) return hip_err(e, "hipDeviceGetAttribute");
  pod_ctx* c = new pod_ctx();
  c->device = device;
  c->float_ws = float_ws;
  c->float_bytes = float_ws_bytes;
  c->int_ws = int_ws;
  c->int_bytes = int_ws_bytes;
  c->num_cus = cus;
  *out = c;
  g_err.clear();
  return POD_OK;
}

int pod_create_graph(pod_ctx_t* out, int device, void* float_ws, size_t float_ws_bytes, void* int_ws,
                     size_t int_ws_bytes, int32_t prefill_batch, int32_t decode_batch) {
  if (out) *out = nullptr;
  if (prefill_batch < 0 || decode_batch < 0)
    return set_err(POD_ERR_INVALID, "batch sizes must be >= 0");
  const int rc = pod_create(out, device, float_ws, float_ws_bytes, int_ws, int_ws_bytes);
  if (rc) return rc;
  (*out)->graph = true;
  (*out)->fixed_batch[0] = prefill_batch;
  (*out)->fixed_batch[1] = decode_batch;
  return POD_OK;
}

int pod_destroy(pod_ctx_t ctx) {
  if (!ctx) return POD_OK;
  {
    DeviceGuard dg(ctx->device);
    for (int i = 0; i < 2; ++i) {
      if (ctx->staged[i]) {
        (void)hipEventSynchronize(ctx->staged[i]);
        (void)hipEventDestroy(ctx->staged[i]);
      }
      if (ctx->used[i]) {
        (void)hipEventSynchronize(ctx->used[i]);
        (void)hipEventDestroy(ctx->used[i]);
      }
      if (ctx->staging[i]) (void)hipHostFree(ctx->staging[i]);
    }
    if (ctx->caller_ready) (void)hipEventDestroy(ctx->caller_ready);
    if (ctx->copy_stream) (void)hipStreamDestroy(ctx->copy_stream);
  }
  delete ctx;
  return POD_OK;
}

int pod_plan(pod_ctx_t ctx, const pod_plan_desc* desc, void* stream) {
  if (!ctx) return set_err(POD_ERR_INVALID, "ctx is NULL");
  if (!desc) return set_err(POD_ERR_INVALID, "desc is NULL");
  pod_plan_desc d = *desc;
  if (d.num_cus <= 0) d.num_cus = ctx->num_cus;
  if (ctx->graph) {
    if (d.prefill.batch != ctx->fixed_batch[0] || d.decode.batch != ctx->fixed_batch[1])
      return set_err(POD_ERR_INVALID, "graph context: batch sizes differ from the fixed ones (" +
                                          std::to_string(ctx->fixed_batch[0]) + " prefill, " +
                                          std::to_string(ctx->fixed_batch[1]) + " decode)");
    if (ctx->policy_set) {
      const pod_plan_desc& f = ctx->policy;
      bool same = d.num_qo_heads == f.num_qo_heads && d.num_kv_heads == f.num_kv_heads &&
                  d.head_dim == f.head_dim && d.page_size == f.page_size && d.dtype == f.dtype &&
                  (d.has_sinks != 0) == (f.has_sinks != 0) && d.num_cus == f.num_cus &&
                  d.decode_kv_dtype == f.decode_kv_dtype;
      const pod_role_desc* a[2] = {&d.prefill, &d.decode};
      const pod_role_desc* b[2] = {&f.prefill, &f.decode};
      for (int r = 0; r < 2; ++r)
        same = same && (a[r]->causal != 0) == (b[r]->causal != 0) &&
               a[r]->window_left == b[r]->window_left && a[r]->sm_scale == b[r]->sm_scale;
      if (!same)
        return set_err(POD_ERR_INVALID,
                       "graph context: heads, head_dim, page_size, dtype, decode_kv_dtype, sinks, "
                       "num_cus and each role's causal / window_left / sm_scale must stay those of "
                       "the first plan");
    }
  }
  DeviceGuard dg(ctx->device);
  if (!dg.ok) return set_err(POD_ERR_HIP, "hipSetDevice failed");
  // the copy runs on the library's stream (pod_run waits for it), or in graph
  // mode on `stream`, ordered with the launches there
  // The planner writes the image straight into a pinned staging buffer (two
  // alternate, each reused once its previous copy has completed).
  const int k = ctx->next_staging;
  hipError_t e = hipSuccess;
  const char* what = nullptr;
  size_t bytes = 0;
  auto sink = [&](size_t n) -> int32_t* {
    bytes = n * sizeof(int32_t);
    if (ctx->staged_pending[k]) {
      e = hipEventSynchronize(ctx->staged[k]);
      if (e != hipSuccess) { what = "hipEventSynchronize"; return nullptr; }
      ctx->staged_pending[k] = false;
    }
    if (ctx->staging_cap[k] < bytes) {
      if (ctx->staging[k]) (void)hipHostFree(ctx->staging[k]);
      ctx->staging[k] = nullptr;
      ctx->staging_cap[k] = 0;
      size_t cap = bytes < 65536 ? 65536 : bytes * 2;
      e = hipHostMalloc(reinterpret_cast<void**>(&ctx->staging[k]), cap, hipHostMallocDefault);
      if (e != hipSuccess) { what = "hipHostMalloc"; return nullptr; }
      ctx->staging_cap[k] = cap;
    }
    return ctx->staging[k];
  };
  pod_plan_info inf;
  std::string err;
  int rc = pod::plan_compute(d, sink, inf, &err, ctx->graph);
  if (rc) return set_err(rc, err);
  if (what) return hip_err(e, what);
  // graph mode keeps one image; otherwise two alternate
  const size_t need = ctx->graph ? bytes : (size_t)inf.int_ws_bytes;
  if (need > ctx->int_bytes)
    return set_err(POD_ERR_WORKSPACE, "int workspace too small: need " + std::to_string(need) + " bytes");
  if (!ctx->graph && !ctx->copy_stream) {
    e = hipStreamCreateWithFlags(&ctx->copy_stream, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_err(e, "hipStreamCreate");
  }
  if ((size_t)inf.float_ws_bytes > ctx->float_bytes)
    return set_err(POD_ERR_WORKSPACE, "float workspace too small: need " +
                                          std::to_string(inf.float_ws_bytes) + " bytes");
  if (!ctx->staged[k]) {
    e = hipEventCreateWithFlags(&ctx->staged[k], hipEventDisableTiming);
    if (e != hipSuccess) return hip_err(e, "hipEventCreate");
  }
  if (!ctx->graph && !ctx->used[k]) {   // a launch's stop event (hipExtLaunchKernel)
    e = hipEventCreate(&ctx->used[k]);
    if (e != hipSuccess) return hip_err(e, "hipEventCreate");
  }
  if (ctx->graph) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    e = hipMemcpyAsync(ctx->int_ws, ctx->staging[k], bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync (work list)");
    e = hipEventRecord(ctx->staged[k], s);   // the staging buffer is free again after it
    if (e != hipSuccess) {
      (void)hipStreamSynchronize(s);   // the copy still reads the staging buffer
      return hip_err(e, "hipEventRecord");
    }
    ctx->staged_pending[k] = true;
    ctx->next_staging = 1 - k;
    if (!ctx->policy_set) {
      ctx->policy = d;
      ctx->policy.prefill.qo_indptr = ctx->policy.prefill.kv_indptr = ctx->policy.prefill.last_page_len = nullptr;
      ctx->policy.decode.qo_indptr = ctx->policy.decode.kv_indptr = ctx->policy.decode.last_page_len = nullptr;
      ctx->policy_set = true;
    }
  } else {
  // half k is free once the launches that read it (the plan before last) are
  // done; the host checks that (they normally are), so the copy stream carries
  // no wait on the launch stream
  if (ctx->used_pending[k]) {
    e = hipEventSynchronize(ctx->used[k]);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize");
    ctx->used_pending[k] = false;
  }
  if (!ctx->half_ordered[k]) {
    if (!ctx->caller_ready) {
      e = hipEventCreateWithFlags(&ctx->caller_ready, hipEventDisableTiming);
      if (e != hipSuccess) return hip_err(e, "hipEventCreate");
    }
    e = hipEventRecord(ctx->caller_ready, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_err(e, "hipEventRecord (caller stream)");
    e = hipStreamWaitEvent(ctx->copy_stream, ctx->caller_ready, 0);
    if (e != hipSuccess) return hip_err(e, "hipStreamWaitEvent");
    ctx->half_ordered[k] = true;
  }
  e = hipMemcpyAsync(int_half(ctx, k), ctx->staging[k], bytes, hipMemcpyHostToDevice, ctx->copy_stream);
  if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync (work list)");
  e = hipEventRecord(ctx->staged[k], ctx->copy_stream);
  if (e != hipSuccess) {
    (void)hipStreamSynchronize(ctx->copy_stream);   // the copy still reads the staging buffer
    return hip_err(e, "hipEventRecord");
  }
  ctx->staged_pending[k] = true;   // the staging buffer is read until the copy ends
  // While the previous plan's launch still runs, the host waits for this copy
  // behind it (a few microseconds; the launch keeps the GPU busy), so pod_run
  // enqueues the next launch alone: a cross-stream wait ahead of each launch
  // measured 2-5 us slower per step. With the GPU idle, that wait would only
  // hold the host: pod_plan returns at once and pod_run orders its launch
  // after the copy on the device.
  bool gpu_busy = false;
  if (ctx->used_pending[ctx->cur]) {
    e = hipEventQuery(ctx->used[ctx->cur]);
    if (e == hipSuccess) {
      ctx->used_pending[ctx->cur] = false;
    } else if (e == hipErrorNotReady) {
      gpu_busy = true;
    } else {
      return hip_err(e, "hipEventQuery");
    }
  }
  if (gpu_busy) {
    e = hipEventSynchronize(ctx->staged[k]);
    if (e != hipSuccess) return hip_err(e, "hipEventSynchronize");
    ctx->staged_pending[k] = false;
  }
  ctx->cur = k;
  ctx->next_staging = 1 - k;
  }

  plan_shape(d, ctx->shape);
  ctx->info = inf;
  memcpy(ctx->hdr, ctx->staging[k], sizeof(ctx->hdr));
  ctx->planned = true;
  g_err.clear();
  return POD_OK;
}

int pod_plan_stats(pod_ctx_t ctx, pod_plan_info* info) {
  if (!ctx || !info) return set_err(POD_ERR_INVALID, "ctx and info are required");
  if (!ctx->planned) return set_err(POD_ERR_NOT_PLANNED, "pod_plan has not been called");
  *info = ctx->info;
  return POD_OK;
}

int pod_run(pod_ctx_t ctx, const pod_run_args* args, void* stream) {
  if (!ctx) return set_err(POD_ERR_INVALID, "ctx is NULL");
  if (!args) return set_err(POD_ERR_INVALID, "args is NULL");
  if (!ctx->planned) return set_err(POD_ERR_NOT_PLANNED, "pod_run called before pod_plan");
  pod::Params p{};
  const int rc = fill_params(ctx->shape, args, p);
  if (rc) return rc;
  p.image = ctx->graph ? reinterpret_cast<int32_t*>(ctx->int_ws) : int_half(ctx, ctx->cur);
  p.partials = reinterpret_cast<float*>(ctx->float_ws);
  DeviceGuard dg(ctx->device);
  if (!dg.ok) return set_err(POD_ERR_HIP, "hipSetDevice failed");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (ctx->graph) {
    // the image copy went on the plan's stream, ahead of this launch; no event
    // work, so the call can be captured into a graph
    const int e = pod::launch_pod_grid(p, ctx->shape.dtype, ctx->info.grid, stream, nullptr);
    if (e != (int)hipSuccess) return hip_err((hipError_t)e, "pod grid launch");
    g_err.clear();
    return POD_OK;
  }
  // this plan's work list must be up: pod_plan waited for its copy when the
  // GPU was busy; otherwise the launch waits for it on the device
  hipError_t he = hipSuccess;
  if (ctx->staged_pending[ctx->cur]) {
    he = hipEventQuery(ctx->staged[ctx->cur]);
    if (he == hipSuccess) {
      ctx->staged_pending[ctx->cur] = false;
    } else if (he == hipErrorNotReady) {
      he = hipStreamWaitEvent(s, ctx->staged[ctx->cur], 0);
      if (he != hipSuccess) return hip_err(he, "hipStreamWaitEvent");
    } else {
      return hip_err(he, "hipEventQuery");
    }
  }
  // used[cur] fires when this launch completes (a launch that is not issued
  // because the plan holds no work reads nothing)
  int e = pod::launch_pod_grid(p, ctx->shape.dtype, ctx->info.grid, stream, ctx->used[ctx->cur]);
  if (e != (int)hipSuccess) return hip_err((hipError_t)e, "pod grid launch");
  if (ctx->info.grid > 0) ctx->used_pending[ctx->cur] = true;
  g_err.clear();
  return POD_OK;
}

int pod_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                     void* o_out, float* lse_out, int64_t rows, int num_heads, int head_dim,
                     int dtype, const float* sinks, int device, void* stream) {
  if (rows < 0 || num_heads <= 0) return set_err(POD_ERR_INVALID, "rows must be >= 0 and num_heads > 0");
  if (head_dim != pod::kHeadDim) return set_err(POD_ERR_UNSUPPORTED, "head_dim must be 128");
  if (dtype != POD_DTYPE_F16 && dtype != POD_DTYPE_BF16)
    return set_err(POD_ERR_UNSUPPORTED, "dtype must be POD_DTYPE_F16 or POD_DTYPE_BF16");
  if (rows == 0) {
    g_err.clear();
    return POD_OK;
  }
  if (!o_a || !o_b || !o_out || !lse_a || !lse_b || !lse_out)
    return set_err(POD_ERR_INVALID, "o_a, lse_a, o_b, lse_b, o_out and lse_out are required");
  for (const void* ptr : {o_a, o_b, (const void*)o_out})
    if (reinterpret_cast<uintptr_t>(ptr) & 15) return set_err(POD_ERR_INVALID, "O buffers must be 16-byte aligned");
  for (const void* ptr : {(const void*)lse_a, (const void*)lse_b, (const void*)lse_out, (const void*)sinks})
    if (reinterpret_cast<uintptr_t>(ptr) & 3) return set_err(POD_ERR_INVALID, "LSE and sink buffers must be 4-byte aligned");
  if (rows > INT64_MAX / 2 / num_heads / pod::kHeadDim) return set_err(POD_ERR_INVALID, "rows too large");
  DeviceGuard dg(device);
  if (!dg.ok) return set_err(POD_ERR_HIP, "hipSetDevice failed");
  const int e = pod::launch_merge_states(o_a, lse_a, o_b, lse_b, o_out, lse_out, rows * num_heads,
                                         num_heads, dtype, sinks, stream);
  if (e != (int)hipSuccess) return hip_err((hipError_t)e, "merge launch");
  g_err.clear();
  return POD_OK;
}

int pod_run_static(const pod_plan_desc* desc, const pod_run_args* args, int device, void* stream) {
  if (!desc) return set_err(POD_ERR_INVALID, "desc is NULL");
  if (!args) return set_err(POD_ERR_INVALID, "args is NULL");
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess) return hip_err(e, "hipGetDeviceCount");
  if (device < 0 || device >= ndev || device >= pod::kMaxDevices)
    return set_err(POD_ERR_INVALID, "device index out of range");
  DeviceGuard dg(device);
  if (!dg.ok) return set_err(POD_ERR_HIP, "hipSetDevice failed");
  pod_plan_desc d = *desc;
  if (d.num_cus <= 0) {
    e = hipDeviceGetAttribute(&d.num_cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_err(e, "hipDeviceGetAttribute");
  }
  void* base = nullptr;
  const int se = pod::static_scratch(device, &base);
  if (se != (int)hipSuccess) return hip_err((hipError_t)se, "hipGetSymbolAddress (static scratch)");

  std::lock_guard<std::mutex> lock(g_static_mu);
  size_t words = 0;
  bool fits = false;
  pod_plan_info inf;
  std::string err;
  int rc = pod::plan_compute(d, [&](size_t n) -> int32_t* {
    words = n;
    fits = n * sizeof(int32_t) <= pod::kStaticImageBytes;
    return fits ? g_static_image : nullptr;
  }, inf, &err, false);
  if (rc) return set_err(rc, err);
  if (!fits)
    return set_err(POD_ERR_WORKSPACE, "work list of " + std::to_string(words * 4) +
                                          " bytes exceeds the static limit of 16 MiB");
  if ((size_t)inf.float_ws_bytes > pod::kStaticPartialBytes)
    return set_err(POD_ERR_WORKSPACE, "split-KV partial states of " + std::to_string(inf.float_ws_bytes) +
                                          " bytes exceed the static limit of 48 MiB");
  PlanShape shape;
  plan_shape(d, shape);
  pod::Params p{};
  rc = fill_params(shape, args, p);
  if (rc) return rc;
  p.image = reinterpret_cast<int32_t*>(base);
  p.partials = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + pod::kStaticImageBytes);
  // the image (its arrival counters and pool queue zero) goes up on the
  // caller's stream ahead of the launch; the host buffer is free again when
  // the copy call returns (host memory that is not pinned is staged at once)
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  e = hipMemcpyAsync(base, g_static_image, words * sizeof(int32_t), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_err(e, "hipMemcpyAsync (work list)");
  const int le = pod::launch_pod_grid(p, d.dtype, inf.grid, stream, nullptr);
  if (le != (int)hipSuccess) return hip_err((hipError_t)le, "pod grid launch");
  g_err.clear();
  return POD_OK;
}

}  // extern "C"
