// Cascade merge of two attention states for gfx950 (MI355X).
//
// A shared-prefix level and a per-request level of the same query rows attend
// disjoint key sets; each returns (O, lse) with a base-2 LSE. The README tour
// (www.gsyq.cn/news/442943, core operator list: "Cascade Attention") names the
// hierarchical shared-prefix KV cache, and the cuDNN backend article
// (www.gsyq.cn/news/452757, "LSE 契约") states that the base-2 LSE goes straight
// into such a merge:
//   L = log2(2^la + 2^lb),  O = 2^(la - L) O_a + 2^(lb - L) O_b
// per (row, head). A state with lse = -inf holds no keys and weighs 0. A sink
// logit, if given, is applied once to the merged state: O / (1 + 2^(sink log2e
// - L)), L unchanged (the same convention as the fused launch).
//
// The merge streams 2 x 256 bytes in and 256 bytes out per (row, head): HBM
// bound. 16 lanes own one (row, head); each moves 16 bytes of each operand
// with one load, so a wave touches four 256-byte rows per instruction.
#include <hip/hip_runtime.h>

#include "pod_internal.h"

namespace pod {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kMergeThreads = 256;
constexpr int kLanesPerPair = kHeadDim / 8;   // 16 lanes x 8 elements
constexpr float kLog2eM = 1.4426950408889634f;

template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
  using type = bf16x8;
};
template <>
struct Vec8<_Float16> {
  using type = f16x8;
};

template <typename T>
__global__ __launch_bounds__(kMergeThreads) void merge_states_kernel(
    // no __restrict__: the outputs may be one of the inputs (each element is
    // read before it is written, by the same thread)
    const T* oa, const float* la, const T* ob, const float* lb, T* oo, float* lo, int64_t n_pairs,
    int heads, const float* __restrict__ sinks) {
  using V = typename Vec8<T>::type;
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  const int64_t pair = t / kLanesPerPair;
  const int part = (int)(t % kLanesPerPair);
  if (pair >= n_pairs) return;
  const float a = la[pair], b = lb[pair];
  const float mx = fmaxf(a, b);
  float wa = 0.f, wb = 0.f, L = -__builtin_inff();
  if (mx != -__builtin_inff()) {
    const float ea = __builtin_amdgcn_exp2f(a - mx), eb = __builtin_amdgcn_exp2f(b - mx);
    const float tot = ea + eb;   // >= 1: the larger term is exp2(0)
    L = mx + __builtin_amdgcn_logf(tot);
    float f = 1.f / tot;
    if (sinks) f /= 1.f + __builtin_amdgcn_exp2f(sinks[pair % heads] * kLog2eM - L);
    wa = ea * f;
    wb = eb * f;
  }
  const int64_t off = pair * kHeadDim + part * 8;
  const V va = __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(oa + off));
  const V vb = __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(ob + off));
  V r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (T)(wa * (float)va[i] + wb * (float)vb[i]);
  *reinterpret_cast<u32x4*>(oo + off) = __builtin_bit_cast(u32x4, r);
  if (part == 0) lo[pair] = L;
}

}  // namespace

int launch_merge_states(const void* oa, const float* la, const void* ob, const float* lb,
                        void* oo, float* lo, int64_t n_pairs, int heads, int dtype,
                        const float* sinks, void* stream) {
  if (n_pairs <= 0) return (int)hipSuccess;
  const int64_t threads = n_pairs * kLanesPerPair;
  const dim3 grid((unsigned)((threads + kMergeThreads - 1) / kMergeThreads));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dtype == POD_DTYPE_BF16)
    hipLaunchKernelGGL(merge_states_kernel<__bf16>, grid, dim3(kMergeThreads), 0, s,
                       static_cast<const __bf16*>(oa), la, static_cast<const __bf16*>(ob), lb,
                       static_cast<__bf16*>(oo), lo, n_pairs, heads, sinks);
  else
    hipLaunchKernelGGL(merge_states_kernel<_Float16>, grid, dim3(kMergeThreads), 0, s,
                       static_cast<const _Float16*>(oa), la, static_cast<const _Float16*>(ob), lb,
                       static_cast<_Float16*>(oo), lo, n_pairs, heads, sinks);
  return (int)hipGetLastError();
}

}  // namespace pod
